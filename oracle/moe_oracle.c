/*
 * moe_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU reference of the W4A8 mixture-of-experts
 * decode layer.  Only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark load this file's library.  The product path never does: it
 * shares no code, table or header with the GPU kernels, and the GPU kernels do
 * not depend on it.
 *
 * Pages cited (by title and section):
 *   [EN] "NVIDIA Shows 3 Ways to Speed Up MoE Inference on DGX Spark, Lifting
 *        Ling-3.0-flash Throughput 42.5%" (MarkTechPost text).
 *   [ZH] "NVIDIA博客:DGX Spark上三项优化使Ling-3.0-flash解码吞吐提升 42.5%".
 * The pages name the formats (MXFP4 expert weights, FP8 activations: the W4A8
 * recipe, [EN] "Why is MoE decoding on DGX Spark memory-bound?") but never
 * define them.  The decoders below follow the public format definitions:
 *   OCP Microscaling Formats (MX) v1.0: E2M1 elements, E8M0 shared scale,
 *   block size 32;  OCP 8-bit floating point (OFP8): E4M3 ("FN": no infinity,
 *   only S.1111.111 is NaN, largest finite 448).
 *
 * Arithmetic: every sum accumulates in double.  The two quantisation steps
 * (activation FP8 and intermediate FP8) are specified in binary32 because the
 * bytes they produce are compared bit for bit; this file must be compiled with
 * strict IEEE semantics (-ffp-contract=off, no fast-math) so that each float
 * division is a single correctly rounded IEEE division.
 *
 * Parity pins for every function live in tests/test_oracle_pins.py.
 */
#define _POSIX_C_SOURCE 199309L
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <time.h>

/* ------------------------------------------------------------------------- */
/* Number formats                                                             */
/* ------------------------------------------------------------------------- */

/* MX v1.0 E2M1 element: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit,
 * no infinity or NaN.  Magnitudes of codes 0..7 (code 8..15 are negatives). */
static const double kE2M1Magnitude[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(unsigned code)
{
    double m = kE2M1Magnitude[code & 7u];
    return (code & 8u) ? -m : m;
}

/* MX v1.0 E8M0 shared scale: an unsigned biased exponent, 2^(c-127); 0xFF is NaN. */
double orc_e8m0_value(unsigned code)
{
    if ((code & 0xFFu) == 0xFFu) return NAN;
    return ldexp(1.0, (int)(code & 0xFFu) - 127);
}

/* OFP8 E4M3: bias 7; exponent field 0 holds subnormals m/8 * 2^-6;
 * S.1111.111 is NaN; there is no infinity. */
double orc_e4m3_value(unsigned code)
{
    unsigned s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
    double v;
    if (e == 15u && m == 7u) return NAN;
    if (e == 0u) v = ldexp((double)m / 8.0, -6);
    else         v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static float bf16_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

double orc_bf16_value(uint16_t b) { return (double)bf16_to_float(b); }

/* E4M3 encoder: round to the nearest finite E4M3 value, ties to the even code,
 * magnitudes above 448 saturate to 448 (the nearest finite value), and the
 * sign of the input is kept (so -0 and negative values that round to zero
 * give 0x80).  Written as a brute-force search over the 127 finite
 * magnitudes, which are increasing in the code.
 *
 * The distances are computed in double.  They are exact whenever the input
 * lies within a few binades of the candidate (Sterbenz-type cancellation on a
 * 24-bit input), which covers every case where two candidates can be close to
 * a tie; when the input is far below every non-zero code the distance to 0 is
 * the input itself (exact) and is smaller than any rounded distance to a
 * non-zero code, so the choice is still correct. */
uint8_t orc_e4m3_encode(float y)
{
    uint32_t bits;
    memcpy(&bits, &y, sizeof bits);
    unsigned sign = (bits >> 31) ? 0x80u : 0u;
    if (isnan(y)) return 0x7Fu;
    double a = fabs((double)y);
    unsigned best = 0;
    double best_d = a;                      /* distance to code 0 (value 0) */
    for (unsigned c = 1; c <= 0x7Eu; ++c) {
        double d = fabs(orc_e4m3_value(c) - a);
        if (d < best_d || (d == best_d && (c & 1u) == 0u)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(best | sign);
}

/* The same encoder over an array (for sweeps). */
void orc_e4m3_encode_n(int64_t n, const float* y, uint8_t* q)
{
    for (int64_t i = 0; i < n; ++i) q[i] = orc_e4m3_encode(y[i]);
}

/* ------------------------------------------------------------------------- */
/* Tensor accessors for the layout the library documents                      */
/* ------------------------------------------------------------------------- */

/* MXFP4 matrix [rows, K] of expert e, stored as codes [E, rows, K/2] (element
 * 2i in bits 3:0 of byte i, element 2i+1 in bits 7:4) and E8M0 scales
 * [E, rows, K/32] (one scale per 32 consecutive elements of a row). */
static double mxfp4_element(const uint8_t* codes, const uint8_t* scales,
                            int64_t rows, int64_t K, int64_t e, int64_t r, int64_t k)
{
    uint8_t byte = codes[(e * rows + r) * (K / 2) + k / 2];
    unsigned c = (k % 2 == 0) ? (byte & 0x0Fu) : (byte >> 4);
    uint8_t sc = scales[(e * rows + r) * (K / 32) + k / 32];
    return orc_e2m1_value(c) * orc_e8m0_value(sc);
}

/* ------------------------------------------------------------------------- */
/* The layer                                                                   */
/* ------------------------------------------------------------------------- */

/* Router ([EN] "What is Ling 3.0...": each token goes to 8 routed experts; the
 * pages do not name the scoring function; the reading used is softmax over all
 * E logits, keep the K largest, renormalise, ties toward the lower index).
 *
 * logits[t,e] = sum_k x[t,k] * Wr[e,k] in double (each bf16 product is exact).
 * ids[t,:]    = the K experts ordered by (logit descending, index ascending).
 * w[t,j]      = exp(L_j - L_1) / sum_{i<K} exp(L_i - L_1): the renormalised
 *               softmax restricted to the selection (the full-softmax
 *               denominator cancels).
 * gap[t]      = L_(K) - L_(K+1) in double, or +inf when K == E. */
void orc_route(int M, int H, int E, int K,
               const uint16_t* x, const uint16_t* wr,
               double* logits, int32_t* ids, double* w, double* gap)
{
    for (int t = 0; t < M; ++t) {
        double* L = logits + (int64_t)t * E;
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int k = 0; k < H; ++k)
                acc += (double)bf16_to_float(x[(int64_t)t * H + k]) *
                       (double)bf16_to_float(wr[(int64_t)e * H + k]);
            L[e] = acc;
        }
        /* selection: K passes, each taking the best not yet taken */
        int32_t* sel = ids + (int64_t)t * K;
        for (int j = 0; j < K; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                int taken = 0;
                for (int i = 0; i < j; ++i) taken |= (sel[i] == e);
                if (taken) continue;
                if (best < 0 || L[e] > L[best]) best = e;   /* strict: lower index kept on ties */
            }
            sel[j] = best;
        }
        if (K < E) {
            int next = -1;
            for (int e = 0; e < E; ++e) {
                int taken = 0;
                for (int i = 0; i < K; ++i) taken |= (sel[i] == e);
                if (taken) continue;
                if (next < 0 || L[e] > L[next]) next = e;
            }
            gap[t] = L[sel[K - 1]] - L[next];
        } else {
            gap[t] = INFINITY;
        }
        double denom = 0.0;
        for (int j = 0; j < K; ++j) denom += exp(L[sel[j]] - L[sel[0]]);
        for (int j = 0; j < K; ++j) w[(int64_t)t * K + j] = exp(L[sel[j]] - L[sel[0]]) / denom;
    }
}

/* Token-to-expert compaction for M > 1 ([EN] "What are the 3
 * optimizations?", item 3: verifying 4 positions touches up to 32 experts;
 * every selected expert's weights should stream once per step).
 * Output: the distinct selected experts in ascending id (act_experts[n_act]),
 * offsets[n_act+1] into the pair list, and for each compacted pair i its token
 * pair_token[i] and original pair index pair_src[i] = t*K + j; pairs of one
 * expert are in ascending token order.  pair_of[t*K+j] is the compacted
 * position of pair (t,j).  Returns n_act. */
int orc_compact(int M, int K, int E, const int32_t* ids,
                int32_t* act_experts, int32_t* offsets,
                int32_t* pair_token, int32_t* pair_src, int32_t* pair_of)
{
    int n_act = 0, count = 0;
    for (int e = 0; e < E; ++e) {
        int used = 0;
        for (int p = 0; p < M * K; ++p) used |= (ids[p] == e);
        if (!used) continue;
        act_experts[n_act] = e;
        offsets[n_act] = count;
        for (int t = 0; t < M; ++t)
            for (int j = 0; j < K; ++j)
                if (ids[t * K + j] == e) {
                    pair_token[count] = t;
                    pair_src[count] = t * K + j;
                    pair_of[t * K + j] = count;
                    ++count;
                }
        ++n_act;
    }
    offsets[n_act] = count;
    return n_act;
}

/* Per-token FP8 E4M3 activation quantisation (the "A8" of W4A8, [EN] "Why is
 * MoE decoding on DGX Spark memory-bound?").  One binary32 scale per token:
 * s = amax/448 (s = 1 when the row is all zero), codes = E4M3(x / s). */
void orc_quant_act(int M, int H, const uint16_t* x, uint8_t* q, float* s)
{
    for (int t = 0; t < M; ++t) {
        float amax = 0.0f;
        for (int k = 0; k < H; ++k) {
            float v = fabsf(bf16_to_float(x[(int64_t)t * H + k]));
            if (v > amax) amax = v;
        }
        float st = (amax == 0.0f) ? 1.0f : amax / 448.0f;
        s[t] = st;
        for (int k = 0; k < H; ++k) {
            float y = bf16_to_float(x[(int64_t)t * H + k]) / st;
            q[(int64_t)t * H + k] = orc_e4m3_encode(y);
        }
    }
}

/* Fused gate/up projection with the SiLU(gate) * up activation ([EN] "What
 * are the 3 optimizations?", item 1: the expert layer is 768 wide; rows [0,I)
 * of w13 are the gate projection, rows [I,2I) the up projection).
 * For pair p = t*K + j with e = ids[p]:
 *   A_k   = E4M3(q[t,k]) * s[t]
 *   r-row = sum_k W13[e,r,k] * A_k,  W = E2M1 * E8M0 (block of 32 along k)
 *   h[p,i] = g_i * sigmoid(g_i) * u_i   (g = row i, u = row I+i), in double. */
void orc_gate_up(int M, int H, int I, int K,
                 const uint8_t* q, const float* s, const int32_t* ids,
                 const uint8_t* w13, const uint8_t* s13, double* h)
{
    const int64_t rows = 2 * (int64_t)I;
    for (int t = 0; t < M; ++t) {
        for (int j = 0; j < K; ++j) {
            const int64_t p = (int64_t)t * K + j;
            const int64_t e = ids[p];
            for (int i = 0; i < I; ++i) {
                double g = 0.0, u = 0.0;
                for (int k = 0; k < H; ++k) {
                    double a = orc_e4m3_value(q[(int64_t)t * H + k]) * (double)s[t];
                    g += mxfp4_element(w13, s13, rows, H, e, i, k) * a;
                    u += mxfp4_element(w13, s13, rows, H, e, I + i, k) * a;
                }
                h[p * I + i] = g / (1.0 + exp(-g)) * u;
            }
        }
    }
}

/* Intermediate FP8 requantisation, one binary32 scale per (token, expert) row
 * of I values, the same scheme as the activation quantisation.  The GPU holds
 * h in binary32, so the row is first rounded to binary32:
 *   b = max_i |fl32(h_i)|,  s2 = fl32(b / 448) (1 when b == 0),
 *   q2_i = E4M3(fl32(fl32(h_i) / s2)). */
void orc_requant(int P, int I, const double* h, uint8_t* q2, float* s2)
{
    for (int p = 0; p < P; ++p) {
        float b = 0.0f;
        for (int i = 0; i < I; ++i) {
            float v = fabsf((float)h[(int64_t)p * I + i]);
            if (v > b) b = v;
        }
        float sc = (b == 0.0f) ? 1.0f : b / 448.0f;
        s2[p] = sc;
        for (int i = 0; i < I; ++i) {
            float y = (float)h[(int64_t)p * I + i] / sc;
            q2[(int64_t)p * I + i] = orc_e4m3_encode(y);
        }
    }
}

/* Down projection and router-weighted combine:
 *   d[p,n]   = s2[p] * sum_k W2[e,n,k] * E4M3(q2[p,k])
 *   out[t,n] = sum_j w[t,j] * d[t*K+j, n]          (all in double). */
void orc_down_combine(int M, int H, int I, int K,
                      const uint8_t* q2, const float* s2,
                      const int32_t* ids, const double* w,
                      const uint8_t* w2, const uint8_t* sc2, double* out)
{
    for (int t = 0; t < M; ++t) {
        for (int n = 0; n < H; ++n) out[(int64_t)t * H + n] = 0.0;
        for (int j = 0; j < K; ++j) {
            const int64_t p = (int64_t)t * K + j;
            const int64_t e = ids[p];
            for (int n = 0; n < H; ++n) {
                double acc = 0.0;
                for (int k = 0; k < I; ++k)
                    acc += mxfp4_element(w2, sc2, H, I, e, n, k) *
                           orc_e4m3_value(q2[p * I + k]);
                out[(int64_t)t * H + n] += w[p] * ((double)s2[p] * acc);
            }
        }
    }
}

/* The whole layer, exporting every stage as a tap.  All outputs are caller
 * buffers: logits[M,E], ids[M,K], w[M,K], gap[M], q[M,H], s[M], h[M*K,I],
 * q2[M*K,I], s2[M*K], out[M,H]. */
void orc_moe_layer(int M, int H, int I, int E, int K,
                   const uint16_t* x, const uint16_t* wr,
                   const uint8_t* w13, const uint8_t* s13,
                   const uint8_t* w2, const uint8_t* sc2,
                   double* logits, int32_t* ids, double* w, double* gap,
                   uint8_t* q, float* s, double* h, uint8_t* q2, float* s2,
                   double* out)
{
    orc_route(M, H, E, K, x, wr, logits, ids, w, gap);
    orc_quant_act(M, H, x, q, s);
    orc_gate_up(M, H, I, K, q, s, ids, w13, s13, h);
    orc_requant(M * K, I, h, q2, s2);
    orc_down_combine(M, H, I, K, q2, s2, ids, w, w2, sc2, out);
}

/* The CPU baseline: runs orc_moe_layer `runs` times on the same inputs and
 * writes each run's wall time in seconds (CLOCK_MONOTONIC around the call
 * only; the inputs and outputs are the caller's, made before the first run).
 * No arithmetic of its own. */
void orc_time_layer(int runs, int M, int H, int I, int E, int K,
                    const uint16_t* x, const uint16_t* wr,
                    const uint8_t* w13, const uint8_t* s13,
                    const uint8_t* w2, const uint8_t* sc2,
                    double* logits, int32_t* ids, double* w, double* gap,
                    uint8_t* q, float* s, double* h, uint8_t* q2, float* s2,
                    double* out, double* seconds)
{
    for (int r = 0; r < runs; ++r) {
        struct timespec a, b;
        clock_gettime(CLOCK_MONOTONIC, &a);
        orc_moe_layer(M, H, I, E, K, x, wr, w13, s13, w2, sc2, logits, ids, w, gap, q, s, h, q2, s2, out);
        clock_gettime(CLOCK_MONOTONIC, &b);
        seconds[r] = (double)(b.tv_sec - a.tv_sec) + 1e-9 * (double)(b.tv_nsec - a.tv_nsec);
    }
}

/* ------------------------------------------------------------------------- */
/* FP8 LM head                                                               */
/* ------------------------------------------------------------------------- */

/* The output projection (hidden 2,560 -> vocabulary 157,184) is stored in
 * BF16 and read in full for every generated token; quantising it once to FP8
 * at load time halves those reads ([EN] "What are the 3 optimizations?",
 * item 2; [ZH] "三项优化分别做了什么").  The pages fix neither the scale
 * granularity nor whether the activations are quantised too.  Reading taken:
 * one binary32 scale per output row, s_v = amax_k |W[v,k]| / 448 (1 for an
 * all-zero row), codes E4M3(W[v,k] / s_v) -- the activation scheme of
 * orc_quant_act applied to each weight row -- while the activations stay
 * BF16 (the saving is in the weight reads).
 *   logits[t,v] = s_v * sum_k E4M3(q[v,k]) * x[t,k]          (in double) */
void orc_lm_head_quant(int V, int H, const uint16_t* w, uint8_t* q, float* s)
{
    orc_quant_act(V, H, w, q, s);
}

void orc_lm_head_gemv(int M, int V, int H, const uint16_t* x, const uint8_t* q, const float* s, double* logits)
{
    for (int t = 0; t < M; ++t) {
        for (int v = 0; v < V; ++v) {
            double acc = 0.0;
            for (int k = 0; k < H; ++k)
                acc += orc_e4m3_value(q[(int64_t)v * H + k]) * (double)bf16_to_float(x[(int64_t)t * H + k]);
            logits[(int64_t)t * V + v] = (double)s[v] * acc;
        }
    }
}
