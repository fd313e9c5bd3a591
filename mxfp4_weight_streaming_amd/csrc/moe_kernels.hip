// moe_kernels.hip -- gfx950 kernels of the W4A8 MoE decode layer (M <= 8 tokens).
//
// The pages find batch-1 MoE decode bound by reading expert weights ([EN]
// "Why is MoE decoding on DGX Spark memory-bound?"), so the kernels are built
// around streaming MXFP4 bytes from HBM once, with wide loads issued before
// any dependent work.  A layer is four kernels on one stream:
//   router_kernel   fp32 router GEMV (one wave per expert row) and per-token
//                   FP8 quantisation of the activations; the last workgroup to
//                   finish derives the routing once: top-K, renormalised
//                   weights and the token->expert compaction ([EN] "What is
//                   Ling 3.0...": 8 routed experts per token; [EN] "What are
//                   the 3 optimizations?", item 3: a 4-token verify touches up
//                   to 32 experts).
//   gate_up_kernel  the fused gate/up MXFP4 GEMV of one selected expert's rows
//                   with the SiLU(gate)*up epilogue ([EN] same section, item 1:
//                   the 768-wide expert layer); it also pulls its expert's
//                   down-projection weights into the memory-side cache.
//   requant_kernel  per-(token, expert) FP8 requantisation of the intermediate.
//   down_kernel     the down GEMV over all selected experts and the
//                   router-weighted combine, in a fixed order (no float atomics).
// Cross-workgroup synchronisation inside a kernel is used once per layer (the
// router's last-arrival step, 64 workgroups): on this chip every device-scope
// release costs a serialised L2 write-back, so kernel boundaries carry the
// other dependencies.
// The M <= 8 path is a GEMV: it uses the vector ALU (dot2 on exactly decoded
// f16 operands, fp32 accumulation), not the matrix cores.
//   [EN] = "NVIDIA Shows 3 Ways to Speed Up MoE Inference on DGX Spark,
//          Lifting Ling-3.0-flash Throughput 42.5%"
#include "device_common.hpp"
#include "moe_internal.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Per-token activation quantisation (one workgroup, one token).
// s = amax / 448 (1 for an all-zero row), q = E4M3(x / s), both divisions
// correctly rounded binary32 divisions.
// ---------------------------------------------------------------------------
template <int H>
__device__ void quantize_token(const uint16_t* __restrict__ x, uint8_t* __restrict__ q,
                               float* __restrict__ s_out, float* red)
{
    float m = 0.0f;
    for (int k = threadIdx.x; k < H; k += blockDim.x) m = fmaxf(m, fabsf(bf16_bits_to_f32(x[k])));
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    float amax = red[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) amax = fmaxf(amax, red[w]);
    const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
    for (int k = threadIdx.x; k < H; k += blockDim.x) q[k] = (uint8_t)e4m3_encode(bf16_bits_to_f32(x[k]) / s);
    if (threadIdx.x == 0) *s_out = s;
    __syncthreads();
}

template <int H>
__global__ __launch_bounds__(256) void quant_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ q,
                                                    float* __restrict__ s)
{
    __shared__ float red[4];
    const int t = blockIdx.x;
    quantize_token<H>(x + (size_t)t * H, q + (size_t)t * H, s + t, red);
}

// ---------------------------------------------------------------------------
// Top-K on one token's logits by one wave: K rounds of a wave-wide maximum of
// the key (orderable logit, ~expert index), so equal logits go to the lower
// index.  Weights are the softmax over the selected logits.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_orderable(float v)
{
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float f32_from_orderable(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ uint64_t topk_key(float v, int e)
{
    return ((uint64_t)f32_orderable(v + 0.0f) << 32) | (uint32_t)(~(uint32_t)e);   // + 0.0f folds -0 into +0
}

// Keys are unique, so each round's maximum belongs to exactly one lane.  Every
// lane sorts its (at most 8) keys once; a round then compares only the lanes'
// heads: first on the 32-bit orderable logit alone (one DPP max chain), and
// only if several lanes share that logit exactly, on the full key, whose low
// half makes the lower expert index win.
__device__ void topk_wave(const float* L, int E, int K, int32_t* ids_out, float* w_out)
{
    const int lane = threadIdx.x & 63;
    constexpr int PER = kMaxExperts / kWave;
    uint64_t k[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + kWave * i;
        k[i] = (e < E) ? topk_key(L[e], e) : 0ull;
    }
#pragma unroll
    for (int i = 1; i < PER; ++i)            // insertion sort, descending
#pragma unroll
        for (int j = i; j > 0; --j) {
            const uint64_t hi = max_u64(k[j - 1], k[j]), lo = k[j - 1] ^ k[j] ^ hi;
            k[j - 1] = hi;
            k[j] = lo;
        }
    uint64_t mine = 0, first = 0;            // lane j keeps the j-th selected key
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
        if (j < K) {
            const uint32_t hi = (uint32_t)(k[0] >> 32);
            const uint32_t best_hi = wave_max_u32(hi);
            const uint64_t tied = __ballot(hi == best_hi);
            uint64_t best;
            if (__popcll(tied) == 1) {
                const int owner = __ffsll((unsigned long long)tied) - 1;
                best = ((uint64_t)best_hi << 32) | (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k[0], owner);
            } else {
                best = wave_max_u64(hi == best_hi ? k[0] : 0ull);
            }
            if (j == 0) first = best;
            if (lane == j) mine = best;
            if (k[0] == best) {
#pragma unroll
                for (int i = 0; i + 1 < PER; ++i) k[i] = k[i + 1];
                k[PER - 1] = 0ull;
            }
        }
    }
    const float top = f32_from_orderable((uint32_t)(first >> 32));
    const float ex = (lane < K) ? expf(f32_from_orderable((uint32_t)(mine >> 32)) - top) : 0.0f;
    const float den = wave_sum(ex);
    if (lane < K) {
        ids_out[lane] = (int32_t)(~(uint32_t)mine);
        w_out[lane] = ex / den;
    }
}

// ---------------------------------------------------------------------------
// Routing prologue, run by every thread of a workgroup: top-K (from logits) or
// caller ids, then token->expert compaction, all in LDS.  Distinct experts get
// slots in ascending id; the pairs of a slot are in ascending token order.
// ---------------------------------------------------------------------------
struct alignas(16) RouteLds {
    int32_t ids[kMaxPairs];
    float w[kMaxPairs];
    int32_t n_act;
    int32_t act_experts[kMaxPairs];
    int32_t offsets[kMaxPairs + 1];
    int32_t pair_token[kMaxPairs];
    int32_t pair_src[kMaxPairs];
};

// One wave; lane p < P owns pair p.  Its compacted position is the number of
// pairs ahead of it in (expert, pair index) order, counted from LDS broadcast
// reads of the ids; a slot starts at every position whose pair is its
// expert's first, and slot numbers come from a ballot prefix count.
__device__ void compact_wave(int P, int K, RouteLds& r)
{
    const int lane = threadIdx.x & 63;
    const int e = (lane < P) ? r.ids[lane] : 0;
    int pos = 0, same_before = 0;
    for (int q0 = 0; q0 < P; q0 += 4) {      // reads stay inside the 64-entry array
        const int4 v = *reinterpret_cast<const int4*>(r.ids + q0);
        const int eq[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q = q0 + u;
            if (q < P) {
                pos += (eq[u] < e) || (eq[u] == e && q < lane);
                same_before += (eq[u] == e) && (q < lane);
            }
        }
    }
    // scratch: by position, the expert and whether it starts a slot
    if (lane < P) {
        r.pair_token[pos] = lane / K;
        r.pair_src[pos] = lane;
        r.act_experts[pos] = (same_before == 0) ? e : -1;   // temporary, compacted below
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const int pe = (lane < P) ? r.act_experts[lane] : -1;
    const uint64_t starts = __ballot(pe >= 0);
    const int slot = __popcll(starts & ((1ull << lane) - 1ull));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (pe >= 0) {
        r.act_experts[slot] = pe;
        r.offsets[slot] = lane;
    }
    if (lane == 0) {
        const int n = __popcll(starts);
        r.n_act = n;
        r.offsets[n] = P;
    }
}

__device__ void route_prologue(const RouteSrc& src, RouteLds& r)
{
    const int tid = threadIdx.x, wave = tid >> 6, nw = blockDim.x >> 6;
    const int M = src.M, E = src.E, K = src.K, P = M * K;
    if (src.logits != nullptr) {
        for (int t = wave; t < M; t += nw) topk_wave(src.logits + (size_t)t * E, E, K, r.ids + t * K, r.w + t * K);
    } else {
        for (int i = tid; i < P; i += blockDim.x) r.ids[i] = min(max(src.ids[i], 0), E - 1);   // clamped, never OOB
    }
    __syncthreads();
    if (wave == 0) compact_wave(P, K, r);
    __syncthreads();
}

// Writes the routing and compaction of one workgroup's prologue to global memory.
__device__ void publish_route(const RouteLds& r, const RouteSrc& src, int32_t* ids_out, float* w_out,
                              const Compaction& cp)
{
    const int tid = threadIdx.x, P = src.M * src.K;
    if (tid < P) {
        if (ids_out != nullptr) ids_out[tid] = r.ids[tid];
        if (w_out != nullptr && src.logits != nullptr) w_out[tid] = r.w[tid];
        cp.pair_token[tid] = r.pair_token[tid];
        cp.pair_src[tid] = r.pair_src[tid];
    }
    if (tid < r.n_act) cp.act_experts[tid] = r.act_experts[tid];
    if (tid <= r.n_act) cp.offsets[tid] = r.offsets[tid];
    if (tid == 0) *cp.n_act = r.n_act;
}

__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a)
{
    __shared__ RouteLds r;
    route_prologue(a.src, r);
    publish_route(r, a.src, a.ids_out, a.w_out, a.cp);
}

// ---------------------------------------------------------------------------
// Router: logits[t,e] = x[t] . Wr[e] in fp32 (exact bf16 products), one wave
// per expert row with 16-byte loads; each workgroup also quantises a slice of
// every token; the last workgroup derives and publishes the routing.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float dot_bf16x8(u32x4 x, u32x4 w, float acc)
{
    acc = fmaf(__uint_as_float(x.x << 16), __uint_as_float(w.x << 16), acc);
    acc = fmaf(__uint_as_float(x.x & 0xFFFF0000u), __uint_as_float(w.x & 0xFFFF0000u), acc);
    acc = fmaf(__uint_as_float(x.y << 16), __uint_as_float(w.y << 16), acc);
    acc = fmaf(__uint_as_float(x.y & 0xFFFF0000u), __uint_as_float(w.y & 0xFFFF0000u), acc);
    acc = fmaf(__uint_as_float(x.z << 16), __uint_as_float(w.z << 16), acc);
    acc = fmaf(__uint_as_float(x.z & 0xFFFF0000u), __uint_as_float(w.z & 0xFFFF0000u), acc);
    acc = fmaf(__uint_as_float(x.w << 16), __uint_as_float(w.w << 16), acc);
    acc = fmaf(__uint_as_float(x.w & 0xFFFF0000u), __uint_as_float(w.w & 0xFFFF0000u), acc);
    return acc;
}

template <int H, int MT>
__global__ __launch_bounds__(256) void router_kernel(RouterArgs a)
{
    constexpr int NCH = H / 8;                       // 16-byte chunks per row
    constexpr int CPL = (NCH + kWave - 1) / kWave;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + wave;
    auto valid = [&](int i) { return NCH % kWave == 0 || lane + kWave * i < NCH; };

    // issue every load up front: the router row, each token's hidden state and
    // this workgroup's quantisation slice
    u32x4 wv[CPL];
    if (e < a.E) {
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            if (valid(i)) wv[i] = load_stream((const u32x4*)(a.wr + (size_t)e * H) + lane + kWave * i);
    }
    u32x4 xv[MT][CPL];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            xv[t][i] = (t < a.M && valid(i)) ? *((const u32x4*)(a.x + (size_t)t * H) + lane + kWave * i)
                                             : u32x4{0u, 0u, 0u, 0u};
    const int per = (H + gridDim.x - 1) / gridDim.x;
    const int kq = blockIdx.x * per + threadIdx.x;
    const bool quant = a.act_q != nullptr && threadIdx.x < per && kq < H;
    uint32_t xq[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) xq[t] = (quant && t < a.M) ? a.x[(size_t)t * H + kq] : 0u;

#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (t >= a.M) continue;
        if (e < a.E) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                if (valid(i)) acc = dot_bf16x8(xv[t][i], wv[i], acc);
            const float sum = wave_sum(acc);
            if (lane == 0) a.logits[(size_t)t * a.E + e] = sum;
        }
        if (a.act_q != nullptr) {
            // every wave holds the whole token, so every wave finds the same amax
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                m = fmaxf(m, fmaxf(fabsf(__uint_as_float(xv[t][i].x << 16)), fabsf(__uint_as_float(xv[t][i].x & 0xFFFF0000u))));
                m = fmaxf(m, fmaxf(fabsf(__uint_as_float(xv[t][i].y << 16)), fabsf(__uint_as_float(xv[t][i].y & 0xFFFF0000u))));
                m = fmaxf(m, fmaxf(fabsf(__uint_as_float(xv[t][i].z << 16)), fabsf(__uint_as_float(xv[t][i].z & 0xFFFF0000u))));
                m = fmaxf(m, fmaxf(fabsf(__uint_as_float(xv[t][i].w << 16)), fabsf(__uint_as_float(xv[t][i].w & 0xFFFF0000u))));
            }
            const float amax = wave_max(m);
            const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
            if (quant) a.act_q[(size_t)t * H + kq] = (uint8_t)e4m3_encode(bf16_bits_to_f32(xq[t]) / s);
            if (blockIdx.x == 0 && threadIdx.x == 0) a.act_s[t] = s;
        }
    }

    // The last workgroup to arrive derives the routing once for the layer.
    // One device-scope release per workgroup (by thread 0, after the barrier
    // that orders the workgroup's stores) and one acquire in the last one.
    __shared__ RouteLds rl;
    __shared__ int last;
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        last = atomicAdd(a.counter, 1u) == gridDim.x - 1;
    }
    __syncthreads();
    if (!last) return;
    __threadfence();
    const RouteSrc src{a.M, a.E, a.K, a.logits, nullptr};
    route_prologue(src, rl);
    publish_route(rl, src, a.ids_out, a.w_out, a.cp);
    if (threadIdx.x == 0) __hip_atomic_store(a.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Fused gate/up GEMV.  A row of W13 is H/32 chunks of 16 code bytes, each
// chunk exactly one E8M0 block.  LPR lanes share a row and each takes CPL
// chunks (lane li takes chunks li, li+LPR, ...), so one load instruction of the
// group covers LPR*16 contiguous bytes.  A lane holds the gate row r and the up
// row I+r of one expert, so SiLU(g)*u is formed in registers.
// ---------------------------------------------------------------------------
template <int H, int I>
struct GateUpGeom {
    static constexpr int kChunks = H / 32;
    static constexpr int kLanesPerRow = (kChunks % 16 == 0) ? 16 : (kChunks % 8 == 0) ? 8
                                      : (kChunks % 4 == 0) ? 4 : (kChunks % 2 == 0) ? 2 : 1;
    static constexpr int kChunksPerLane = kChunks / kLanesPerRow;
    static constexpr int kRowsPerWave = kWave / kLanesPerRow;
    static constexpr int kWaves = 4;
    static constexpr int kRowsPerBlock = kRowsPerWave * kWaves;
    static_assert(H % 32 == 0 && I % kRowsPerBlock == 0, "unsupported gate/up shape");
    static constexpr int kBlocksPerExpert = I / kRowsPerBlock;
};

template <int H, int I, int MT>
__global__ __launch_bounds__(256) void gate_up_kernel(GateUpArgs a)
{
    using G = GateUpGeom<H, I>;
    constexpr int CH = G::kChunks, LPR = G::kLanesPerRow, CPL = G::kChunksPerLane;
    __shared__ u32x4 act[MT * 4 * CH];          // [token][q][chunk] of 8 halves

    // 0. this workgroup's expert and its tokens, from the published compaction
    const int P = a.M * a.K;
    const int slot = blockIdx.y;
    if (slot >= *a.cp.n_act) return;
    const int e = min(max(a.cp.act_experts[slot], 0), a.E - 1);
    const int p0 = min(max(a.cp.offsets[slot], 0), P);
    const int nt = max(0, min(min(a.cp.offsets[slot + 1], P) - p0, MT));   // at most M <= MT tokens
    int tok_of[MT], pair_of[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        tok_of[t] = (t < nt) ? min(max(a.cp.pair_token[p0 + t], 0), a.M - 1) : 0;
        pair_of[t] = (t < nt) ? min(max(a.cp.pair_src[p0 + t], 0), P - 1) : 0;
    }

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane % LPR, grp = lane / LPR;
    const int r = blockIdx.x * G::kRowsPerBlock + wave * G::kRowsPerWave + grp;

    // 1. issue the weight stream for this lane
    const u32x4* grow = (const u32x4*)(a.w13 + ((size_t)e * 2 * I + r) * (H / 2));
    const u32x4* urow = grow + (size_t)I * CH;
    const uint8_t* gsc = a.s13 + ((size_t)e * 2 * I + r) * CH;
    const uint8_t* usc = gsc + (size_t)I * CH;
    u32x4 wg[CPL], wu[CPL];
    uint32_t sg[CPL], su[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        wg[i] = load_stream(grow + li + LPR * i);
        wu[i] = load_stream(urow + li + LPR * i);
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        sg[i] = gsc[li + LPR * i];
        su[i] = usc[li + LPR * i];
    }

    // 1b. pull this workgroup's share of the expert's down-projection weights
    // into the memory-side cache, so the down kernel finds them there
    constexpr size_t W2C = (size_t)H * I / 2, W2S = (size_t)H * I / 32;     // bytes per expert
    constexpr int PFC = (int)(W2C / G::kBlocksPerExpert / 16), PFS = (int)(W2S / G::kBlocksPerExpert / 16);
    static_assert(W2C % (16 * G::kBlocksPerExpert) == 0 && W2S % (16 * G::kBlocksPerExpert) == 0, "prefetch split");
    constexpr int PF_PER = (PFC + PFS + 255) / 256;
    u32x4 pf[PF_PER];
    if (a.w2 != nullptr) {
#pragma unroll
        for (int j = 0; j < PF_PER; ++j) {
            const int i = threadIdx.x + 256 * j;
            if (i < PFC) pf[j] = *((const u32x4*)(a.w2 + e * W2C) + blockIdx.x * PFC + i);
            else if (i < PFC + PFS) pf[j] = *((const u32x4*)(a.sw2 + e * W2S) + blockIdx.x * PFS + (i - PFC));
            else pf[j] = u32x4{0u, 0u, 0u, 0u};
        }
    }

    // 2. stage this expert's tokens' activations as f16 in LDS
    for (int idx = threadIdx.x; idx < nt * (H / 8); idx += blockDim.x) {
        const int t = idx / (H / 8), g8 = idx % (H / 8);
        const int tok = min(max(a.cp.pair_token[p0 + t], 0), a.M - 1);
        const u32x2 codes = *((const u32x2*)(a.act_q + (size_t)tok * H) + g8);
        act[(t * 4 + (g8 & 3)) * CH + (g8 >> 2)] = e4m3x8_to_half8(codes);
    }
    __syncthreads();

    // 3. dot products, one E8M0 block at a time
    float accg[MT], accu[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) accg[t] = accu[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = li + LPR * i;
        half2_t hg[16], hu[16];
        e2m1x8_to_half(wg[i].x, hg + 0);
        e2m1x8_to_half(wg[i].y, hg + 4);
        e2m1x8_to_half(wg[i].z, hg + 8);
        e2m1x8_to_half(wg[i].w, hg + 12);
        e2m1x8_to_half(wu[i].x, hu + 0);
        e2m1x8_to_half(wu[i].y, hu + 4);
        e2m1x8_to_half(wu[i].z, hu + 8);
        e2m1x8_to_half(wu[i].w, hu + 12);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t < nt) {
                const u32x4 a0 = act[(t * 4 + 0) * CH + c], a1 = act[(t * 4 + 1) * CH + c];
                const u32x4 a2 = act[(t * 4 + 2) * CH + c], a3 = act[(t * 4 + 3) * CH + c];
                accg[t] += ldexp_e8m0(block_dot(hg, a0, a1, a2, a3), sg[i]);
                accu[t] += ldexp_e8m0(block_dot(hu, a0, a1, a2, a3), su[i]);
            }
        }
    }

    // 4. reduce over the LPR lanes of a row, SiLU(g)*u
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (t < nt) {
            accg[t] = group_sum<LPR>(accg[t]);
            accu[t] = group_sum<LPR>(accu[t]);
            const float st = a.act_s[tok_of[t]];
            const float g = accg[t] * st, u = accu[t] * st;
            if (li == 0) a.h[(size_t)pair_of[t] * I + r] = g / (1.0f + expf(-g)) * u;
        }
    }
    if (a.w2 != nullptr) {           // retire the prefetch loads
        uint32_t x = 0;
#pragma unroll
        for (int j = 0; j < PF_PER; ++j) x ^= pf[j].x ^ pf[j].y ^ pf[j].z ^ pf[j].w;
        if (a.sink != nullptr) a.sink[threadIdx.x] = x;
    }
}

// ---------------------------------------------------------------------------
// Per-(token, expert) FP8 requantisation of the intermediate, a wave per row
// of I values: s2 = amax / 448 (1 for an all-zero row), q2 = E4M3(h / s2),
// with a correctly rounded division.
// ---------------------------------------------------------------------------
template <int I>
__global__ __launch_bounds__(256) void requant_kernel(RequantArgs a)
{
    constexpr int PER = I / kWave;
    static_assert(I % kWave == 0, "requantisation needs I % 64 == 0");
    const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (p >= a.P) return;
    const int lane = threadIdx.x & 63;
    float v[PER];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        v[i] = a.h[(size_t)p * I + lane + kWave * i];
        m = fmaxf(m, fabsf(v[i]));
    }
    m = wave_max(m);
    const float s = (m == 0.0f) ? 1.0f : m / 448.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) a.q2[(size_t)p * I + lane + kWave * i] = (uint8_t)e4m3_encode(v[i] / s);
    if (lane == 0) a.s2[p] = s;
}

// ---------------------------------------------------------------------------
// Down GEMV + combine.  A workgroup owns RPB output rows for every token; its
// 8 waves split the selected experts (wave w takes slots w, w+8, ...), each
// accumulating per-token partial sums in a fixed slot order; the waves' sums
// are then added in wave order.  The FP8 intermediate of every pair is held
// once per workgroup as f16 in LDS.
// ---------------------------------------------------------------------------
template <int H, int I>
struct DownGeom {
    static constexpr int kChunks = I / 32;
    static constexpr int kLanesPerRow = (kChunks % 8 == 0) ? 8 : (kChunks % 4 == 0) ? 4
                                      : (kChunks % 2 == 0) ? 2 : 1;
    static constexpr int kChunksPerLane = kChunks / kLanesPerRow;
    static constexpr int kRowsPerBlock = kWave / kLanesPerRow;
    static constexpr int kWaves = 8;
    static_assert(I % 32 == 0 && H % kRowsPerBlock == 0, "unsupported down shape");
};

template <int H, int I, int MT>
__global__ __launch_bounds__(512) void down_kernel(DownArgs a)
{
    using G = DownGeom<H, I>;
    constexpr int CH = G::kChunks, LPR = G::kLanesPerRow, CPL = G::kChunksPerLane, RPB = G::kRowsPerBlock;
    extern __shared__ u32x4 q2h[];                 // [pair][q][chunk] of 8 halves
    __shared__ float red[G::kWaves][RPB][MT];
    __shared__ float s2l[kMaxPairs];

    const int P = a.M * a.K;
    const int n_act = min(*a.cp.n_act, min(a.E, P));
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane % LPR, grp = lane / LPR;
    const int n = blockIdx.x * RPB + grp;

    auto load_slot = [&](int slot, u32x4* wv, uint32_t* sv) {
        const int e = min(max(a.cp.act_experts[slot], 0), a.E - 1);
        const u32x4* row = (const u32x4*)(a.w2 + ((size_t)e * H + n) * (I / 2));
        const uint8_t* sc = a.sw2 + ((size_t)e * H + n) * CH;
#pragma unroll
        for (int i = 0; i < CPL; ++i) wv[i] = load_stream(row + li + LPR * i);
#pragma unroll
        for (int i = 0; i < CPL; ++i) sv[i] = sc[li + LPR * i];
    };

    int slot = wave;
    u32x4 wv[CPL];
    uint32_t sv[CPL];
    if (slot < n_act) load_slot(slot, wv, sv);

    // the FP8 intermediate as f16, while the weight loads are in flight
    for (int idx = threadIdx.x; idx < P * (I / 8); idx += blockDim.x) {
        const int p = idx / (I / 8), g8 = idx % (I / 8);
        const u32x2 codes = *((const u32x2*)(a.q2 + (size_t)p * I) + g8);
        q2h[(p * 4 + (g8 & 3)) * CH + (g8 >> 2)] = e4m3x8_to_half8(codes);
    }
    for (int p = threadIdx.x; p < P; p += blockDim.x) s2l[p] = a.s2[p];
    __syncthreads();

    float acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = 0.0f;
    for (; slot < n_act; slot += G::kWaves) {
        u32x4 nwv[CPL];
        uint32_t nsv[CPL];
        const int nslot = slot + G::kWaves;
        if (nslot < n_act) load_slot(nslot, nwv, nsv);
        half2_t hw[CPL * 16];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            e2m1x8_to_half(wv[i].x, hw + 16 * i + 0);
            e2m1x8_to_half(wv[i].y, hw + 16 * i + 4);
            e2m1x8_to_half(wv[i].z, hw + 16 * i + 8);
            e2m1x8_to_half(wv[i].w, hw + 16 * i + 12);
        }
        const int q0 = min(max(a.cp.offsets[slot], 0), P), q1 = min(a.cp.offsets[slot + 1], P);
        for (int qq = q0; qq < q1; ++qq) {
            const int p = min(max(a.cp.pair_src[qq], 0), P - 1);
            const int tok = a.cp.pair_token[qq];
            float d = 0.0f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = li + LPR * i;
                const u32x4 a0 = q2h[(p * 4 + 0) * CH + c], a1 = q2h[(p * 4 + 1) * CH + c];
                const u32x4 a2 = q2h[(p * 4 + 2) * CH + c], a3 = q2h[(p * 4 + 3) * CH + c];
                d += ldexp_e8m0(block_dot(hw + 16 * i, a0, a1, a2, a3), sv[i]);
            }
            d = group_sum<LPR>(d);
            const float coef = a.topk_w[p] * s2l[p];
#pragma unroll
            for (int t = 0; t < MT; ++t)
                if (t == tok) acc[t] = fmaf(coef, d, acc[t]);
        }
        if (nslot < n_act) {
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                wv[i] = nwv[i];
                sv[i] = nsv[i];
            }
        }
    }
    if (li == 0) {
#pragma unroll
        for (int t = 0; t < MT; ++t) red[wave][grp][t] = acc[t];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < RPB * a.M; idx += blockDim.x) {
        const int row = idx % RPB, t = idx / RPB;
        float s = red[0][row][t];
#pragma unroll
        for (int w = 1; w < G::kWaves; ++w) s += red[w][row][t];
        a.out[(size_t)t * H + blockIdx.x * RPB + row] = s;
    }
}

// ---------------------------------------------------------------------------
// Small utility kernels.
// ---------------------------------------------------------------------------
__global__ void fp8_encode_range_kernel(uint32_t first, int64_t n, uint8_t* __restrict__ q)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        q[i] = (uint8_t)e4m3_encode(__uint_as_float(first + (uint32_t)i));
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t v)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

// ---------------------------------------------------------------------------
// Launchers: the compiled shape set is (H, I) in {(256, 64), (2560, 768)} with
// token bounds 1, 2, 4 and 8.
// ---------------------------------------------------------------------------
bool gemv_shape_supported(int H, int I)
{
    return (H == 256 && I == 64) || (H == 2560 && I == 768);
}

template <int H, int I, int MT>
static hipError_t launch_gate_up_t(int S, const GateUpArgs& a, hipStream_t s)
{
    using G = GateUpGeom<H, I>;
    hipLaunchKernelGGL((gate_up_kernel<H, I, MT>), dim3(G::kBlocksPerExpert, S), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int H, int I, int MT>
static hipError_t launch_down_t(const DownArgs& a, hipStream_t s)
{
    using G = DownGeom<H, I>;
    const size_t lds = (size_t)a.M * a.K * I * 2;
    if (lds > 64 * 1024) {   // above the default dynamic-LDS limit (gfx950 has 160 KiB per CU)
        hipError_t err = hipFuncSetAttribute((const void*)down_kernel<H, I, MT>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL((down_kernel<H, I, MT>), dim3(H / G::kRowsPerBlock), dim3(512), lds, s, a);
    return hipGetLastError();
}

template <int H, int MT>
static hipError_t launch_router_t(const RouterArgs& a, hipStream_t s)
{
    // one wave per expert row; workgroup t also quantises token t, so there
    // are at least M workgroups
    const int blocks = (a.E + 3) / 4 > a.M ? (a.E + 3) / 4 : a.M;
    hipLaunchKernelGGL((router_kernel<H, MT>), dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

#define MOE_DISPATCH_MT(MT_VAR, CALL)                      \
    switch (MT_VAR) {                                      \
        case 1: { constexpr int MTc = 1; return CALL; }    \
        case 2: { constexpr int MTc = 2; return CALL; }    \
        case 4: { constexpr int MTc = 4; return CALL; }    \
        case 8: { constexpr int MTc = 8; return CALL; }    \
        default: return hipErrorInvalidValue;              \
    }

hipError_t launch_router(int H, int mt, const RouterArgs& a, hipStream_t s)
{
    if (H == 256) { MOE_DISPATCH_MT(mt, (launch_router_t<256, MTc>(a, s))) }
    if (H == 2560) { MOE_DISPATCH_MT(mt, (launch_router_t<2560, MTc>(a, s))) }
    return hipErrorInvalidValue;
}

hipError_t launch_quant(int H, const uint16_t* x, int M, uint8_t* q, float* sc, hipStream_t s)
{
    if (H == 256) hipLaunchKernelGGL(quant_kernel<256>, dim3(M), dim3(256), 0, s, x, q, sc);
    else if (H == 2560) hipLaunchKernelGGL(quant_kernel<2560>, dim3(M), dim3(256), 0, s, x, q, sc);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s)
{
    hipLaunchKernelGGL(topk_kernel, dim3(1), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gate_up(int H, int I, int mt, int S, const GateUpArgs& a, hipStream_t s)
{
    if (H == 256 && I == 64) { MOE_DISPATCH_MT(mt, (launch_gate_up_t<256, 64, MTc>(S, a, s))) }
    if (H == 2560 && I == 768) { MOE_DISPATCH_MT(mt, (launch_gate_up_t<2560, 768, MTc>(S, a, s))) }
    return hipErrorInvalidValue;
}

hipError_t launch_down(int H, int I, int mt, const DownArgs& a, hipStream_t s)
{
    if (H == 256 && I == 64) { MOE_DISPATCH_MT(mt, (launch_down_t<256, 64, MTc>(a, s))) }
    if (H == 2560 && I == 768) { MOE_DISPATCH_MT(mt, (launch_down_t<2560, 768, MTc>(a, s))) }
    return hipErrorInvalidValue;
}

hipError_t launch_requant(int I, const RequantArgs& a, hipStream_t s)
{
    if (a.P <= 0) return hipSuccess;
    const dim3 grid((a.P + 3) / 4);
    if (I == 64) hipLaunchKernelGGL(requant_kernel<64>, grid, dim3(256), 0, s, a);
    else if (I == 768) hipLaunchKernelGGL(requant_kernel<768>, grid, dim3(256), 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_fp8_encode_range(uint32_t first, int64_t n, uint8_t* q, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    const int64_t blocks64 = (n + 255) / 256;
    const int blocks = (int)(blocks64 < 16384 ? blocks64 : 16384);
    hipLaunchKernelGGL(fp8_encode_range_kernel, dim3(blocks), dim3(256), 0, s, first, n, q);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

const char* kernel_names(int H, int I, int mt)
{
    (void)mt;
    if (H == 256 && I == 64)
        return "router_kernel<H=256> (top-K + compaction in the last WG) -> gate_up_kernel<H=256,I=64> (8 lanes/row, "
               "32 row-pairs/WG) -> requant_kernel<I=64> -> down_kernel<H=256,I=64> (2 lanes/row, 32 rows/WG)";
    if (H == 2560 && I == 768)
        return "router_kernel<H=2560> (top-K + compaction in the last WG) -> gate_up_kernel<H=2560,I=768> "
               "(16 lanes/row, 16 row-pairs/WG, 48 WGs/expert, prefetches the down weights) -> requant_kernel<I=768> "
               "-> down_kernel<H=2560,I=768> (8 lanes/row, 8 rows/WG, 320 WGs)";
    return "unsupported";
}

}  // namespace moe
