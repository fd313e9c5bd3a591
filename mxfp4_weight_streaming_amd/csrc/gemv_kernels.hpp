// gemv_kernels.hpp -- gfx950 kernels of the W4A8 MoE decode layer (M <= 8 tokens),
// device code only: compiled ahead of time through moe_kernels.hip and at run
// time by hipRTC for shapes outside the ahead-of-time set.
//
// The pages find batch-1 MoE decode bound by reading expert weights ([EN]
// "Why is MoE decoding on DGX Spark memory-bound?"), so the kernels are built
// around streaming MXFP4 bytes from HBM once, with wide loads issued before
// any dependent work.  A layer is three kernels on one stream:
//   router_kernel   fp32 router GEMV (one wave per expert row) and per-token
//                   FP8 quantisation of the activations.
//   gate_up_kernel  every workgroup derives the routing from the logits
//                   (top-K, renormalised weights, token->expert compaction:
//                   [EN] "What is Ling 3.0...", 8 routed experts per token;
//                   [EN] "What are the 3 optimizations?", item 3: a 4-token
//                   verify touches up to 32 experts), then streams the fused
//                   gate/up MXFP4 GEMV of (expert, row block) items with the
//                   SiLU(gate)*up epilogue ([EN] same section, item 1: the
//                   768-wide expert layer).  (Pulling the down weights into
//                   the memory-side cache here was measured slower: it adds
//                   their bytes to this kernel's stream for little gain in
//                   the next.)
//   down_kernel     requantises the intermediate to FP8 per (token, expert)
//                   row while its weight loads are in flight, then the down
//                   GEMV over all selected experts and the router-weighted
//                   combine in a fixed order (no float atomics).
// Workgroups never synchronise with each other inside a kernel: on this chip
// a device-scope release costs every workgroup a serialised L2 write-back,
// far dearer than repeating a little work in every workgroup.
// The M <= 8 path is a GEMV: it uses the vector ALU (dot2 on exactly decoded
// f16 operands, fp32 accumulation), not the matrix cores.
//   [EN] = "NVIDIA Shows 3 Ways to Speed Up MoE Inference on DGX Spark,
//          Lifting Ling-3.0-flash Throughput 42.5%"
#pragma once

#include "device_common.hpp"
#include "moe_types.hpp"
#include "topk_wave.hpp"

namespace moe {


// ---------------------------------------------------------------------------
// Per-token activation quantisation (one workgroup, one token).
// s = amax / 448 (1 for an all-zero row), a correctly rounded binary32
// division, and q = E4M3(x / s) with the code of the correctly rounded
// quotient (quant_div).
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
    const QuantScale qs = quant_scale(amax);
    for (int k = threadIdx.x; k < H; k += blockDim.x) q[k] = (uint8_t)e4m3_encode(quant_div(bf16_bits_to_f32(x[k]), qs));
    if (threadIdx.x == 0) *s_out = qs.s;
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
// Routing prologue, run by every thread of a workgroup: top-K (from logits) or
// caller ids, then token->expert compaction, all in LDS.  Distinct experts get
// slots in ascending id; the pairs of a slot are in ascending token order.
// ---------------------------------------------------------------------------
struct alignas(16) RouteLds {
    uint32_t keys[kMaxPairs];                   // compaction scratch: each pair's sort key
    int32_t ids[kMaxPairs];
    float w[kMaxPairs];
    int32_t n_act;
    int32_t act_experts[kMaxPairs + 1];
    int32_t offsets[kMaxPairs + 2];
    int32_t pair_token[kMaxPairsExt];
    int32_t pair_src[kMaxPairsExt];
    int32_t sorted_e[kMaxPairs];                // compaction scratch: expert at each position
};

// One wave; lane p < P owns pair p, its expert e_p and the key e_p * 64 + p
// (keys are distinct).  The pair's position in (expert, pair index) order is
// the number of smaller keys, counted against every pair's key read from LDS
// (broadcast reads, all issued before the first compare; a chain of readlane
// steps was slower).  The pairs are stored at their positions; a position
// opens a slot when its expert differs from the previous position's, and
// slots are numbered by counting the opening positions below.
template <int PMAX>
__device__ void compact_wave_t(int P, int K, RouteLds& r)
{
    static_assert(PMAX % 4 == 0 && PMAX <= kMaxPairs, "compaction keys are read four at a time");
    const int lane = threadIdx.x & 63;
    const int e = r.ids[min(lane, P - 1)];
    const uint32_t key = lane < P ? (uint32_t)e * 64u + (uint32_t)lane : 0xFFFFFFFFu;
    if (lane < PMAX) r.keys[lane] = key;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    uint4 kq[PMAX / 4];
#pragma unroll
    for (int q = 0; q < PMAX / 4; ++q) kq[q] = reinterpret_cast<const uint4*>(r.keys)[q];
    int pos = 0;
#pragma unroll
    for (int q = 0; q < PMAX / 4; ++q)
        pos += (kq[q].x < key ? 1 : 0) + (kq[q].y < key ? 1 : 0) + (kq[q].z < key ? 1 : 0) + (kq[q].w < key ? 1 : 0);
    if (lane < P) {
        r.sorted_e[pos] = e;
        r.pair_token[pos] = lane / K;
        r.pair_src[pos] = lane;
    }
    // the stores above are read back by other lanes of this wave
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
    const int i = min(lane, P - 1);
    const int se = r.sorted_e[i], prev = r.sorted_e[max(i - 1, 0)];
    const bool open = lane < P && (lane == 0 || se != prev);
    const uint64_t opens = __ballot(open);
    const int slot = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(opens >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)opens, 0u));
    if (open) {
        r.act_experts[slot] = se;
        r.offsets[slot] = lane;
    }
    if (lane == 0) {
        const int n = __popcll(opens);
        r.n_act = n;
        r.offsets[n] = P;
    }
}

__device__ void compact_wave(int P, int K, RouteLds& r)
{
    if (P <= 8) compact_wave_t<8>(P, K, r);
    else if (P <= 16) compact_wave_t<16>(P, K, r);
    else if (P <= 32) compact_wave_t<32>(P, K, r);
    else compact_wave_t<64>(P, K, r);
}

// Compaction of the ids in r.ids (and the shared expert's slot), by wave 0;
// the caller synchronises before and after.  distinct: the ids of the one
// token are known to be distinct (routed by top-K), which takes a fast path.
__device__ __forceinline__ void route_compact(int M, int K, bool distinct, int shared, RouteLds& r)
{
    const int tid = threadIdx.x, P = M * K;
    if ((tid >> 6) != 0) return;
    if (M == 1 && distinct) {
        // one token routed here: its K experts are distinct, so the slots
        // are the experts in ascending id and slot s holds exactly one
        // pair (caller ids may repeat an expert: they take the general
        // compaction)
        const int lane = tid & 63;
        const int4 a4 = *reinterpret_cast<const int4*>(r.ids), b4 = *reinterpret_cast<const int4*>(r.ids + 4);
        const int all[8] = {a4.x, a4.y, a4.z, a4.w, b4.x, b4.y, b4.z, b4.w};
        const int e = r.ids[lane & (kMaxTopK - 1)];
        int slot = 0;
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) slot += (k < K) && all[k] < e;
        if (lane < K) {
            r.act_experts[slot] = e;
            r.offsets[slot] = slot;
            r.pair_token[slot] = 0;
            r.pair_src[slot] = lane;
        }
        if (lane == 0) {
            r.n_act = K;
            r.offsets[K] = K;
        }
    } else {
        compact_wave(P, K, r);
    }
    if (shared) {
        // the shared expert's slot follows the routed ones: every token,
        // pair row P + t (its weight, 1, is applied by the down kernel)
        const int lane = tid & 63;
        if (lane < M) {
            r.pair_token[P + lane] = lane;
            r.pair_src[P + lane] = P + lane;
        }
        if (lane == 0) {
            const int n = r.n_act;
            r.act_experts[n] = kSharedExpert;
            r.offsets[n + 1] = P + M;
            r.n_act = n + 1;
        }
    }
}

// LOGITS = false: the caller routes from logits itself (the one-token gate/up
// kernel ranks them in registers), so the top-K is not compiled in here.
// want_w: the softmax weights are wanted in r.w (only the workgroup that
// publishes the routing needs them; the others skip their arithmetic).
template <bool LOGITS = true>
__device__ void route_prologue(const RouteSrc& src, RouteLds& r, bool want_w = true)
{
    const int tid = threadIdx.x, wave = tid >> 6, nw = blockDim.x >> 6;
    const int M = src.M, E = src.E, K = src.K, P = M * K;
    if (LOGITS && src.logits != nullptr) {
        for (int t = wave; t < M; t += nw)
            topk_wave(src.logits + (size_t)t * E, E, K, r.ids + t * K, want_w ? r.w + t * K : nullptr);
    } else {
        for (int i = tid; i < P; i += blockDim.x) r.ids[i] = min(max(src.ids[i], 0), E - 1);   // clamped, never OOB
    }
    __syncthreads();
    route_compact(M, K, src.logits != nullptr, src.shared, r);
    __syncthreads();
}

// Writes the routing and compaction of one workgroup's prologue to global memory.
__device__ void publish_route(const RouteLds& r, const RouteSrc& src, int32_t* ids_out, float* w_out,
                              const Compaction& cp)
{
    const int tid = threadIdx.x, P = src.M * src.K, Pe = P + (src.shared ? src.M : 0);
    if (tid < P) {
        if (ids_out != nullptr) ids_out[tid] = r.ids[tid];
        if (w_out != nullptr && src.logits != nullptr) w_out[tid] = r.w[tid];
    }
    if (tid < Pe) {
        cp.pair_token[tid] = r.pair_token[tid];
        cp.pair_src[tid] = r.pair_src[tid];
    }
    if (tid < r.n_act) cp.act_experts[tid] = r.act_experts[tid];
    if (tid <= r.n_act) cp.offsets[tid] = r.offsets[tid];
    if (tid == 0) *cp.n_act = r.n_act;
}

// One token routed from its logits, in the gate/up kernel: the ranks held by
// wave 0 of workgroup 0 (TopkRanks, all K) are published as the routing and
// the ascending-id compaction that route_prologue and publish_route would
// give.  Lane r < K holds the rank-r expert.
__device__ void publish_rank1(const TopkRanks& t, const RouteSrc& src, int32_t* ids_out, float* w_out,
                              const Compaction& cp)
{
    const int lane = threadIdx.x & 63, K = src.K;
    const int n = K + (src.shared ? 1 : 0);
    const float w = topk_weight(t, K);
    int s = 0;                                  // ascending-id slot: the selected experts below (distinct)
#pragma unroll
    for (int q = 0; q < kMaxTopK; ++q) s += (q < K && __builtin_amdgcn_readlane(t.e, q) < t.e) ? 1 : 0;
    if (lane < K) {
        cp.act_experts[s] = t.e;
        cp.offsets[s] = s;
        cp.pair_token[s] = 0;
        cp.pair_src[s] = lane;
        if (ids_out != nullptr) ids_out[lane] = t.e;
        if (w_out != nullptr) w_out[lane] = w;
    }
    if (lane == 0) {
        if (src.shared) {
            cp.act_experts[K] = kSharedExpert;
            cp.pair_token[K] = 0;
            cp.pair_src[K] = K;
        }
        cp.offsets[K] = K;
        cp.offsets[n] = n;
        *cp.n_act = n;
    }
}

__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a)
{
    __shared__ RouteLds r;
    route_prologue(a.src, r);
    publish_route(r, a.src, a.ids_out, a.w_out, a.cp);
}

// ---------------------------------------------------------------------------
// Router: logits[t,e] = x[t] . Wr[e] in fp32 (exact bf16 products).  One
// workgroup per expert row: thread c holds the 16-byte chunk c (8 values) of
// the row and of every token, so a workgroup sees every token whole and finds
// its amax with 8 values per thread; the per-thread partial dot products and
// maxima are reduced on DPP within rows of 16 lanes and then in LDS in a fixed
// order.  The activation quantisation (chunk, token) items are spread over
// the threads of the whole grid, one item each.
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

// Largest |value| of 8 bf16 (NaN inputs are skipped, as by fmaxf).
__device__ __forceinline__ float amax_bf16x8(u32x4 x)
{
    float m = fmaxf(fabsf(__uint_as_float(x.x << 16)), fabsf(__uint_as_float(x.x & 0xFFFF0000u)));
    m = fmaxf(m, fmaxf(fabsf(__uint_as_float(x.y << 16)), fabsf(__uint_as_float(x.y & 0xFFFF0000u))));
    m = fmaxf(m, fmaxf(fabsf(__uint_as_float(x.z << 16)), fabsf(__uint_as_float(x.z & 0xFFFF0000u))));
    return fmaxf(m, fmaxf(fabsf(__uint_as_float(x.w << 16)), fabsf(__uint_as_float(x.w & 0xFFFF0000u))));
}

// Maximum over aligned rows of 16 lanes; every lane of a row gets it.
__device__ __forceinline__ float row16_max(float v)
{
    v = fmaxf(v, dpp_f32<kDppXor1>(v));
    v = fmaxf(v, dpp_f32<kDppXor2>(v));
    v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
    return fmaxf(v, dpp_f32<kDppMirror>(v));
}

template <int H, int MT>
__global__ __launch_bounds__(router_threads(H)) void router_kernel(RouterArgs a)
{
    constexpr int NCH = H / 8;                       // 16-byte chunks per row
    constexpr int NT = router_threads(H);
    constexpr int NR = NT / 16;                      // rows of 16 lanes
    __shared__ float red_dot[MT][NR], red_max[MT][NR];
    const int tid = threadIdx.x, lane = tid & 63;
    const int e = blockIdx.x;                        // the grid is one workgroup per expert
    const int M = a.M;
    const bool own = tid < NCH;
    const int c = own ? tid : NCH - 1;               // past the row: a copy of the last chunk, counted nowhere

    // every load first, unconditional (clamped): the row chunk, every token's
    // chunk and this thread's quantisation item (chunk qi of the [M,H] array)
    const u32x4 w = load_stream(reinterpret_cast<const u32x4*>(a.wr + (size_t)e * H) + c);
    u32x4 xv[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) xv[t] = *(reinterpret_cast<const u32x4*>(a.x + (size_t)min(t, M - 1) * H) + c);
    const int nq = a.act_q != nullptr ? NCH * M : 0;
    const int qi = blockIdx.x + gridDim.x * tid;
    const u32x4 xq = *(reinterpret_cast<const u32x4*>(a.x) + min(qi, NCH * M - 1));

#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const float d = group_sum<16>(own ? dot_bf16x8(xv[t], w, 0.0f) : 0.0f);
        const float m = row16_max(own ? amax_bf16x8(xv[t]) : 0.0f);
        if ((lane & 15) == 0) {
            red_dot[t][tid >> 4] = d;
            red_max[t][tid >> 4] = m;
        }
    }
    __syncthreads();
    // token t's scale, found by every thread that needs it from the row maxima
    // (max is exact in any order, so all find the same value)
    auto token_scale = [&](int t) {
        float m = 0.0f;
#pragma unroll
        for (int r = 0; r < NR; ++r) m = fmaxf(m, red_max[t][r]);
        return quant_scale(m);
    };
    if (tid < M) {
        float d = 0.0f;
#pragma unroll
        for (int r = 0; r < NR; ++r) d += red_dot[tid][r];
        a.logits[(size_t)tid * a.E + e] = d;
        if (blockIdx.x == 0 && a.act_q != nullptr) a.act_s[tid] = token_scale(tid).s;
    }
    auto quantise = [&](int item, u32x4 v) {
        const QuantScale qs = token_scale(item / NCH);
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
        uint32_t code[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t b = (j & 1) ? (vv[j >> 1] & 0xFFFF0000u) : (vv[j >> 1] << 16);
            code[j >> 2] |= e4m3_encode(quant_div(__uint_as_float(b), qs)) << (8 * (j & 3));
        }
        *reinterpret_cast<u32x2*>(a.act_q + (size_t)item * 8) = u32x2{code[0], code[1]};
    };
    if (qi < nq) quantise(qi, xq);
    // more items than threads in the grid (few experts): one at a time
    for (int q = qi + gridDim.x * NT; q < nq; q += gridDim.x * NT)
        quantise(q, *(reinterpret_cast<const u32x4*>(a.x) + q));
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
    static constexpr int kLanesPerRow = gate_up_lanes_per_row(H);
    static constexpr int kChunksPerLane = kChunks / kLanesPerRow;
    static constexpr int kRowsPerWave = kWave / kLanesPerRow;
    static constexpr int kWaves = 4;
    static constexpr int kRowsPerBlock = kRowsPerWave * kWaves;
    static_assert(kRowsPerBlock == gate_up_rows_per_block(H), "gate/up blocking");
    static_assert(H % 32 == 0 && I % kRowsPerBlock == 0, "unsupported gate/up shape");
    static constexpr int kBlocksPerExpert = I / kRowsPerBlock;
};

template <int H, int I, int MT>
__global__ __launch_bounds__(256) void gate_up_kernel(GateUpArgs a)
{
    using G = GateUpGeom<H, I>;
    constexpr int CH = G::kChunks, LPR = G::kLanesPerRow, CPL = G::kChunksPerLane, BPE = G::kBlocksPerExpert;
    __shared__ RouteLds rl;
    __shared__ u32x4 act[MT * 4 * CH];          // [token][q][chunk] of 8 halves
    __shared__ float act_sl[MT];                // per-token activation scales

    const int M = a.src.M;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = lane % LPR, grp = lane / LPR;

    // 0. every token's activations as f16 in LDS.  From FP8 codes (act_q):
    //    their loads go out first and overlap the routing prologue.  From the
    //    bf16 hidden states of one or two tokens (x): the waves from M on
    //    quantise them while waves 0..M-1 derive the routing, each reading a
    //    whole token so that they agree on its amax without a barrier (the
    //    same arithmetic as the router's quantisation: s = amax / 448, codes
    //    E4M3(x / s)).  One token is split over waves 1-3, two tokens take
    //    waves 2 and 3.
    // (compiled for one or two tokens only: the larger kernels were measured
    // slower with this code in them, unused)
    const bool from_x = MT <= 2 && a.x != nullptr;
    constexpr int NST = (MT * (H / 8) + 255) / 256;
    const int n8 = M * (H / 8);
    u32x2 stg[NST];
    float s_tok = 0.0f;
    if (!from_x) {
#pragma unroll
        for (int j = 0; j < NST; ++j) stg[j] = ((const u32x2*)a.act_q)[min((int)threadIdx.x + 256 * j, n8 - 1)];
        s_tok = a.act_s[min((int)threadIdx.x, M - 1)];
    } else if constexpr (MT <= 2) {
        if (wave >= M) {
            constexpr int NC8 = H / 8, CPL8 = (NC8 + kWave - 1) / kWave;   // 16-byte chunks of a token
            const int qw = wave - M, t = qw % M, split = (4 - M) / M, part = qw / M;
            u32x4 xv[CPL8];
#pragma unroll
            for (int i = 0; i < CPL8; ++i)
                xv[i] = reinterpret_cast<const u32x4*>(a.x + (size_t)t * H)[min(lane + kWave * i, NC8 - 1)];
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < CPL8; ++i)
                if (lane + kWave * i < NC8) m = fmaxf(m, amax_bf16x8(xv[i]));
            const QuantScale qs = quant_scale(wave_max(m));
#pragma unroll
            for (int i = 0; i < CPL8; ++i) {
                const int c = lane + kWave * i;
                if (c < NC8 && i % split == part) {
                    const uint32_t vv[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
                    uint32_t code[2] = {0u, 0u};
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const uint32_t b = (j & 1) ? (vv[j >> 1] & 0xFFFF0000u) : (vv[j >> 1] << 16);
                        code[j >> 2] |= e4m3_encode(quant_div(__uint_as_float(b), qs)) << (8 * (j & 3));
                    }
                    act[(t * 4 + (c & 3)) * CH + (c >> 2)] = e4m3x8_to_half8(u32x2{code[0], code[1]});
                }
            }
            if (part == 0 && lane == 0) act_sl[t] = qs.s;
        }
    }

    // 1. routing.  One token routed from its logits (ranks): slots are ranks
    //    (slot s < K is the rank-s expert with pair s, slot K the shared
    //    expert with pair K), and wave 0 ranks the logits only up to the slot
    //    of the workgroup's last item (the items are blockIdx.x, + gridDim.x,
    //    ...; their count, (K + shared) * BPE, is known before the routing:
    //    one token's K experts are distinct).  Its ranks reach the other waves
    //    through LDS at the one barrier before the first weight loads.
    //    Workgroup 0 ranks all K and publishes the routing for the down kernel
    //    (and the caller).  Otherwise (caller ids, or 2+ tokens) every
    //    workgroup derives the routing and compaction in LDS (route_prologue,
    //    with its own barriers), and workgroup 0 publishes them.
    const bool ranks = MT == 1 && a.src.logits != nullptr;
    int n_items;
    if (ranks) {
        const int K = a.src.K;
        n_items = (K + a.src.shared) * BPE;
        if (wave == 0) {
            int last = blockIdx.x;
            if (last < n_items) last += ((n_items - 1 - last) / (int)gridDim.x) * (int)gridDim.x;
            const int R = blockIdx.x == 0 ? K : min(last / BPE + 1, K);
            // the threshold pass's LDS: pair_token and pair_src, unused when
            // slots are ranks (576 contiguous bytes, 16-byte aligned)
            static_assert(__builtin_offsetof(RouteLds, pair_src) == __builtin_offsetof(RouteLds, pair_token) + 4 * kMaxPairsExt &&
                          __builtin_offsetof(RouteLds, pair_token) % 16 == 0 && 8 * kMaxPairsExt >= 8 * (kWave + kMaxTopK),
                          "rank scratch");
            const TopkRanks tr = topk_wave_ranks(a.src.logits, a.src.E, R, reinterpret_cast<uint64_t*>(rl.pair_token));
            if (lane < R) rl.ids[lane] = tr.e;
            if (blockIdx.x == 0) publish_rank1(tr, a.src, a.ids_out, a.w_out, a.cp);
        }
    } else {
        route_prologue<MT != 1>(a.src, rl, blockIdx.x == 0);
        if (blockIdx.x == 0) publish_route(rl, a.src, a.ids_out, a.w_out, a.cp);
        n_items = rl.n_act * BPE;
    }
    // the expert of a slot
    auto slot_expert = [&](int slot) -> int {
        if (ranks) return slot < a.src.K ? rl.ids[slot] : kSharedExpert;
        return rl.act_experts[slot];
    };

    // 2. work items (selected expert, block of rows), strided over the grid;
    //    the next item's weight loads are in flight while this one computes.
    //    A row's CH block scales are contiguous bytes.  When LPR and CH are
    //    multiples of 4, the row's LPR lanes load them as dwords (lane li:
    //    dwords li, li + LPR, ...), and the lane that uses block li + LPR i
    //    takes that byte from the lane holding its dword, in dword register
    //    i / 4 (a cross-lane read): NSW dword loads per row instead of CPL
    //    byte loads.  Otherwise each lane loads its CPL scale bytes.
    constexpr bool kScaleDw = LPR % 4 == 0 && CH % 4 == 0;
    constexpr int NSW = kScaleDw ? (CH / 4 + LPR - 1) / LPR : CPL;
    struct Stage {
        u32x4 wg[CPL], wu[CPL];
        uint32_t sg[NSW], su[NSW];
    };
    // The block scales are requested before the weights: the arithmetic reads
    // them first, and with the scales last its first wait covered every load
    // of the item (the load counter is in order), so no block's arithmetic
    // started before the whole item had landed.
    // dummy: the look-ahead past a workgroup's last item.  Its loads are still
    // issued (the waits then stay exact, see below), but every lane reads the
    // first 16 bytes of the item's expert, so each instruction fetches one
    // line instead of the item's rows again (those re-reads were a fifth of
    // the gate/up traffic at four tokens: the loads are non-temporal).
    auto issue = [&](int item, Stage& st, bool dummy = false) {
        const int slot = item / BPE, rb = item % BPE;
        const int e = slot_expert(slot);
        const bool shared = e == kSharedExpert;
        const int r = dummy ? 0 : rb * G::kRowsPerBlock + wave * G::kRowsPerWave + grp;
        const int lo = dummy ? 0 : li;                  // lane's first chunk / scale dword
        const int step = dummy ? 0 : LPR;
        const uint8_t* w13e = shared ? a.sh.w13 : a.w13 + (size_t)e * 2 * I * (H / 2);
        const uint8_t* s13e = shared ? a.sh.s13 : a.s13 + (size_t)e * 2 * I * CH;
        const u32x4* grow = (const u32x4*)(w13e + (size_t)r * (H / 2));
        const u32x4* urow = dummy ? grow : grow + (size_t)I * CH;
        const uint8_t* gsc = s13e + (size_t)r * CH;
        const uint8_t* usc = dummy ? gsc : gsc + (size_t)I * CH;
        if constexpr (kScaleDw) {
#pragma unroll
            for (int j = 0; j < NSW; ++j) {
                const int d = min(lo + step * j, CH / 4 - 1);      // past the row's end: its last dword again
                st.sg[j] = reinterpret_cast<const uint32_t*>(gsc)[d];
                st.su[j] = reinterpret_cast<const uint32_t*>(usc)[d];
            }
        } else {
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                st.sg[i] = gsc[lo + step * i];
                st.su[i] = usc[lo + step * i];
            }
        }
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            st.wg[i] = load_stream(grow + lo + step * i);
            st.wu[i] = load_stream(urow + lo + step * i);
        }
    };
    // the scale code of block li + LPR i of this lane's row
    auto scale_of = [&](const uint32_t* sw, int i) -> uint32_t {
        if constexpr (kScaleDw) {
            const int src = LPR * grp + ((LPR / 4) * i + li / 4) % LPR;
            const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute(src * 4, (int)sw[i / 4]);
            return (v >> (8 * (li & 3))) & 0xFFu;
        } else {
            return sw[i];
        }
    };
    auto compute = [&](int item, Stage& st) {
        const int slot = item / BPE, rb = item % BPE;
        const int r = rb * G::kRowsPerBlock + wave * G::kRowsPerWave + grp;
        const int p0 = ranks ? slot : rl.offsets[slot];
        const int nt = ranks ? 1 : min(rl.offsets[slot + 1] - p0, MT);   // an expert has at most M <= MT tokens
        float accg[MT], accu[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) accg[t] = accu[t] = 0.0f;
        uint32_t scg[CPL], scu[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            scg[i] = scale_of(st.sg, i);
            scu[i] = scale_of(st.su, i);
        }
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = li + LPR * i;
            half2_t hg[16], hu[16];
            e2m1x8_to_half(st.wg[i].x, hg + 0);
            e2m1x8_to_half(st.wg[i].y, hg + 4);
            e2m1x8_to_half(st.wg[i].z, hg + 8);
            e2m1x8_to_half(st.wg[i].w, hg + 12);
            e2m1x8_to_half(st.wu[i].x, hu + 0);
            e2m1x8_to_half(st.wu[i].y, hu + 4);
            e2m1x8_to_half(st.wu[i].z, hu + 8);
            e2m1x8_to_half(st.wu[i].w, hu + 12);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t < nt) {
                    const int tok = ranks ? 0 : rl.pair_token[p0 + t];
                    const u32x4 a0 = act[(tok * 4 + 0) * CH + c], a1 = act[(tok * 4 + 1) * CH + c];
                    const u32x4 a2 = act[(tok * 4 + 2) * CH + c], a3 = act[(tok * 4 + 3) * CH + c];
                    accg[t] += ldexp_e8m0(block_dot(hg, a0, a1, a2, a3), scg[i]);
                    accu[t] += ldexp_e8m0(block_dot(hu, a0, a1, a2, a3), scu[i]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t < nt) {
                accg[t] = group_sum<LPR>(accg[t]);
                accu[t] = group_sum<LPR>(accu[t]);
                const float sc = act_sl[ranks ? 0 : rl.pair_token[p0 + t]];
                const float g = accg[t] * sc, u = accu[t] * sc;
                const int src = ranks ? slot : rl.pair_src[p0 + t];
                if (li == 0) a.h[(size_t)src * I + r] = g / (1.0f + expf(-g)) * u;
            }
        }
    };

    // Items blockIdx.x, blockIdx.x + grid, ...: the next item's loads are
    // issued before the current one is computed.
    constexpr int IPW = ((MT * kMaxTopK + 1) * BPE + 511) / 512;   // most items per workgroup
    // FP8 activations to LDS first (their loads, issued before the routing's,
    // are in: waiting for them after the first item's loads would wait for
    // those too, the load counter being in order).  Then, with ranks, the
    // barrier that hands wave 0's ranks to the other waves and the first
    // item's loads; otherwise (the routing already in LDS) the first item's
    // loads and the barrier that makes the activations visible.
    if (!from_x) {
#pragma unroll
        for (int j = 0; j < NST; ++j) {
            const int idx = threadIdx.x + 256 * j;
            if (idx < n8) {
                const int t = idx / (H / 8), g8 = idx % (H / 8);
                act[(t * 4 + (g8 & 3)) * CH + (g8 >> 2)] = e4m3x8_to_half8(stg[j]);
            }
        }
        if ((int)threadIdx.x < M) act_sl[threadIdx.x] = s_tok;
    }
    const bool has_item = (int)blockIdx.x < n_items;
    Stage st[2];
    if (ranks) {
        __syncthreads();
        if (has_item) issue(blockIdx.x, st[0]);
    } else {
        if (has_item) issue(blockIdx.x, st[0]);
        __syncthreads();
    }
    if (!has_item) return;
    if constexpr (IPW <= 4) {
        // Unrolled over IPW items, with the look-ahead unconditional (past the
        // last item, a dummy issue, unused; none from the IPW-th item, whose
        // successor the loop below loads itself): the two stages are never
        // carried around a loop edge (register copies there would wait for
        // the loads in flight) and each wait covers exactly the item in use.
#pragma unroll
        for (int k = 0; k < IPW; ++k) {
            const int cur = blockIdx.x + k * gridDim.x;
            if (cur >= n_items) break;
            const int nxt = cur + gridDim.x;
            if (k + 1 < IPW) issue(nxt < n_items ? nxt : cur, st[(k + 1) & 1], nxt >= n_items);
            compute(cur, st[k & 1]);
        }
        // beyond IPW items (not reached with the launch geometry): one at a time
        for (int cur = blockIdx.x + IPW * gridDim.x; cur < n_items; cur += gridDim.x) {
            issue(cur, st[0]);
            compute(cur, st[0]);
        }
    } else {
        // more items per workgroup (8 tokens): a loop, whose unrolled form
        // would not fit the instruction cache
        int item = blockIdx.x;
        for (;;) {
            const int next = item + gridDim.x;
            if (next < n_items) issue(next, st[1]);
            compute(item, st[0]);
            if (next >= n_items) break;
            item = next;
            const int after = item + gridDim.x;
            if (after < n_items) issue(after, st[0]);
            compute(item, st[1]);
            if (after >= n_items) break;
            item = after;
        }
    }
}

// ---------------------------------------------------------------------------
// Per-(token, expert) FP8 requantisation of the intermediate, a wave per row
// of I values: s2 = fl32(amax / 448) (1 for an all-zero row), and the codes
// E4M3(h * fl32(1 / s2)).  (The codes may differ from E4M3(h / s2) only where
// h / s2 lies within an ulp of a rounding midpoint.)  Lane l holds the I/64
// consecutive elements starting at l * I/64.
// ---------------------------------------------------------------------------
template <int I>
struct RequantRow {
    static constexpr int PER = I / kWave;
    static_assert(I % kWave == 0, "requantisation needs I % 64 == 0");
    float v[PER];

    __device__ __forceinline__ void load(const float* __restrict__ h, int p)
    {
        const float* row = h + (size_t)p * I + (threadIdx.x & 63) * PER;
        if constexpr (PER % 4 == 0) {
#pragma unroll
            for (int i = 0; i < PER; i += 4) {
                const float4 f = *reinterpret_cast<const float4*>(row + i);
                v[i] = f.x; v[i + 1] = f.y; v[i + 2] = f.z; v[i + 3] = f.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < PER; ++i) v[i] = row[i];
        }
    }
    __device__ __forceinline__ float scale() const
    {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < PER; ++i) m = fmaxf(m, fabsf(v[i]));
        m = wave_max(m);
        return (m == 0.0f) ? 1.0f : m / 448.0f;
    }
    // codes[j] holds elements 4j..4j+3 of this lane (PER % 4 == 0), or one
    // code per entry otherwise
    __device__ __forceinline__ void encode(float sc, uint32_t* codes) const
    {
        const float inv = 1.0f / sc;
        if constexpr (PER % 4 == 0) {
#pragma unroll
            for (int i = 0; i < PER; i += 4)
                codes[i / 4] = e4m3x4_encode(v[i] * inv, v[i + 1] * inv, v[i + 2] * inv, v[i + 3] * inv);
        } else {
#pragma unroll
            for (int i = 0; i < PER; ++i) codes[i] = e4m3_encode(v[i] * inv);
        }
    }
    static constexpr int NCODE = (PER % 4 == 0) ? PER / 4 : PER;
};

template <int I>
__global__ __launch_bounds__(256) void requant_kernel(RequantArgs a)
{
    using R = RequantRow<I>;
    const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (p >= a.P) return;
    const int lane = threadIdx.x & 63;
    R row;
    row.load(a.h, p);
    const float sc = row.scale();
    uint32_t codes[R::NCODE];
    row.encode(sc, codes);
    uint8_t* dst = a.q2 + (size_t)p * I + lane * R::PER;
    if constexpr (R::PER % 4 == 0) {
#pragma unroll
        for (int j = 0; j < R::NCODE; ++j) reinterpret_cast<uint32_t*>(dst)[j] = codes[j];
    } else {
#pragma unroll
        for (int j = 0; j < R::NCODE; ++j) dst[j] = (uint8_t)codes[j];
    }
    if (lane == 0) a.s2[p] = sc;
}

// ---------------------------------------------------------------------------
// Down GEMV + combine.  A workgroup owns RPB output rows for every token; its
// 8 waves split the selected experts (wave w takes slots w, w+8, ...).  Each
// lane accumulates, per token, its share of the row's dot products over the
// wave's slots in slot order; the lanes' sums are then added in a fixed order
// (waves, then the row's lanes).  The FP8 intermediate of every pair is held
// once per workgroup as f16 in LDS.
// ---------------------------------------------------------------------------
template <int H, int I>
struct DownGeom {
    static constexpr int kChunks = I / 32;
    static constexpr int kRowsPerBlock = down_rows_per_block(H, I);
    static constexpr int kPasses = down_row_passes(H, I);
    static constexpr int kRowsPerPass = kRowsPerBlock / kPasses;
    static constexpr int kLanesPerRow = down_lanes_per_row(H, I);
    static constexpr int kChunksPerLane = kChunks / kLanesPerRow;   // per pass
    static constexpr int kLanesUsed = kRowsPerPass * kLanesPerRow;
    static constexpr int kWaves = 8;
    static_assert(I % 32 == 0 && kChunks % kLanesPerRow == 0 && kLanesUsed <= kWave && H % kRowsPerBlock == 0 &&
                  kRowsPerBlock % kPasses == 0, "unsupported down shape");
};

template <int H, int I, int MT, bool FROM_H>
__global__ __launch_bounds__(512) void down_kernel(DownArgs a)
{
    using G = DownGeom<H, I>;
    constexpr int CH = G::kChunks, LPR = G::kLanesPerRow, CPL = G::kChunksPerLane, RPB = G::kRowsPerBlock;
    constexpr int RP = G::kPasses, RPW = G::kRowsPerPass, NW = RP * CPL;   // NW blocks of 32 per lane and slot
    extern __shared__ u32x4 q2h[];    // [pair][q][chunk] of 8 halves; at the end [wave][token][pass][lane] sums
    __shared__ float s2l[kMaxPairsExt];
    __shared__ int32_t c_exp[kMaxPairs + 1], c_off[kMaxPairs + 2], c_src[kMaxPairsExt], c_tok[kMaxPairsExt];
    __shared__ float c_w[kMaxPairsExt];            // router weight of each pair (1 for the shared expert's rows)

    const bool shared = a.sh.w2 != nullptr;
    const int P = a.M * a.K, Pe = P + (shared ? a.M : 0);   // routed pairs, plus the shared expert's rows
    const int n_act = min(*a.cp.n_act, min(a.E, P) + (shared ? 1 : 0));
    // wave-uniform (an SGPR), so that every read of the compaction below is a
    // scalar load: its waits then never hold up the vector loads of h and of
    // the weights, which are counted separately
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    // this lane's row in pass h is n + h * RPW; lanes past RPW * LPR repeat
    // the last row's loads, and their sums are unused
    const int li = lane % LPR, grp = min(lane / LPR, RPW - 1);
    const int n = blockIdx.x * RPB + grp;

    // The compaction, copied to LDS once: its loads go out first, so waiting
    // for them never waits for the h rows or the weights issued after them.
    // All loads below are unconditional (clamped indices), which keeps the
    // count of loads in flight the same on every path.
    const int nc = min(a.E, P) + (shared ? 1 : 0);
    const int tid = threadIdx.x;
    const int32_t ce = a.cp.act_experts[min(tid, nc - 1)];
    const int32_t co = a.cp.offsets[min(tid, nc)];
    const int32_t cs = a.cp.pair_src[min(tid, Pe - 1)];
    const int32_t ct = a.cp.pair_token[min(tid, Pe - 1)];
    const float cw = a.topk_w[min(tid, P - 1)];
    const int last = max(n_act - 1, 0);
    // a slot's loads: a wave-uniform expert base plus this lane's fixed
    // offsets; block j = h * CPL + i is chunk li + LPR i of the pass-h row
    // (24-bit products: a 64-bit multiply-add here takes an unused high half
    // from whatever register, which can be one a load in flight writes)
    const uint32_t woff = __umul24((uint32_t)n, (uint32_t)(I / 2)) + (uint32_t)li * 16;
    const uint32_t soff = __umul24((uint32_t)n, (uint32_t)CH) + (uint32_t)li;
    // The block scales go out before the weights (as in gate/up: the load
    // counter is in order, and the dot products wait for the scales).
    // dummy (the look-ahead past a wave's last slot): the same loads, all at
    // the expert's first 16 bytes (the offsets masked to zero, arithmetic, so
    // the loads stay on one path), one line per instruction instead of the
    // slot's rows again
    auto load_slot = [&](int ea_any, u32x4* wv, uint32_t* sv, bool dummy) {
        const int ea = __builtin_amdgcn_readfirstlane(ea_any);
        const bool sh = shared && ea == kSharedExpert;
        const int e = min(max(ea, 0), a.E - 1);
        const uint8_t* wb = sh ? a.sh.w2 : a.w2 + (size_t)e * H * (I / 2);
        const uint8_t* sb = sh ? a.sh.s2 : a.sw2 + (size_t)e * H * CH;
        const uint32_t keep = 0u - (uint32_t)!dummy;
#pragma unroll
        for (int h = 0; h < RP; ++h)
#pragma unroll
            for (int i = 0; i < CPL; ++i) sv[h * CPL + i] = sb[keep & (soff + (uint32_t)(h * RPW) * CH + LPR * i)];
#pragma unroll
        for (int h = 0; h < RP; ++h)
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                wv[h * CPL + i] = load_stream(reinterpret_cast<const u32x4*>(
                    wb + (keep & (woff + (uint32_t)(h * RPW) * (I / 2) + LPR * 16 * i))));
        __builtin_amdgcn_sched_barrier(0);   // the slot's loads go out here, not next to their uses
    };

    // The intermediate in LDS as f16.  From h: a wave per (token, expert) row
    // requantises it (the same arithmetic as requant_kernel), which every
    // workgroup repeats so that no workgroup waits for another; the rows'
    // loads go out before the weight stream so they are not queued behind it.
    using R = RequantRow<I>;
    constexpr int RB = MT < 4 ? MT : 4;            // rows per wave held at once
    R rows[RB];
    if constexpr (FROM_H) {
#pragma unroll
        for (int j = 0; j < RB; ++j) rows[j].load(a.h, min(wave + G::kWaves * j, Pe - 1));
    }
    // two weight buffers used in turn (no register copies, which would wait
    // for loads in flight): A holds this wave's first slot from here on
    u32x4 wA[NW], wB[NW];
    uint32_t sA[NW], sB[NW];
    // the expert id by a scalar load, its index clamped by a bound from the
    // arguments rather than by the count of active experts (one load fewer
    // before the weights go out; past that count the id is stale but in
    // range, and its slot is never used)
    load_slot(a.cp.act_experts[min(wave, nc - 1)], wA, sA, false);
    if (tid < nc) c_exp[tid] = ce;
    if (tid <= nc) c_off[tid] = co;
    if (tid < Pe) {
        c_src[tid] = cs;
        c_tok[tid] = ct;
        c_w[tid] = tid < P ? cw : 1.0f;
    }

    if constexpr (FROM_H) {
        _Float16* q16 = reinterpret_cast<_Float16*>(q2h);
        const bool tap = blockIdx.x == 0 && a.q2_out != nullptr;
        // a compile-time trip count (at most MT (K + 1) rows) keeps the loop
        // unrolled, so each wait covers exactly the rows it needs
        constexpr int NIT = (MT * (kMaxTopK + 1) + G::kWaves * RB - 1) / (G::kWaves * RB);
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int base = it * G::kWaves * RB;
            if (base >= Pe) break;
            if (base > 0) {
#pragma unroll
                for (int j = 0; j < RB; ++j) rows[j].load(a.h, min(base + wave + G::kWaves * j, Pe - 1));
            }
#pragma unroll
            for (int j = 0; j < RB; ++j) {
                const int p = base + wave + G::kWaves * j;
                if (p >= Pe) break;
                const float sc = rows[j].scale();
                uint32_t codes[R::NCODE];
                rows[j].encode(sc, codes);
                const int k0 = lane * R::PER;
                if constexpr (R::PER % 4 == 0) {
#pragma unroll
                    for (int c4 = 0; c4 < R::NCODE; ++c4) {
                        const int k = k0 + 4 * c4;       // 4 consecutive elements, inside one group of 8
                        uint2 hv2;
                        hv2.x = e4m3x2_to_half2<false>(codes[c4]);
                        hv2.y = e4m3x2_to_half2<true>(codes[c4]);
                        *reinterpret_cast<uint2*>(q16 + ((p * 4 + ((k & 31) >> 3)) * CH + (k >> 5)) * 8 + (k & 7)) = hv2;
                        if (tap) reinterpret_cast<uint32_t*>(a.q2_out + (size_t)p * I + k0)[c4] = codes[c4];
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < R::NCODE; ++i) {
                        const int k = k0 + i;
                        q16[((p * 4 + ((k & 31) >> 3)) * CH + (k >> 5)) * 8 + (k & 7)] = (_Float16)e4m3_decode(codes[i]);
                        if (tap) a.q2_out[(size_t)p * I + k] = (uint8_t)codes[i];
                    }
                }
                if (lane == 0) {
                    s2l[p] = sc;
                    if (tap && a.s2_out != nullptr) a.s2_out[p] = sc;
                }
            }
        }
    } else {
        constexpr int NST = (MT * 8 * (I / 8) + 511) / 512;
        const int n8 = P * (I / 8);
        u32x2 stg[NST];
#pragma unroll
        for (int j = 0; j < NST; ++j) stg[j] = ((const u32x2*)a.q2)[min((int)threadIdx.x + 512 * j, n8 - 1)];
#pragma unroll
        for (int j = 0; j < NST; ++j) {
            const int idx = threadIdx.x + 512 * j;
            if (idx < n8) {
                const int p = idx / (I / 8), g8 = idx % (I / 8);
                q2h[(p * 4 + (g8 & 3)) * CH + (g8 >> 2)] = e4m3x8_to_half8(stg[j]);
            }
        }
        for (int p = threadIdx.x; p < P; p += blockDim.x) s2l[p] = a.s2[p];
    }
    __syncthreads();

    float acc[RP][MT];
#pragma unroll
    for (int h = 0; h < RP; ++h)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[h][t] = 0.0f;
    auto consume = [&](int slot, const u32x4* wv, const uint32_t* sv) {
        half2_t hw[NW * 16];
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            e2m1x8_to_half(wv[j].x, hw + 16 * j + 0);
            e2m1x8_to_half(wv[j].y, hw + 16 * j + 4);
            e2m1x8_to_half(wv[j].z, hw + 16 * j + 8);
            e2m1x8_to_half(wv[j].w, hw + 16 * j + 12);
        }
        const int q0 = min(max(c_off[slot], 0), Pe), q1 = min(c_off[slot + 1], Pe);
        for (int qq = q0; qq < q1; ++qq) {
            const int p = min(max(c_src[qq], 0), Pe - 1);
            const int tok = c_tok[qq];
            float d[RP];
#pragma unroll
            for (int h = 0; h < RP; ++h) d[h] = 0.0f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                // the pair's chunk c serves this lane's row of every pass
                const int c = li + LPR * i;
                const u32x4 a0 = q2h[(p * 4 + 0) * CH + c], a1 = q2h[(p * 4 + 1) * CH + c];
                const u32x4 a2 = q2h[(p * 4 + 2) * CH + c], a3 = q2h[(p * 4 + 3) * CH + c];
#pragma unroll
                for (int h = 0; h < RP; ++h)
                    d[h] += ldexp_e8m0(block_dot(hw + 16 * (h * CPL + i), a0, a1, a2, a3), sv[h * CPL + i]);
            }
            const float coef = c_w[p] * s2l[p];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const float ct = (t == tok) ? coef : 0.0f;    // a select, not an indexed store
#pragma unroll
                for (int h = 0; h < RP; ++h) acc[h][t] = fmaf(ct, d[h], acc[h][t]);
            }
        }
    };
    // slots wave, wave + 8, ...: the next slot's weights load while this one
    // is used (past the end, a dummy load of one line, unused).
    // The loop is unrolled over the most slots a wave can have, so each step
    // is straight-line code whose waits cover exactly the slot in use.
    constexpr int NS = (MT * (kMaxTopK + 1) + G::kWaves - 1) / G::kWaves;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        const int slot = wave + G::kWaves * k;
        if (slot >= n_act) break;
        const bool past = slot + G::kWaves >= n_act;
        const int next = past ? slot : slot + G::kWaves;
        if (k % 2 == 0) {
            load_slot(c_exp[next], wB, sB, past);
            consume(slot, wA, sA);
        } else {
            load_slot(c_exp[next], wA, sA, past);
            consume(slot, wB, sB);
        }
    }
    // the lanes' sums go to the intermediate's LDS once every wave is past
    // its last read of it
    __syncthreads();
    float* red = reinterpret_cast<float*>(q2h);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int h = 0; h < RP; ++h) red[((wave * MT + t) * RP + h) * kWave + lane] = acc[h][t];
    __syncthreads();
    for (int idx = threadIdx.x; idx < RPB * a.M; idx += blockDim.x) {
        const int row = idx % RPB, t = idx / RPB;
        const int h = row / RPW, rr = row % RPW;
        float s = 0.0f;
        for (int w = 0; w < G::kWaves; ++w) {
#pragma unroll
            for (int j = 0; j < LPR; ++j) s += red[((w * MT + t) * RP + h) * kWave + rr * LPR + j];
        }
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

}  // namespace moe
