// chunk_kernels.hpp -- gfx950 kernels of the MoE layer for chunks of 9..2048
// tokens (a prefill chunk, or a large verify batch); device code only,
// compiled ahead of time through moe_chunk.hip and at run time by hipRTC.
//
// At these token counts every expert is picked by several tokens, so the
// expert layers are grouped contractions: per active expert e, the FP8 rows of
// its tokens times the MXFP4 weights of e.  They run on the scaled FP4xFP8
// matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4): the E8M0 block scales of
// the weights enter the instruction directly, the per-token fp32 activation
// and intermediate scales are applied in the epilogues, and the router weight
// in the combine.  The
// pages profile MoE decode as bound by reading expert weights ([EN] "Why is
// MoE decoding on DGX Spark memory-bound?"); here too each weight byte is read
// from HBM once per chunk record, by the wave that owns its 16 rows (an expert
// has one record, or several of up to 256 rows when more rows picked it).
//
// A chunk is seven kernels on one stream:
//   chunk_router_kernel   bf16 MFMA router GEMM, fp32 logits
//   chunk_topk_kernel     one wave per token: top-K and renormalised weights,
//                         and the token's per-token FP8 activations (for
//                         H > 4096 those come from quant_kernel, run before)
//   sort_pairs_kernel     one workgroup: token bitmasks per expert in LDS,
//                         ranks by popcount (a bitonic sort when a token names
//                         an expert twice) -> active experts, per-expert
//                         offsets, pair lists, chunk records
//   chunk_gate_up_kernel  per (expert, 32 intermediate rows): gate and up
//                         tiles on MFMA, K split over the workgroup's waves,
//                         SiLU(gate)*up epilogue -> h fp32
//   requant_kernel        per (token, expert) FP8 requantisation of h
//   chunk_down_kernel     per (expert, 256 output rows): down tiles on MFMA,
//                         epilogue scales by s2 -> y
//   combine_kernel        out[t] = sum over the token's K pairs of w * y, in
//                         selection order (no float atomics)
//
// Operand layouts of the 16x16x128 scaled MFMA (lane l, r = l % 16,
// g = l / 16), established by direct tests on gfx950:
//   FP8 operand: row r; bytes 0..15 hold K = 16g..16g+15 and bytes 16..31
//                hold K = 64+16g..64+16g+15.
//   FP4 operand: row r; the 32 nibbles of dwords 0..3 hold K = 32g..32g+31,
//                low nibble first (the MX byte order).
//   Scales:      lane l supplies the E8M0 code of row r, K block g.
//   Result:      lane l holds C[4g + i][r], i = 0..3.
// bf16 16x16x32 MFMA: row r holds K = 8g..8g+7 of each operand; same result
// layout.
//   [EN] = "NVIDIA Shows 3 Ways to Speed Up MoE Inference on DGX Spark,
//          Lifting Ling-3.0-flash Throughput 42.5%"
#pragma once

#include <type_traits>
#include <utility>

#include "device_common.hpp"
#include "moe_types.hpp"
#include "topk_wave.hpp"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 (compile-time loop
// index, for operands that must be constants).
template <int N, typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>)
{
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// The unit E8M0 scale code (127) of the FP8 operand, in a VGPR.  The scale
// operands of v_mfma_scale take VGPRs; one compiler release (the hipRTC that
// ships with PyTorch's ROCm 7.0 libraries) encodes a constant code there as an
// SGPR, which the instruction reads as something else, so the code is
// materialised in a VGPR explicitly.
__device__ __forceinline__ int unit_scale_vgpr()
{
    int v;
    asm("v_mov_b32 %0, 127" : "=v"(v));
    return v;
}

// C += A(FP8, unit scale) * B(FP4, E8M0 scale code sb)
__device__ __forceinline__ f32x4 mfma_fp8_fp4(i32x8 a, i32x8 b, f32x4 c, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, unit_scale_vgpr(), 0, sb);
}

// The same with the B scale code taken from byte SEL of a packed register.
template <int SEL>
__device__ __forceinline__ f32x4 mfma_fp8_fp4_sel(i32x8 a, i32x8 b, f32x4 c, int packed)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, unit_scale_vgpr(), SEL, packed);
}

// Scale code q of a lane, packed four per register, applied with op_sel.
template <int Q>
__device__ __forceinline__ f32x4 mfma_packed_scale(i32x8 a, i32x8 b, f32x4 c, const int* packed)
{
    return mfma_fp8_fp4_sel<Q % 4>(a, b, c, packed[Q / 4]);
}

__device__ __forceinline__ i32x8 fp8_operand(u32x4 lo, u32x4 hi)
{
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__device__ __forceinline__ i32x8 fp4_operand(u32x4 v)
{
    return i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

// ---------------------------------------------------------------------------
// Router: logits[t, e] = sum_k x[t, k] * Wr[e, k] on bf16 MFMA with fp32
// accumulation.  One workgroup per 16x16 (token, expert) tile; its 8 waves
// take K slices of H/8 with every load issued up front, and the slices are
// added in LDS in wave order.
// ---------------------------------------------------------------------------
template <int H>
__global__ __launch_bounds__(kRouterWaves * kWave) void chunk_router_kernel(ChunkRouterArgs a)
{
    constexpr int KW = H / kRouterWaves;                 // K slice of a wave
    constexpr int NS = KW / 32;                          // MFMA steps per slice
    static_assert(H % (kRouterWaves * 32) == 0, "router slice must be a whole number of MFMA steps");
    __shared__ float red[kRouterWaves][4][kWave];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int tiles_e = a.E >> 4;
    const int tm = blockIdx.x / tiles_e, te = blockIdx.x - tm * tiles_e;
    const int m = min(tm * 16 + r, a.M - 1);            // ragged tail: repeat the last token
    const uint16_t* xr = a.x + (size_t)m * H + w * KW + 8 * g;
    const uint16_t* wr = a.wr + (size_t)(te * 16 + r) * H + w * KW + 8 * g;
    bf16x8 av[NS], bv[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        av[q] = *reinterpret_cast<const bf16x8*>(xr + 32 * q);
        bv[q] = *reinterpret_cast<const bf16x8*>(wr + 32 * q);
    }
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < NS; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[q], bv[q], acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) red[w][i][lane] = acc[i];
    __syncthreads();
    if (threadIdx.x < 256) {                             // thread (i, l): C[4 (l >> 4) + i][l & 15]
        const int l = threadIdx.x & 63, i = threadIdx.x >> 6;
        float v = red[0][i][l];
#pragma unroll
        for (int u = 1; u < kRouterWaves; ++u) v += red[u][i][l];
        const int row = tm * 16 + 4 * (l >> 4) + i;
        if (row < a.M) a.logits[(size_t)row * a.E + te * 16 + (l & 15)] = v;
    }
}

// ---------------------------------------------------------------------------
// Top-K and weights, one wave per token; with act_q, the token's FP8
// activations too.  The token's logits are requested first and its
// activations next, so the activations arrive during the top-K rounds; the
// keys are waited for before the dispatch on E (topk_keys8), the activations
// only where they are used (the top-K is inlined here: a call would wait for
// every load in flight).  The quantisation is quant_kernel's: s = amax / 448
// over the token's row (one wave holds the whole row; a maximum is exact in
// any order), codes E4M3(x / s) with the correctly rounded quotient.
// ---------------------------------------------------------------------------
constexpr int kTopkQuantChunks = kTopkQuantMaxH / 8 / kWave;   // 16-byte chunks of a row per lane

template <int PER, bool QUANT>
__device__ __forceinline__ void topk_quant_token(const ChunkTopkArgs& a, int t, const TopkKeys8& k,
                                                 const u32x4 (&xv)[kTopkQuantChunks])
{
    constexpr int NQ = kTopkQuantChunks;
    const int lane = threadIdx.x & 63;
    uint32_t u[PER];
    int sl[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        u[i] = k.u[i];
        sl[i] = i;
    }
    const int nc8 = a.H / 8;
    topk_select_t<PER>(u, sl, a.K, a.ids + (size_t)t * a.K, a.w + (size_t)t * a.K, a.K);
    if constexpr (!QUANT) return;
    auto bf = [](uint32_t v, int hi) { return __uint_as_float(hi ? (v & 0xFFFF0000u) : (v << 16)); };
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        if (lane + kWave * i < nc8) {
            const uint32_t vv[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(bf(vv[j >> 1], j & 1)));
        }
    }
    const QuantScale qs = quant_scale(wave_max(m));
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int c = lane + kWave * i;
        if (c < nc8) {
            const uint32_t vv[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
            uint32_t code[2] = {0u, 0u};
#pragma unroll
            for (int j = 0; j < 8; ++j) code[j >> 2] |= e4m3_encode(quant_div(bf(vv[j >> 1], j & 1), qs)) << (8 * (j & 3));
            *reinterpret_cast<u32x2*>(a.act_q + (size_t)t * a.H + 8 * c) = u32x2{code[0], code[1]};
        }
    }
    if (lane == 0) a.act_s[t] = qs.s;
}

template <bool QUANT>
__global__ __launch_bounds__(256) void chunk_topk_kernel(ChunkTopkArgs a)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.M) return;                              // whole wave; no barrier follows
    const int lane = threadIdx.x & 63;
    const TopkLogits8 lg = topk_load_logits8(a.logits + (size_t)t * a.E, a.E);
    u32x4 xv[kTopkQuantChunks];
    if constexpr (QUANT) {
        __builtin_amdgcn_sched_barrier(0);              // the logits first: the top-K waits only for them
        const int nc8 = a.H / 8;
        const u32x4* xr = reinterpret_cast<const u32x4*>(a.x + (size_t)t * a.H);
#pragma unroll
        for (int i = 0; i < kTopkQuantChunks; ++i) xv[i] = xr[min(lane + kWave * i, nc8 - 1)];   // clamped: no branch
    }
    const TopkKeys8 k = topk_keys8(lg, a.E);
    if (a.E <= 64) topk_quant_token<1, QUANT>(a, t, k, xv);
    else if (a.E <= 128) topk_quant_token<2, QUANT>(a, t, k, xv);
    else if (a.E <= 256) topk_quant_token<4, QUANT>(a, t, k, xv);
    else topk_quant_token<8, QUANT>(a, t, k, xv);
}

// ---------------------------------------------------------------------------
// Expert-major ordering of the M*K (token, slot) pairs by one workgroup.  The
// pairs of an expert end up contiguous and in (token, slot) order (the decode
// path's compaction order); active experts get slots in ascending id.  Each
// expert gets an M-bit token mask in LDS; when no token names an expert twice
// (always so for routed ids) the masks' popcounts are the expert counts and a
// pair's rank inside its expert is a popcount of the mask below its token.
// A token naming an expert more than once shows as a popcount total below
// M*K; such ids take exact counts and a bitonic sort of (expert << 16 | pair)
// keys.  The rows of every slot are then cut into chunk records for the
// grouped kernels: a busy expert's (more than kChunkRows rows) first, cut
// evenly into records of at most kBigChunkRows rows, then the others as one
// record each, 4-tile records before 3-, 2- and 1-tile ones.
// ---------------------------------------------------------------------------
constexpr int kSortThreads = 1024;
constexpr int kSortPairsPerThread = kMaxChunkPairs / kSortThreads;

// Inclusive prefix sum over the wave on DPP: shifts by 1, 2, 4 and 8 within
// rows of 16 lanes, then each row adds the totals of the rows before it.
__device__ __forceinline__ int wave_incl_scan(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xA, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xC, 0xF, false);
    return v;
}

// Exclusive prefix sum of one value per thread over the workgroup, in thread
// order; every thread must call it.  Values may pack several counters in
// separate bit fields, as long as no field's total overflows it.
__device__ int block_excl_scan(int v, int* tmp, int& total)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int x = wave_incl_scan(v);
    if (lane == kWave - 1) tmp[w] = x;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kSortThreads / kWave; ++i) {
        const int t = tmp[i];
        base += (i < w) ? t : 0;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return base + x - v;
}

__global__ __launch_bounds__(kSortThreads) void sort_pairs_kernel(SortArgs a)
{
    extern __shared__ uint32_t sh[];                     // token masks, or sort keys
    __shared__ int32_t cnt[kMaxExperts];
    __shared__ int32_t pre[kMaxExperts];
    __shared__ int32_t tmp[kSortThreads / kWave];
    // W mask words per expert, stored WS = W | 1 words apart: an odd stride
    // puts the same word of different experts' masks (read together by the
    // threads of a wave) on different LDS banks
    const int P = a.M * a.K, K = a.K, E = a.E, W = (a.M + 31) >> 5, WS = W | 1;
    const int tid = threadIdx.x;
    auto clamp_e = [&](int e) { return e < 0 ? 0 : (e >= E ? E - 1 : e); };
    // every pair's expert, loaded once (all loads first)
    int eid[kSortPairsPerThread];
#pragma unroll
    for (int i = 0; i < kSortPairsPerThread; ++i) {
        const int p = tid + kSortThreads * i;
        eid[i] = clamp_e(a.ids[p < P ? p : P - 1]);
    }
    for (int i = tid; i < E * WS; i += kSortThreads) sh[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSortPairsPerThread; ++i) {
        const int p = tid + kSortThreads * i;
        if (p < P) {
            const int t = p / K;
            atomicOr(&sh[eid[i] * WS + (t >> 5)], 1u << (t & 31));
        }
    }
    __syncthreads();
    // per expert (thread e < E; thread E stands for the shared expert, whose M
    // rows follow the routed pairs in one more slot): its count, and with it
    // whether it is active; one scan gives offsets (low 16 bits) and slots
    int c = 0;
    if (tid < E)
        for (int w = 0; w < W; ++w) c += __popc(sh[tid * WS + w]);
    const bool virt = a.shared != 0 && tid == E;
    const int extra = a.shared != 0 ? a.M : 0;
    int total = 0;
    int cc = (tid < E) ? c : (virt ? a.M : 0);
    int packed = block_excl_scan(((cc > 0 ? 1 : 0) << 16) | cc, tmp, total);
    const bool dup = (total & 0xFFFF) - extra != P;      // uniform: some token names an expert twice
    if (dup) {
        // exact counts (the masks hold each (token, expert) once)
        for (int e = tid; e < kMaxExperts; e += kSortThreads) cnt[e] = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kSortPairsPerThread; ++i)
            if (tid + kSortThreads * i < P) atomicAdd(&cnt[eid[i]], 1);
        __syncthreads();
        cc = (tid < E) ? cnt[tid] : (virt ? a.M : 0);
        packed = block_excl_scan(((cc > 0 ? 1 : 0) << 16) | cc, tmp, total);
    }
    const int off_e = packed & 0xFFFF, slot_e = packed >> 16;
    const int total_pairs = total & 0xFFFF, n_act = total >> 16;
    const int rec_e = virt ? kSharedExpert : tid;
    if (tid < E) pre[tid] = off_e;
    if (cc > 0) {
        a.cp.act_experts[slot_e] = rec_e;
        a.cp.offsets[slot_e] = off_e;
    }
    if (tid == 0) {
        *a.cp.n_act = n_act;
        a.cp.offsets[n_act] = total_pairs;
    }
    if (a.shared != 0) {
        for (int t = tid; t < a.M; t += kSortThreads) {
            a.cp.pair_token[P + t] = t;
            a.cp.pair_src[P + t] = P + t;
            a.pos_of[P + t] = P + t;
        }
    }
    __syncthreads();
    if (!dup) {
#pragma unroll
        for (int i = 0; i < kSortPairsPerThread; ++i) {
            const int p = tid + kSortThreads * i;
            if (p < P) {
                const int t = p / K;
                const uint32_t* mrow = sh + eid[i] * WS;
                int rank = __popc(mrow[t >> 5] & ((1u << (t & 31)) - 1u));
                for (int w = 0; w < (t >> 5); ++w) rank += __popc(mrow[w]);
                const int pos = pre[eid[i]] + rank;
                a.cp.pair_token[pos] = t;
                a.cp.pair_src[pos] = p;
                a.pos_of[p] = pos;
            }
        }
    } else {
        int NP = 64;
        while (NP < P) NP <<= 1;
        for (int i = tid; i < NP; i += kSortThreads)
            sh[i] = (i < P) ? (((uint32_t)clamp_e(a.ids[i]) << 16) | (uint32_t)i) : 0xFFFFFFFFu;
        __syncthreads();
        for (int size = 2; size <= NP; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = tid; i < NP / 2; i += kSortThreads) {
                    const int lo = 2 * i - (i & (stride - 1));
                    const int hi = lo + stride;
                    const bool ascending = (lo & size) == 0;
                    const uint32_t x = sh[lo], y = sh[hi];
                    if ((x > y) == ascending) {
                        sh[lo] = y;
                        sh[hi] = x;
                    }
                }
                __syncthreads();
            }
        }
        for (int pos = tid; pos < P; pos += kSortThreads) {
            const int p = (int)(sh[pos] & 0xFFFFu);
            a.cp.pair_token[pos] = p / K;
            a.cp.pair_src[pos] = p;
            a.pos_of[p] = pos;
        }
    }
    // chunk list, from the expert's own thread (its count cc and slot_e): a
    // busy expert's (more than kChunkRows rows) chunks first, cut evenly into
    // at most kBigChunkRows rows each; then the others in the group of their
    // tile count, 4 tiles down to 1; two scans, packing the group counters
    // (the big chunks in 16 bits, the tile groups in 10-bit fields: at most
    // kMaxExperts + 1 experts each)
    const bool big = cc > kChunkRows;
    const int nbig = big ? (cc + kBigChunkRows - 1) / kBigChunkRows : 0;
    const int tiles = (!big && cc > 0) ? (cc + 15) / 16 : 0;
    int tb4 = 0, t321 = 0;
    const int sb4 = block_excl_scan((nbig << 16) | (tiles == 4 ? 1 : 0), tmp, tb4);
    const int s321 = block_excl_scan(((tiles == 3 ? 1 : 0) << 20) | ((tiles == 2 ? 1 : 0) << 10) | (tiles == 1 ? 1 : 0),
                                     tmp, t321);
    const int atb = sb4 >> 16, at4 = sb4 & 0xFFFF;
    const int at3 = s321 >> 20, at2 = (s321 >> 10) & 0x3FF, at1 = s321 & 0x3FF;
    const int nb = tb4 >> 16, n4 = tb4 & 0xFFFF, n3 = t321 >> 20, n2 = (t321 >> 10) & 0x3FF, n1 = t321 & 0x3FF;
    if (big) {
        const int q = (cc + nbig - 1) / nbig;           // rows per chunk; the last takes the rest
        for (int k = 0; k < nbig; ++k) {
            const int rows = cc - k * q;
            a.chunks.rec[atb + k] = make_int4(rec_e, off_e + k * q, rows < q ? rows : q, 0);
        }
    } else if (tiles > 0) {
        const int idx = nb + (tiles == 4 ? at4 : tiles == 3 ? n4 + at3 : tiles == 2 ? n4 + n3 + at2 : n4 + n3 + n2 + at1);
        a.chunks.rec[idx] = make_int4(rec_e, off_e, cc, 0);
    }
    const int n_chunks = nb + n4 + n3 + n2 + n1;
    for (int i = n_chunks + tid; i < a.chunks.C; i += kSortThreads) a.chunks.rec[i] = make_int4(0, 0, 0, 0);
    if (tid == 0) *a.chunks.n_chunks = n_chunks;
}

// ---------------------------------------------------------------------------
// Gate/up: workgroup (chunk, jq) owns the kGuRows = 16 NJ intermediate rows
// j = kGuRows jq .. +kGuRows-1 of the chunk's expert, for both the gate (rows j)
// and the up (rows I + j) projection, over the chunk's tokens (at most
// kBigChunkRows).
// Its waves split K = H into KSPLIT slices: each wave issues all the weight
// loads of its slice at once (NJ n-tiles of gate and of up, so one activation
// operand feeds 2 NJ MFMAs), after the chunk's token ids and before the first
// tile's activations; the block scales of the workgroup's rows are read with
// full-width loads into LDS.  The 16-token tiles then run with the next
// tile's activations loading while the current one is reduced; the slices'
// partial sums are added in LDS in a fixed wave order, where SiLU(g)*u and
// the per-token activation scale are applied.
// ---------------------------------------------------------------------------
template <int H>
struct ChunkSplit {
    static constexpr int KS = chunk_k_steps(H);         // 128-deep k-steps
    static constexpr int KSPLIT = chunk_k_split(H);     // waves with a K slice
    static constexpr int KQ = KS / KSPLIT;              // k-steps per slice
    static_assert(H % 128 == 0 && KS % KSPLIT == 0, "unsupported H for the chunk gate/up");
};

template <int H, int I>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void chunk_gate_up_kernel(
    ChunkGateUpArgs a)
{
    using G = ChunkSplit<H>;
    constexpr int KQ = G::KQ, NJ = kGuNJ, SROW = H / 32;
    static_assert(I % kGuRows == 0 && (kGuRows * SROW) % 16 == 0, "chunk gate/up row blocking");
    __shared__ float red[4][NJ][2][4][kWave];            // [wave][n-tile][gate/up][i][lane]
    __shared__ uint8_t sc_lds[2][kGuRows * SROW] __attribute__((aligned(16)));   // [gate/up][row][block]
    __shared__ float tok_scale[16];
    const int jq = blockIdx.x % (I / kGuRows);
    const int4 rec = a.chunks.rec[blockIdx.x / (I / kGuRows)];
    const int e = rec.x, off = rec.y, n = rec.z;
    if (n == 0) return;                                 // whole workgroup: past the last chunk
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const bool has_k = w < G::KSPLIT;
    const int ks0 = (has_k ? w : 0) * KQ;
    const int j0 = jq * kGuRows;
    const uint8_t* w13e = e == kSharedExpert ? a.sh.w13 : a.w13 + (size_t)e * 2 * I * (H / 2);
    // The wave's K slice of a row is BPR 16-byte blocks (one E8M0 block each).
    // Load i of lane l fetches block 64 i + l of an n-tile's 16 x BPR blocks in
    // row-major order, so each row's slice arrives as one contiguous run (the
    // operand layout itself would read 64 bytes from each of 16 rows per
    // load, a slower pattern on HBM).  Group t < NJ is gate n-tile t, group
    // NJ + t is up n-tile t.
    constexpr int BPR = 4 * KQ, RSTR = BPR + 1;         // blocks per slice row; LDS row stride in blocks
    __shared__ u32x4 xpose[4][16 * RSTR];               // per wave: one n-tile being rearranged
    // Token ids come first, since the first tile's activations need them:
    // this lane's row of the first tile, and row threadIdx.x of the record
    // for the table the later tiles read from LDS (a record has at most
    // kBigChunkRows rows, one per thread; rows past the record repeat its
    // last row).  The vector-memory counter is in issue order, so the loads
    // are issued in the order they are waited for: ids, weights, the first
    // tile's activations, block scales.
    static_assert(kBigChunkRows == 256, "one token id per thread of the workgroup");
    __shared__ int tok_lds[kBigChunkRows];
    auto tok_at = [&](int row) { return a.cp.pair_token[off + (row < n ? row : n - 1)]; };
    const int tok0 = tok_at(r);
    const int my_tok = tok_at(threadIdx.x);
    u32x4 raw[2 * NJ][KQ];
#pragma unroll
    for (int t = 0; t < 2 * NJ; ++t) {
        const uint8_t* nt = w13e + (size_t)((t < NJ ? 0 : I) + j0 + 16 * (t % NJ)) * (H / 2) + ks0 * 64;
#pragma unroll
        for (int i = 0; i < KQ; ++i) {
            const int b = i * 64 + lane;
            raw[t][i] = load_stream(reinterpret_cast<const u32x4*>(nt + (size_t)(b / BPR) * (H / 2) + (b % BPR) * 16));
        }
    }
    __builtin_amdgcn_sched_barrier(0);                  // every weight load before the wait for tok0
    u32x4 alo[KQ], ahi[KQ];
    float s_row = 0.0f;
    auto load_tile = [&](int t) {
        s_row = a.act_s[t];                             // first: in by the time the codes are
        const uint8_t* ar = a.act_q + (size_t)t * H + ks0 * 128 + 16 * g;
#pragma unroll
        for (int q = 0; q < KQ; ++q) {
            alo[q] = *reinterpret_cast<const u32x4*>(ar + q * 128);
            ahi[q] = *reinterpret_cast<const u32x4*>(ar + q * 128 + 64);
        }
    };
    load_tile(tok0);
    // the block scales of the workgroup's gate and up rows: NSC 16-byte loads
    // per thread and matrix, stored to LDS after the weights are in
    constexpr int SCH = kGuRows * SROW / 16, NSC = (SCH + 255) / 256;
    const uint8_t* s13e = e == kSharedExpert ? a.sh.s13 : a.s13 + (size_t)e * 2 * I * SROW;
    u32x4 scg[NSC], scu[NSC];
#pragma unroll
    for (int i = 0; i < NSC; ++i) {
        const int c = threadIdx.x + 256 * i, ci = c < SCH ? c : SCH - 1;
        scg[i] = *reinterpret_cast<const u32x4*>(s13e + (size_t)j0 * SROW + 16 * ci);
        scu[i] = *reinterpret_cast<const u32x4*>(s13e + (size_t)(I + j0) * SROW + 16 * ci);
    }
    tok_lds[threadIdx.x] = my_tok;
    // into the operand layout through the wave's LDS area: lane (r, g) of
    // k-step q takes block 4 q + g of row r (the row stride of BPR + 1 blocks
    // keeps the 16 rows of one read on distinct banks)
    i32x8 bg[NJ][KQ], bu[NJ][KQ];
    u32x4* xw = xpose[w];
#pragma unroll
    for (int t = 0; t < 2 * NJ; ++t) {
#pragma unroll
        for (int i = 0; i < KQ; ++i) {
            const int b = i * 64 + lane;
            xw[(b / BPR) * RSTR + b % BPR] = raw[t][i];
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = 0; q < KQ; ++q) {
            const i32x8 v = fp4_operand(xw[r * RSTR + 4 * q + g]);
            if (t < NJ) bg[t][q] = v;
            else bu[t - NJ][q] = v;
        }
        __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int i = 0; i < NSC; ++i) {
        const int c = threadIdx.x + 256 * i;
        if (c < SCH) {
            reinterpret_cast<u32x4*>(sc_lds[0])[c] = scg[i];
            reinterpret_cast<u32x4*>(sc_lds[1])[c] = scu[i];
        }
    }
    lds_barrier();                                      // block scales and token ids in LDS
    constexpr int NP = (KQ + 3) / 4;                    // packed scale registers per n-tile
    int sg[NJ][NP], su[NJ][NP];
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
#pragma unroll
        for (int u = 0; u < NP; ++u) sg[nj][u] = su[nj][u] = 0;
#pragma unroll
        for (int q = 0; q < KQ; ++q) {
            const int idx = (16 * nj + r) * SROW + (ks0 + q) * 4 + g;
            sg[nj][q / 4] |= (int)sc_lds[0][idx] << (8 * (q % 4));
            su[nj][q / 4] |= (int)sc_lds[1][idx] << (8 * (q % 4));
        }
    }
    const int ntiles = (n + 15) / 16;
    for (int tile = 0; tile < ntiles; ++tile) {
        f32x4 accg[NJ], accu[NJ];
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) {
            accg[nj] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            accu[nj] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        static_for<KQ>([&](auto qc) {
            constexpr int q = decltype(qc)::value;
            const i32x8 av = fp8_operand(alo[q], ahi[q]);
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj) {
                accg[nj] = mfma_packed_scale<q>(av, bg[nj][q], accg[nj], sg[nj]);
                accu[nj] = mfma_packed_scale<q>(av, bu[nj][q], accu[nj], su[nj]);
            }
        });
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                red[w][nj][0][i][lane] = has_k ? accg[nj][i] : 0.0f;
                red[w][nj][1][i][lane] = has_k ? accu[nj][i] : 0.0f;
            }
        }
        if (w == 0 && g == 0) tok_scale[r] = s_row;
        // the next tile's activations, in flight while this tile is reduced
        if (tile + 1 < ntiles) load_tile(tok_lds[(tile + 1) * 16 + r]);
        lds_barrier();                                  // the loads and stores in flight stay so
        // thread (ii, l) finalises C[4 (l >> 4) + ii][l & 15] of each n-tile.
        // A row past the record ran on row n - 1's token (tok_of), so its
        // value is row n - 1's, bit for bit, and is stored there: the stores
        // are then unconditional, and the next tile's wait for its operands
        // counts them exactly instead of waiting for every store in flight.
        const int l = threadIdx.x & 63, ii = threadIdx.x >> 6;
        const int trow = 4 * (l >> 4) + ii;
        const int row = tile * 16 + trow;
        const int srow = row < n ? row : n - 1;
        const float sc = tok_scale[trow];
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) {
            float gs = red[0][nj][0][ii][l], us = red[0][nj][1][ii][l];
#pragma unroll
            for (int v = 1; v < G::KSPLIT; ++v) {
                gs += red[v][nj][0][ii][l];
                us += red[v][nj][1][ii][l];
            }
            const float gv = gs * sc, uv = us * sc;
            a.h[(size_t)(off + srow) * I + j0 + 16 * nj + (l & 15)] = gv / (1.0f + expf(-gv)) * uv;
        }
        lds_barrier();
    }
}

// ---------------------------------------------------------------------------
// Down: workgroup (chunk, nq) owns output rows [kDnRows nq, kDnRows (nq + 1))
// of the chunk's expert; wave w holds the down weights of its NJ 16-row
// n-tiles (all of K = I) in registers, the block scales come through LDS, and
// the chunk's token tiles run through them, every activation load of a tile
// issued before its MFMAs (one activation operand feeds NJ MFMAs) and the
// next tile's loads in flight while the current tile is stored.
// y[pos, n] = s2 * acc (the router weight is applied by the combine).
// ---------------------------------------------------------------------------
template <int H, int I, bool BY_PAIR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 8))) void chunk_down_kernel(
    ChunkDownArgs a)
{
    static_assert(H % kDnRows == 0 && I % 32 == 0, "chunk down row blocking");
    constexpr int KS = (I + 127) / 128, NJ = kDnNJ, SROW = I / 32;
    constexpr int SBYTES = kDnRows * SROW;
    __shared__ uint8_t sc_lds[(SBYTES + 15) / 16 * 16] __attribute__((aligned(16)));
    const int nq = blockIdx.x % (H / kDnRows);
    const int4 rec = a.chunks.rec[blockIdx.x / (H / kDnRows)];
    const int e = rec.x, off = rec.y, n = rec.z;
    if (n == 0) return;                                 // whole workgroup: past the last chunk
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int n0 = nq * kDnRows;
    const uint8_t* w2e = e == kSharedExpert ? a.sh.w2 : a.w2 + (size_t)e * H * (I / 2);
    const uint8_t* sw2e = e == kSharedExpert ? a.sh.s2 : a.sw2 + (size_t)e * H * SROW;
    // The intermediate row of record row `row` (rows past the record repeat
    // its last row): its position, or by pair its source pair, which comes
    // from memory; the later tiles read those from a table in LDS (a record
    // has at most kBigChunkRows rows, one per thread).  The vector-memory
    // counter is in issue order, so the loads are issued in the order they
    // are waited for: (by pair) the first tile's rows, weights, the first
    // tile's activations, block scales.
    static_assert(kBigChunkRows == 256, "one source row per thread of the workgroup");
    __shared__ int src_lds[BY_PAIR ? kBigChunkRows : 1];
    auto src_at = [&](int row) {
        const int pos = off + (row < n ? row : n - 1);
        return BY_PAIR ? a.cp.pair_src[pos] : pos;
    };
    auto src_row = [&](int row) {                       // rows below kBigChunkRows
        if constexpr (BY_PAIR) return src_lds[row];
        else return off + (row < n ? row : n - 1);
    };
    int arow0 = src_at(r), erow0[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) erow0[i] = src_at(4 * g + i);
    const int my_src = BY_PAIR ? src_at(threadIdx.x) : 0;
    // A row is BPR 16-byte blocks (one E8M0 block each) and an n-tile's 16
    // rows are one contiguous run of 16 BPR blocks: load i of lane l fetches
    // block 64 i + l of it (the gate/up kernel's scheme; the operand layout
    // would read 64 bytes from each of 16 rows per load).
    constexpr int BPR = I / 32, NBLK = 16 * BPR, NLD = (NBLK + 63) / 64, RSTR = BPR + 1;
    __shared__ u32x4 xpose[4][16 * RSTR];               // per wave: one n-tile being rearranged
    u32x4 raw[NJ][NLD];
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
        const uint8_t* nt = w2e + (size_t)(n0 + (w * NJ + nj) * 16) * (I / 2);
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int b = i * 64 + lane;
            raw[nj][i] = load_stream(reinterpret_cast<const u32x4*>(nt + (size_t)(b < NBLK ? b : NBLK - 1) * 16));
        }
    }
    __builtin_amdgcn_sched_barrier(0);                  // every weight load before the first wait
    u32x4 alo[KS], ahi[KS];
    float es[4];                                          // s2 of the rows this lane stores
    auto load_tile = [&](int arow, const int (&erow)[4]) {
        const uint8_t* q = a.q2 + (size_t)arow * I + 16 * g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (I % 128 == 0) {
                alo[ks] = *reinterpret_cast<const u32x4*>(q + ks * 128);
                ahi[ks] = *reinterpret_cast<const u32x4*>(q + ks * 128 + 64);
            } else {
                const bool lo_in = ks * 128 + 16 * g + 16 <= I, hi_in = ks * 128 + 64 + 16 * g + 16 <= I;
                alo[ks] = lo_in ? *reinterpret_cast<const u32x4*>(q + (lo_in ? ks * 128 : 0)) : u32x4{0u, 0u, 0u, 0u};
                ahi[ks] = hi_in ? *reinterpret_cast<const u32x4*>(q + (hi_in ? ks * 128 + 64 : 0))
                                : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) es[i] = a.s2[erow[i]];
    };
    load_tile(arow0, erow0);
    // the block scales of the workgroup's rows: NSC 16-byte loads per thread,
    // stored to LDS after the weights are in
    static_assert(SBYTES % 16 == 0, "block scales in 16-byte loads");
    constexpr int SCH = SBYTES / 16, NSC = (SCH + 255) / 256;
    u32x4 scv[NSC];
#pragma unroll
    for (int i = 0; i < NSC; ++i) {
        const int c = threadIdx.x + 256 * i;
        scv[i] = *reinterpret_cast<const u32x4*>(sw2e + (size_t)n0 * SROW + 16 * (c < SCH ? c : SCH - 1));
    }
    if constexpr (BY_PAIR) src_lds[threadIdx.x] = my_src;
    // into the operand layout through the wave's LDS area: lane (r, g) of
    // k-step ks takes block 4 ks + g of row r, zero codes past the row
    i32x8 b[NJ][KS];
    u32x4* xw = xpose[w];
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int bi = i * 64 + lane;
            if (NBLK % 64 == 0 || bi < NBLK) xw[(bi / BPR) * RSTR + bi % BPR] = raw[nj][i];
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int blk = 4 * ks + g;
            if constexpr (I % 128 == 0) {
                b[nj][ks] = fp4_operand(xw[r * RSTR + blk]);
            } else {                                      // K padded with zero codes
                const u32x4 v = xw[r * RSTR + (blk < BPR ? blk : 0)];
                b[nj][ks] = blk < BPR ? fp4_operand(v) : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int i = 0; i < NSC; ++i) {
        const int c = threadIdx.x + 256 * i;
        if (c < SCH) reinterpret_cast<u32x4*>(sc_lds)[c] = scv[i];
    }
    lds_barrier();                                        // block scales (and source rows) in LDS
    constexpr int NP = (KS + 3) / 4;                    // packed scale registers per n-tile
    int sc[NJ][NP];
#pragma unroll
    for (int nj = 0; nj < NJ; ++nj) {
#pragma unroll
        for (int u = 0; u < NP; ++u) sc[nj][u] = 0;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int kb = ks * 128 + 32 * g;
            const int code = (kb < I) ? sc_lds[((w * NJ + nj) * 16 + r) * SROW + (kb < I ? kb / 32 : 0)] : 127;
            sc[nj][ks / 4] |= code << (8 * (ks % 4));
        }
    }
    for (int base = 0; base < n; base += 16) {
        f32x4 acc[NJ];
#pragma unroll
        for (int nj = 0; nj < NJ; ++nj) acc[nj] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        static_for<KS>([&](auto kc) {
            constexpr int ks = decltype(kc)::value;
            const i32x8 av = fp8_operand(alo[ks], ahi[ks]);
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj) acc[nj] = mfma_packed_scale<ks>(av, b[nj][ks], acc[nj], sc[nj]);
        });
        float esc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) esc[i] = es[i];
        if (base + 16 < n) {
            int erow[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) erow[i] = src_row(base + 16 + 4 * g + i);
            load_tile(src_row(base + 16 + r), erow);
        }
        // A row past the record ran on row n - 1's activations and scale, so
        // its value is row n - 1's, bit for bit, and is stored there: the
        // stores are then unconditional, and the next tile's wait for its
        // operands counts them exactly instead of waiting for every store.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row2 = base + 4 * g + i;
            float* yr = a.y + (size_t)(off + (row2 < n ? row2 : n - 1)) * H + n0 + w * NJ * 16 + r;
#pragma unroll
            for (int nj = 0; nj < NJ; ++nj) yr[16 * nj] = acc[nj][i] * esc[i];
        }
    }
}

// ---------------------------------------------------------------------------
// Combine: out[t, :] = sum_{j < K} w[t, j] * y[pos_of[t K + j], :], added in
// j order, then (with a shared expert) + y[pos_of[M K + t], :].
// ---------------------------------------------------------------------------
template <int H>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a)
{
    constexpr int Q = H / 4;
    const int total = a.M * Q;
    for (int idx = blockIdx.x * 256 + threadIdx.x; idx < total; idx += gridDim.x * 256) {
        const int t = idx / Q, c = (idx - t * Q) * 4;
        float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        for (int j = 0; j < a.K; ++j) {
            const int pos = a.pos_of[t * a.K + j];
            const float wj = a.w[t * a.K + j];
            const float4 v = *reinterpret_cast<const float4*>(a.y + (size_t)pos * H + c);
            s.x += wj * v.x; s.y += wj * v.y; s.z += wj * v.z; s.w += wj * v.w;
        }
        if (a.shared != 0) {
            const float4 v = *reinterpret_cast<const float4*>(a.y + (size_t)a.pos_of[a.M * a.K + t] * H + c);
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
        *reinterpret_cast<float4*>(a.out + (size_t)t * H + c) = s;
    }
}

// dst row p = src row pos_of[p] (rows of `words` 32-bit words): turns
// sorted-order intermediates into pair order for the caller's taps.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                                                          const int32_t* __restrict__ pos_of, int P, int words)
{
    const int64_t total = (int64_t)P * words;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
        const int p = (int)(idx / words), w = (int)(idx - (int64_t)p * words);
        dst[idx] = src[(int64_t)pos_of[p] * words + w];
    }
}

}  // namespace moe
