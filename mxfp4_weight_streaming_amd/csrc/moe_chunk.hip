// moe_chunk.hip -- gfx950 kernels of the MoE layer for chunks of 9..2048
// tokens (a prefill chunk, or a large verify batch).
//
// At these token counts every expert is picked by several tokens, so the
// expert layers are grouped contractions: per active expert e, the FP8 rows of
// its tokens times the MXFP4 weights of e.  They run on the scaled FP4xFP8
// matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4): the E8M0 block scales of
// the weights enter the instruction directly, and the per-token fp32
// activation scale (and the router weight) are applied in the epilogue.  The
// pages profile MoE decode as bound by reading expert weights ([EN] "Why is
// MoE decoding on DGX Spark memory-bound?"); here too each weight byte is read
// from HBM once per call, by the wave that owns its 16 rows.
//
// A chunk is eight kernels on one stream:
//   chunk_router_kernel   bf16 MFMA router GEMM, fp32 logits
//   quant_kernel          per-token FP8 activations (shared with the decode path)
//   chunk_topk_kernel     one wave per token: top-K and renormalised weights
//   sort_pairs_kernel     one workgroup: (expert, pair) bitonic sort in LDS ->
//                         active experts, per-expert offsets, pair lists
//   chunk_gate_up_kernel  per (expert, 64 intermediate rows): gate and up
//                         tiles on MFMA, SiLU(gate)*up epilogue -> h fp32
//   requant_kernel        per (token, expert) FP8 requantisation of h
//   chunk_down_kernel     per (expert, 64 output rows): down tiles on MFMA,
//                         epilogue scales by s2 and the router weight -> y
//   combine_kernel        out[t] = sum over the token's K pairs of y, in
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
#include <hip/hip_ext.h>

#include "device_common.hpp"
#include "moe_internal.hpp"
#include "topk_wave.hpp"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// C += A(FP8, unit scale) * B(FP4, E8M0 scale code sb)
__device__ __forceinline__ f32x4 mfma_fp8_fp4(i32x8 a, i32x8 b, f32x4 c, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, 127, 0, sb);
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
// accumulation.  One wave per 16x16 (token, expert) tile.
// ---------------------------------------------------------------------------
template <int H>
__global__ __launch_bounds__(256) void chunk_router_kernel(ChunkRouterArgs a)
{
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int tiles_e = a.E >> 4;
    const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int tm = wv / tiles_e, te = wv - tm * tiles_e;
    if (tm * 16 >= a.M) return;                        // whole wave; no barrier follows
    const int m = min(tm * 16 + r, a.M - 1);           // ragged tail: repeat the last token
    const uint16_t* xr = a.x + (size_t)m * H + 8 * g;
    const uint16_t* wr = a.wr + (size_t)(te * 16 + r) * H + 8 * g;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
    for (int k0 = 0; k0 < H; k0 += 32) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(xr + k0);
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(wr + k0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = tm * 16 + 4 * g + i;
        if (row < a.M) a.logits[(size_t)row * a.E + te * 16 + r] = acc[i];
    }
}

// ---------------------------------------------------------------------------
// Top-K and weights, one wave per token.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void chunk_topk_kernel(ChunkTopkArgs a)
{
    __shared__ TopkScratch sc[4];
    const int w = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + w;
    if (t >= a.M) return;                              // whole wave; only wave-level syncs follow
    topk_wave(a.logits + (size_t)t * a.E, a.E, a.K, a.ids + (size_t)t * a.K, a.w + (size_t)t * a.K, sc[w]);
}

// ---------------------------------------------------------------------------
// Expert-major ordering of the M*K (token, slot) pairs, by one workgroup:
// keys (expert << 16 | pair) are bitonic-sorted in LDS, so the pairs of an
// expert are contiguous and in ascending token order, the same order as the
// decode path's compaction.  Active experts get slots in ascending id.
// ---------------------------------------------------------------------------
constexpr int kSortThreads = 1024;

__global__ __launch_bounds__(kSortThreads) void sort_pairs_kernel(SortArgs a)
{
    __shared__ uint32_t keys[kMaxChunkPairs];
    __shared__ int32_t slot_of[kMaxExperts];
    __shared__ int32_t wave_total[kSortThreads / kWave];
    const int P = a.M * a.K;
    int NP = 64;
    while (NP < P) NP <<= 1;
    for (int i = threadIdx.x; i < NP; i += kSortThreads) {
        uint32_t k = 0xFFFFFFFFu;                      // padding sorts last
        if (i < P) {
            int e = a.ids[i];
            e = e < 0 ? 0 : (e >= a.E ? a.E - 1 : e);
            k = ((uint32_t)e << 16) | (uint32_t)i;
        }
        keys[i] = k;
    }
    for (int e = threadIdx.x; e < kMaxExperts; e += kSortThreads) slot_of[e] = 0;
    __syncthreads();
    for (int size = 2; size <= NP; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < NP / 2; i += kSortThreads) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool ascending = (lo & size) == 0;
                const uint32_t x = keys[lo], y = keys[hi];
                if ((x > y) == ascending) {
                    keys[lo] = y;
                    keys[hi] = x;
                }
            }
            __syncthreads();
        }
    }
    // mark the experts present, then number them in ascending id
    for (int pos = threadIdx.x; pos < P; pos += kSortThreads) {
        const uint32_t e = keys[pos] >> 16;
        if (pos == 0 || (keys[pos - 1] >> 16) != e) slot_of[e] = 1;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int present = (threadIdx.x < a.E) ? slot_of[threadIdx.x] : 0;
    const uint64_t ball = __ballot(present);
    const int before = __popcll(ball & ((1ull << lane) - 1ull));
    if (lane == 0) wave_total[wv] = __popcll(ball);
    __syncthreads();
    int base = 0, total = 0;
    for (int w = 0; w < kSortThreads / kWave; ++w) {
        base += (w < wv) ? wave_total[w] : 0;
        total += wave_total[w];
    }
    if (threadIdx.x < a.E) slot_of[threadIdx.x] = present ? base + before : -1;
    __syncthreads();
    if (threadIdx.x == 0) {
        *a.cp.n_act = total;
        a.cp.offsets[total] = P;
    }
    for (int pos = threadIdx.x; pos < P; pos += kSortThreads) {
        const uint32_t key = keys[pos];
        const int e = (int)(key >> 16), p = (int)(key & 0xFFFFu);
        a.cp.pair_token[pos] = p / a.K;
        a.cp.pair_src[pos] = p;
        a.pos_of[p] = pos;
        if (pos == 0 || (keys[pos - 1] >> 16) != (uint32_t)e) {
            const int s = slot_of[e];
            a.cp.act_experts[s] = e;
            a.cp.offsets[s] = pos;
        }
    }
}

// ---------------------------------------------------------------------------
// Gate/up: workgroup (slot, jq) owns intermediate rows [64 jq, 64 jq + 64) of
// the slot's expert; wave w owns the 16 rows j0 = 64 jq + 16 w .. +15 of both
// the gate (rows j) and the up (rows I + j) projection, so SiLU(g)*u is formed
// in registers.  The expert's tokens are taken in passes of up to 8 tiles of
// 16: the weights stream once per pass (once in total for up to 128 tokens).
// ---------------------------------------------------------------------------
template <int H, int I, int NT>
__device__ __forceinline__ void chunk_gate_up_pass(const ChunkGateUpArgs& a, int e, int off, int n, int base)
{
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int j = (blockIdx.x % (I / 64)) * 64 + (threadIdx.x >> 6) * 16 + r;   // this lane's weight row
    int tok[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        const int row = base + tt * 16 + r;
        tok[tt] = a.cp.pair_token[off + (row < n ? row : n - 1)];
    }
    const uint8_t* wg = a.w13 + ((size_t)e * 2 * I + j) * (H / 2) + 16 * g;
    const uint8_t* wu = wg + (size_t)I * (H / 2);
    const uint8_t* sg = a.s13 + ((size_t)e * 2 * I + j) * (H / 32) + g;
    const uint8_t* su = sg + (size_t)I * (H / 32);
    f32x4 accg[NT], accu[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        accg[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        accu[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll 2
    for (int ks = 0; ks < H / 128; ++ks) {
        const i32x8 bg = fp4_operand(load_stream(reinterpret_cast<const u32x4*>(wg + ks * 64)));
        const i32x8 bu = fp4_operand(load_stream(reinterpret_cast<const u32x4*>(wu + ks * 64)));
        const int scg = sg[ks * 4], scu = su[ks * 4];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const uint8_t* ar = a.act_q + (size_t)tok[tt] * H + ks * 128 + 16 * g;
            const i32x8 av = fp8_operand(*reinterpret_cast<const u32x4*>(ar), *reinterpret_cast<const u32x4*>(ar + 64));
            accg[tt] = mfma_fp8_fp4(av, bg, accg[tt], scg);
            accu[tt] = mfma_fp8_fp4(av, bu, accu[tt], scu);
        }
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = base + tt * 16 + 4 * g + i;
            if (row < n) {
                const int pos = off + row;
                const float s = a.act_s[a.cp.pair_token[pos]];
                const float gv = accg[tt][i] * s, uv = accu[tt][i] * s;
                a.h[(size_t)pos * I + j] = gv / (1.0f + expf(-gv)) * uv;
            }
        }
    }
}

template <int H, int I>
__global__ __launch_bounds__(256) void chunk_gate_up_kernel(ChunkGateUpArgs a)
{
    static_assert(H % 128 == 0 && I % 64 == 0, "chunk gate/up needs H % 128 == 0 and I % 64 == 0");
    const int slot = blockIdx.x / (I / 64);
    if (slot >= *a.cp.n_act) return;
    const int e = a.cp.act_experts[slot];
    const int off = a.cp.offsets[slot];
    const int n = a.cp.offsets[slot + 1] - off;
    for (int base = 0; base < n; base += 128) {
        const int rem = n - base;
        if (rem > 64) chunk_gate_up_pass<H, I, 8>(a, e, off, n, base);
        else if (rem > 32) chunk_gate_up_pass<H, I, 4>(a, e, off, n, base);
        else if (rem > 16) chunk_gate_up_pass<H, I, 2>(a, e, off, n, base);
        else chunk_gate_up_pass<H, I, 1>(a, e, off, n, base);
    }
}

// ---------------------------------------------------------------------------
// Down: workgroup (slot, nq) owns output rows [64 nq, 64 nq + 64) of the
// slot's expert; wave w holds the down weights of its 16 rows (all of K = I)
// in registers and runs the expert's token tiles through them.  The epilogue
// writes y[pos, n] = w_pair * s2_pair * acc, one row per pair.
// ---------------------------------------------------------------------------
template <int H, int I>
__global__ __launch_bounds__(256) void chunk_down_kernel(ChunkDownArgs a)
{
    static_assert(H % 64 == 0 && I % 32 == 0, "chunk down needs H % 64 == 0");
    constexpr int KS = (I + 127) / 128;
    const int slot = blockIdx.x / (H / 64);
    if (slot >= *a.cp.n_act) return;
    const int e = a.cp.act_experts[slot];
    const int off = a.cp.offsets[slot];
    const int n = a.cp.offsets[slot + 1] - off;
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    const int nrow = (blockIdx.x % (H / 64)) * 64 + (threadIdx.x >> 6) * 16 + r;
    const uint8_t* wrow = a.w2 + ((size_t)e * H + nrow) * (I / 2);
    const uint8_t* srow = a.sw2 + ((size_t)e * H + nrow) * (I / 32);
    i32x8 b[KS];
    int sc[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int kb = ks * 128 + 32 * g;                 // first K of this lane's block
        if constexpr (I % 128 == 0) {
            b[ks] = fp4_operand(load_stream(reinterpret_cast<const u32x4*>(wrow + kb / 2)));
            sc[ks] = srow[kb / 32];
        } else {                                          // K padded with zero codes
            const bool in = kb < I;
            b[ks] = in ? fp4_operand(load_stream(reinterpret_cast<const u32x4*>(wrow + (in ? kb / 2 : 0))))
                       : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
            sc[ks] = in ? srow[in ? kb / 32 : 0] : 127;
        }
    }
    for (int base = 0; base < n; base += 16) {
        const int row = base + r;
        const int pos = off + (row < n ? row : n - 1);
        const int arow = a.by_pair ? a.cp.pair_src[pos] : pos;
        const uint8_t* q = a.q2 + (size_t)arow * I + 16 * g;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 lo, hi;
            if constexpr (I % 128 == 0) {
                lo = *reinterpret_cast<const u32x4*>(q + ks * 128);
                hi = *reinterpret_cast<const u32x4*>(q + ks * 128 + 64);
            } else {
                const bool lo_in = ks * 128 + 16 * g + 16 <= I, hi_in = ks * 128 + 64 + 16 * g + 16 <= I;
                lo = lo_in ? *reinterpret_cast<const u32x4*>(q + (lo_in ? ks * 128 : 0)) : u32x4{0u, 0u, 0u, 0u};
                hi = hi_in ? *reinterpret_cast<const u32x4*>(q + (hi_in ? ks * 128 + 64 : 0)) : u32x4{0u, 0u, 0u, 0u};
            }
            acc = mfma_fp8_fp4(fp8_operand(lo, hi), b[ks], acc, sc[ks]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row2 = base + 4 * g + i;
            if (row2 < n) {
                const int pos2 = off + row2;
                const int src = a.cp.pair_src[pos2];
                const float scale = a.s2[a.by_pair ? src : pos2] * a.topk_w[src];
                a.y[(size_t)pos2 * H + nrow] = acc[i] * scale;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Combine: out[t, :] = sum_{j < K} y[pos_of[t K + j], :], added in j order.
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
            const float4 v = *reinterpret_cast<const float4*>(a.y + (size_t)pos * H + c);
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

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
template <typename F, typename... Args>
static void launch(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s, const LaunchEvents& ev, Args... args)
{
    if (ev.start != nullptr || ev.stop != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, block, lds, s, ev.start, ev.stop, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

bool chunk_shape_supported(int H, int I, int E)
{
    return ((H == 256 && I == 64) || (H == 2560 && I == 768)) && E % 16 == 0;
}

hipError_t launch_chunk_router(int H, const ChunkRouterArgs& a, hipStream_t s, const LaunchEvents& ev)
{
    const int waves = ((a.M + 15) / 16) * (a.E / 16);
    const dim3 grid((waves + 3) / 4);
    if (H == 256) launch(chunk_router_kernel<256>, grid, dim3(256), 0, s, ev, a);
    else if (H == 2560) launch(chunk_router_kernel<2560>, grid, dim3(256), 0, s, ev, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_chunk_topk(const ChunkTopkArgs& a, hipStream_t s, const LaunchEvents& ev)
{
    launch(chunk_topk_kernel, dim3((a.M + 3) / 4), dim3(256), 0, s, ev, a);
    return hipGetLastError();
}

hipError_t launch_sort_pairs(const SortArgs& a, hipStream_t s, const LaunchEvents& ev)
{
    if (a.M * a.K > kMaxChunkPairs || a.E > kMaxExperts) return hipErrorInvalidValue;
    launch(sort_pairs_kernel, dim3(1), dim3(kSortThreads), 0, s, ev, a);
    return hipGetLastError();
}

hipError_t launch_chunk_gate_up(int H, int I, int S, const ChunkGateUpArgs& a, hipStream_t s, const LaunchEvents& ev)
{
    const dim3 grid((unsigned)(S * (I / 64)));
    if (H == 256 && I == 64) launch(chunk_gate_up_kernel<256, 64>, grid, dim3(256), 0, s, ev, a);
    else if (H == 2560 && I == 768) launch(chunk_gate_up_kernel<2560, 768>, grid, dim3(256), 0, s, ev, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_chunk_down(int H, int I, int S, const ChunkDownArgs& a, hipStream_t s, const LaunchEvents& ev)
{
    const dim3 grid((unsigned)(S * (H / 64)));
    if (H == 256 && I == 64) launch(chunk_down_kernel<256, 64>, grid, dim3(256), 0, s, ev, a);
    else if (H == 2560 && I == 768) launch(chunk_down_kernel<2560, 768>, grid, dim3(256), 0, s, ev, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_combine(int H, const CombineArgs& a, hipStream_t s, const LaunchEvents& ev)
{
    const int total = a.M * (H / 4);
    const int blocks = (total + 255) / 256;
    const dim3 grid((unsigned)(blocks < 2048 ? blocks : 2048));
    if (H == 256) launch(combine_kernel<256>, grid, dim3(256), 0, s, ev, a);
    else if (H == 2560) launch(combine_kernel<2560>, grid, dim3(256), 0, s, ev, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_gather_rows(const void* src, void* dst, const int32_t* pos_of, int P, int row_bytes, hipStream_t s)
{
    if (P <= 0 || row_bytes <= 0) return hipSuccess;
    if (row_bytes % 4 != 0) return hipErrorInvalidValue;
    const int words = row_bytes / 4;
    const int64_t total = (int64_t)P * words;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s,
                       static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), pos_of, P, words);
    return hipGetLastError();
}

const char* chunk_kernel_names(int H, int I)
{
    if (H == 2560 && I == 768)
        return "chunk_router_kernel<H=2560> (bf16 MFMA 16x16x32) -> quant_kernel<2560> -> chunk_topk_kernel -> "
               "sort_pairs_kernel (1 workgroup, bitonic in LDS) -> chunk_gate_up_kernel<2560,768> (scaled FP8xFP4 "
               "MFMA 16x16x128, 12 workgroups/expert) -> requant_kernel<768> -> chunk_down_kernel<2560,768> "
               "(scaled FP8xFP4 MFMA, 40 workgroups/expert) -> combine_kernel<2560>";
    if (H == 256 && I == 64)
        return "chunk_router_kernel<H=256> -> quant_kernel<256> -> chunk_topk_kernel -> sort_pairs_kernel -> "
               "chunk_gate_up_kernel<256,64> -> requant_kernel<64> -> chunk_down_kernel<256,64> -> combine_kernel<256>";
    return "unsupported";
}

}  // namespace moe
