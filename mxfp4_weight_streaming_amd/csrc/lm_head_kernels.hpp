// lm_head_kernels.hpp -- the FP8 LM head on gfx950: load-time quantisation of
// the bf16 output projection to E4M3 with one fp32 scale per vocabulary row,
// and the decode GEMV that streams the FP8 rows.  Device code only, compiled
// ahead of time through lm_head.hip and at run time by hipRTC.
//
// The pages name the LM head (hidden 2,560 -> vocabulary 157,184, stored in
// BF16) as the second memory-bound hotspot of batch-1 decode: every token
// reads all of it, and quantising it to FP8 once at load time halves those
// reads ([EN] "What are the 3 optimizations?", item 2).  The row scale is the
// activation scheme applied to weight rows (amax/448); the activations stay
// bf16.  E4M3 values are exact in bf16 (8 exponent bits, 3 of 7 mantissa bits
// used), so each FP8 pair is decoded to a bf16 pair and multiplied with
// v_dot2c_f32_bf16 into fp32.
//   [EN] = "NVIDIA Shows 3 Ways to Speed Up MoE Inference on DGX Spark,
//          Lifting Ling-3.0-flash Throughput 42.5%"
#pragma once

#include "device_common.hpp"
#include "moe_types.hpp"

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Quantisation: one wave per row; s = amax / 448 (1 for an all-zero row),
// codes E4M3(w / s), both divisions correctly rounded binary32 divisions.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lm_head_quant_kernel(const uint16_t* __restrict__ w, int V, int H,
                                                            uint8_t* __restrict__ q, float* __restrict__ scale)
{
    const int v = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (v >= V) return;                                 // whole wave; no barrier follows
    const u32x4* row = reinterpret_cast<const u32x4*>(w + (size_t)v * H);
    const int nch = H / 8;                              // 16-byte chunks of 8 bf16
    float m = 0.0f;
    for (int c = lane; c < nch; c += kWave) {
        const u32x4 d = row[c];
        const uint32_t u[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            m = fmaxf(m, fmaxf(fabsf(__uint_as_float(u[j] << 16)), fabsf(__uint_as_float(u[j] & 0xFFFF0000u))));
    }
    const float amax = wave_max(m);
    const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
    u32x2* qrow = reinterpret_cast<u32x2*>(q + (size_t)v * H);
    for (int c = lane; c < nch; c += kWave) {
        const u32x4 d = row[c];
        const uint32_t u[4] = {d.x, d.y, d.z, d.w};
        uint32_t b[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            b[2 * j] = e4m3_encode(__uint_as_float(u[j] << 16) / s);
            b[2 * j + 1] = e4m3_encode(__uint_as_float(u[j] & 0xFFFF0000u) / s);
        }
        qrow[c] = u32x2{b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
    }
    if (lane == 0) scale[v] = s;
}

// ---------------------------------------------------------------------------
// GEMV: logits[t, v] = s_v * sum_k E4M3(q[v, k]) * x[t, k].  16 lanes share a
// row, each lane taking 16-code chunks li, li + 16, ... (one load instruction
// of the group covers 256 contiguous bytes); a wave holds 4 rows and a
// workgroup 16.  Workgroups stride over row blocks with the next block's
// loads in flight while the current one computes.  The activations are staged
// once per workgroup in LDS as bf16.
// ---------------------------------------------------------------------------
// Two E4M3 codes (bytes HI*2, HI*2+1 of `codes`) as a bf16 pair (exact).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t codes)
{
    const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, HI);
    return __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
}

__device__ __forceinline__ float dot_bf16x2(uint32_t a, uint32_t b, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}

// Row blocks per unrolled round of the GEMV loop (even: the stage a round's
// last look-ahead fills is the one its next round starts on).  Inside a round
// the two stages are never carried around a loop edge; a rolled loop did carry
// them, and the compiler then waited for every load in flight at its head, so
// each workgroup had one block in flight instead of two.
__host__ __device__ constexpr int lm_head_blocks_per_round(int mt) { return mt <= 4 ? 8 : 4; }

// (The compiler unrolls each round of the loop below, NB bodies with exact
// waits, yet reports a loop transformation it did not perform; that warning
// is silenced for this kernel.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wpass-failed"
template <int H, int MT>
__global__ __launch_bounds__(256) void lm_head_gemv_kernel(const uint16_t* __restrict__ x, int M,
                                                           const uint8_t* __restrict__ q,
                                                           const float* __restrict__ scale, int V,
                                                           float* __restrict__ logits)
{
    constexpr int LPR = 16, CPL = H / 16 / LPR;        // 16-code chunks per lane
    constexpr int NB = lm_head_blocks_per_round(MT);
    static_assert(NB % 2 == 0, "a round ends on the stage the next one starts with");
    static_assert(H % (16 * LPR) == 0, "LM-head GEMV needs H % 256 == 0");
    __shared__ u32x4 xs[MT * H / 8];                    // [token][8-element group] of bf16
    for (int i = threadIdx.x; i < M * H / 8; i += 256) xs[i] = reinterpret_cast<const u32x4*>(x)[i];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane % LPR, grp = lane / LPR;
    const int blocks = (V + 15) / 16;
    struct Stage {
        u32x4 w[CPL];
        float sc;                                       // the row's scale, loaded with its codes
    };
    // dummy: the look-ahead past the workgroup's last block.  Its loads are
    // still issued, so that every wait covers exactly the block in use, but
    // all at the first 16 bytes of the head (one line per instruction).
    auto load = [&](int blk, Stage& st, bool dummy) {
        const int v = dummy ? 0 : min(blk * 16 + wave * 4 + grp, V - 1);
        const u32x4* row = reinterpret_cast<const u32x4*>(q + (size_t)v * H);
        const int lo = dummy ? 0 : li, step = dummy ? 0 : LPR;
#pragma unroll
        for (int i = 0; i < CPL; ++i) st.w[i] = load_stream(row + lo + step * i);
        st.sc = scale[v];
    };
    const int blk0 = blockIdx.x;
    if (blk0 >= blocks) return;
    Stage st[2];
    load(blk0, st[0], false);
    __syncthreads();                                    // activations staged
    auto compute = [&](int b, const Stage& sg) {
        float acc[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = li + LPR * i;                 // 16 codes = elements 16c .. 16c+15
            const uint32_t d[4] = {sg.w[i].x, sg.w[i].y, sg.w[i].z, sg.w[i].w};
            uint32_t wb[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                wb[2 * j] = e4m3x2_to_bf16x2<false>(d[j]);
                wb[2 * j + 1] = e4m3x2_to_bf16x2<true>(d[j]);
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t < M) {
                    const u32x4 x0 = xs[t * (H / 8) + 2 * c], x1 = xs[t * (H / 8) + 2 * c + 1];
                    float s = acc[t];
                    s = dot_bf16x2(wb[0], x0.x, s);
                    s = dot_bf16x2(wb[1], x0.y, s);
                    s = dot_bf16x2(wb[2], x0.z, s);
                    s = dot_bf16x2(wb[3], x0.w, s);
                    s = dot_bf16x2(wb[4], x1.x, s);
                    s = dot_bf16x2(wb[5], x1.y, s);
                    s = dot_bf16x2(wb[6], x1.z, s);
                    s = dot_bf16x2(wb[7], x1.w, s);
                    acc[t] = s;
                }
            }
        }
        const int v = b * 16 + wave * 4 + grp;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t < M) {
                const float sum = group_sum<LPR>(acc[t]);
                if (li == 0 && v < V) logits[(size_t)t * V + v] = sum * sg.sc;
            }
        }
    };
    // blocks blk0, blk0 + grid, ...: the next block's loads are issued before
    // the current one is computed (past the last, a dummy issue, unused)
    int cur = blk0;
    for (;;) {
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            if (cur >= blocks) return;
            const int nxt = cur + (int)gridDim.x;
            load(nxt < blocks ? nxt : cur, st[(k + 1) & 1], nxt >= blocks);
            compute(cur, st[k & 1]);
            cur = nxt;
        }
    }
}
#pragma clang diagnostic pop

}  // namespace moe
