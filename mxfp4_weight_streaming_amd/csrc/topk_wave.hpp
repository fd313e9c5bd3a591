// topk_wave.hpp -- top-K routing of one token by one wave (gfx950), shared by
// the decode kernels and the chunk kernels.
//
// The pages route each token to 8 experts ([EN] "What is Ling 3.0, and why
// does it suit DGX Spark?"); the selection is the K largest logits with equal
// logits going to the lower expert index, and the weights are the softmax
// over the selected logits (equal to the full softmax renormalised over the
// selection).
//   [EN] = "NVIDIA Shows 3 Ways to Speed Up MoE Inference on DGX Spark,
//          Lifting Ling-3.0-flash Throughput 42.5%"
#pragma once

#include "device_common.hpp"
#include "moe_internal.hpp"

namespace moe {

// Orderable key of a float: unsigned comparison of keys is float comparison.
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

// Per-wave LDS scratch of the top-K: the selected keys in ascending expert order.
struct TopkScratch {
    uint32_t u[kMaxTopK];
    int32_t e[kMaxTopK];
};

__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Top-K of one token's E logits by one wave, as a radix select: 32 steps of
// ballot counting find T, the K-th largest orderable logit; the selection is
// every logit above T plus, among those equal to T, the lowest expert
// indices.  The K winners are then ranked by (logit descending, index
// ascending) and their weights are the softmax over the selected logits.
template <int PER>
__device__ void topk_wave_t(const float* L, int E, int K, int32_t* ids_out, float* w_out, TopkScratch& sc)
{
    const int lane = threadIdx.x & 63;
    uint32_t u[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {             // unconditional loads: all in flight together
        const int e = lane + kWave * i;
        const float v = L[e < E ? e : E - 1];
        u[i] = (e < E) ? f32_orderable(v + 0.0f) : 0u;   // + 0.0f folds -0 into +0
    }
    // Radix select of T, the largest value with count(u >= T) >= K.  As soon
    // as some candidate has exactly K keys at or above it, those K keys are
    // the selection (every other key is strictly smaller) and the search stops.
    uint32_t T = 0;
    bool exact = false;
    for (int b = 31; b >= 0; --b) {
        const uint32_t cand = T | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) cnt += __popcll(__ballot(u[i] >= cand));
        if (cnt >= K) {
            T = cand;
            if (cnt == K) {
                exact = true;
                break;
            }
        }
    }
    uint64_t sel[PER];
    if (exact) {
#pragma unroll
        for (int i = 0; i < PER; ++i) sel[i] = __ballot(u[i] >= T);
    } else {
        // T is the K-th largest value: every key above T, then keys equal to T
        // in ascending expert order (expert = lane + 64 * slot: slot-major)
        int need = K;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            sel[i] = __ballot(u[i] > T);
            need -= __popcll(sel[i]);
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            uint64_t m = __ballot(u[i] == T);
            while (need > 0 && m != 0ull) {
                const uint64_t low = m & (~m + 1ull);
                sel[i] |= low;
                m ^= low;
                --need;
            }
        }
    }
    int base = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if ((sel[i] >> lane) & 1ull) {
            const int pos = base + __popcll(sel[i] & ((1ull << lane) - 1ull));
            sc.u[pos] = u[i];
            sc.e[pos] = lane + kWave * i;
        }
        base += __popcll(sel[i]);
    }
    wave_lds_sync();
    // every lane reads all kMaxTopK scratch entries (broadcast, unconditional);
    // entries at or past K are masked out of the arithmetic
    const uint32_t uj = sc.u[lane & (kMaxTopK - 1)];
    const int ej = sc.e[lane & (kMaxTopK - 1)];
    uint32_t umax = 0;
    int rank = 0;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        const uint32_t uk = sc.u[k];
        const int ek = sc.e[k];
        const bool in = k < K;
        rank += in && ((uk > uj) || (uk == uj && ek < ej));
        umax = in ? max(umax, uk) : umax;
    }
    const float ex = (lane < K) ? expf(f32_from_orderable(uj) - f32_from_orderable(umax)) : 0.0f;
    const float den = wave_sum(ex);
    if (lane < K) {
        ids_out[rank] = ej;
        w_out[rank] = ex / den;
    }
    wave_lds_sync();   // the scratch may be reused by this wave's next token
}

__device__ void topk_wave(const float* L, int E, int K, int32_t* ids_out, float* w_out, TopkScratch& sc)
{
    if (E <= 64) topk_wave_t<1>(L, E, K, ids_out, w_out, sc);
    else if (E <= 128) topk_wave_t<2>(L, E, K, ids_out, w_out, sc);
    else if (E <= 256) topk_wave_t<4>(L, E, K, ids_out, w_out, sc);
    else topk_wave_t<8>(L, E, K, ids_out, w_out, sc);
}

}  // namespace moe
