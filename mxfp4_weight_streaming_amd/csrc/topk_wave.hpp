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
#include "moe_types.hpp"

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

// Top-K of one token's E logits by one wave, as K rounds of a wave-wide
// maximum of the orderable logit: each round takes the largest remaining
// value and, among the experts holding it, the lowest index (expert
// e = lane + 64 i, so the first slot i whose ballot matches, at its lowest
// lane), so the winners come out in canonical order (logit descending, lower
// index first among equal logits).  A taken value is cleared to 0, below
// every real value.  The weights are the softmax over the selected logits.
template <int PER>
__device__ void topk_wave_t(const float* L, int E, int K, int32_t* ids_out, float* w_out)
{
    const int lane = threadIdx.x & 63;
    uint32_t u[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {             // unconditional loads: all in flight together
        const int e = lane + kWave * i;
        const float v = L[e < E ? e : E - 1];
        u[i] = (e < E) ? f32_orderable(v + 0.0f) : 0u;   // + 0.0f folds -0 into +0
    }
    uint32_t my_u = 0u;                         // lane r ends with the rank-r value and expert
    int my_e = 0;
    uint32_t top = 0u;
    for (int r = 0; r < K; ++r) {
        uint32_t best = u[0];
#pragma unroll
        for (int i = 1; i < PER; ++i) best = max(best, u[i]);
        const uint32_t m = wave_max_u32(best);
        int wi = PER, wl = 0;
#pragma unroll
        for (int i = PER - 1; i >= 0; --i) {    // the lowest slot with a match wins
            const uint64_t b = __ballot(u[i] == m);
            if (b != 0ull) {
                wi = i;
                wl = (int)__builtin_ctzll(b);
            }
        }
        if (r == 0) top = m;
        if (lane == r) {
            my_u = m;
            my_e = wl + kWave * wi;
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) u[i] = (i == wi && lane == wl) ? 0u : u[i];
    }
    const float lmax = f32_from_orderable(top);
    const float ex = (lane < K) ? expf(f32_from_orderable(my_u) - lmax) : 0.0f;
    const float den = wave_sum(ex);
    if (lane < K) {
        ids_out[lane] = my_e;
        w_out[lane] = ex / den;
    }
}

__device__ void topk_wave(const float* L, int E, int K, int32_t* ids_out, float* w_out)
{
    if (E <= 64) topk_wave_t<1>(L, E, K, ids_out, w_out);
    else if (E <= 128) topk_wave_t<2>(L, E, K, ids_out, w_out);
    else if (E <= 256) topk_wave_t<4>(L, E, K, ids_out, w_out);
    else topk_wave_t<8>(L, E, K, ids_out, w_out);
}

}  // namespace moe
