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

// Top-K of one token's E logits by one wave.  Lane l holds the logits of
// experts l + 64 i (slot i), as orderable keys, sorted once inside the lane
// by (key descending, slot ascending).  Each of the K rounds takes the
// wave-wide maximum of the lanes' first entries; the lane holding it (among
// several lanes with an equal first key, the one whose expert index is
// lowest) gives up that entry.  Since a lane's equal keys are in slot order,
// the winners come out in canonical order: logit descending, lower expert
// index first among equal logits.  The weights are the softmax over the
// selected logits.
template <int PER>
__device__ __forceinline__ void lane_sort_step(uint32_t* u, int* s, int a, int b)
{
    const bool sw = u[b] > u[a] || (u[b] == u[a] && s[b] < s[a]);
    const uint32_t ua = u[a], ub = u[b];
    const int sa = s[a], sb = s[b];
    u[a] = sw ? ub : ua;
    u[b] = sw ? ua : ub;
    s[a] = sw ? sb : sa;
    s[b] = sw ? sa : sb;
}

// One out-of-line body per logits-per-lane count, called through the inlined
// dispatch below, where E is wave-uniform: every body inlined at every call
// site made the gate/up kernels larger and slower.
template <int PER>
__device__ __noinline__ void topk_wave_t(const float* Lg, int E, int K, int32_t* ids_out, float* w_out, int R)
{
    const int lane = threadIdx.x & 63;
    // the logits are in global memory: loads through a global pointer are
    // counted by one counter and waited for together (a generic pointer gives
    // flat loads, counted by two)
    const __attribute__((address_space(1))) float* L = (const __attribute__((address_space(1))) float*)Lg;
    uint32_t u[PER];
    int s[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {             // unconditional loads: all in flight together
        const int e = lane + kWave * i;
        const float v = L[e < E ? e : E - 1];
        // + 0.0f folds -0 into +0; 0 is below every key.  The mask is
        // arithmetic, so the load's result is always used and the compiler
        // cannot move the load into a branch (with a wait of its own)
        u[i] = f32_orderable(v + 0.0f) & (0u - (uint32_t)(e < E));
        s[i] = i;
    }
    // sorting network over the lane's entries (a strict order: slots differ)
    if constexpr (PER == 2) {
        lane_sort_step<PER>(u, s, 0, 1);
    } else if constexpr (PER == 4) {
        lane_sort_step<PER>(u, s, 0, 1);
        lane_sort_step<PER>(u, s, 2, 3);
        lane_sort_step<PER>(u, s, 0, 2);
        lane_sort_step<PER>(u, s, 1, 3);
        lane_sort_step<PER>(u, s, 1, 2);
    } else if constexpr (PER > 4) {              // odd-even transposition
#pragma unroll
        for (int ph = 0; ph < PER; ++ph)
#pragma unroll
            for (int a = ph & 1; a + 1 < PER; a += 2) lane_sort_step<PER>(u, s, a, a + 1);
    }
    uint32_t my_u = 0u;                         // lane r ends with the rank-r value and expert
    int my_e = 0;
    uint32_t top = 0u;
    for (int r = 0; r < R; ++r) {
        const uint32_t m = wave_max_u32(u[0]);
        const uint64_t b = __ballot(u[0] == m);
        int wl = (int)__builtin_ctzll(b);
        if (__popcll(b) > 1) {                  // equal first keys in several lanes (an exact tie)
            const uint32_t cand = (u[0] == m) ? (uint32_t)(lane + kWave * s[0]) : 0xFFFFFFFFu;
            wl = (int)(wave_min_u32(cand) & (kWave - 1));
        }
        const int we = wl + kWave * __builtin_amdgcn_readlane(s[0], wl);
        if (r == 0) top = m;
        if (lane == r) {
            my_u = m;
            my_e = we;
        }
        if (lane == wl) {                       // the winner gives up its first entry
#pragma unroll
            for (int i = 0; i + 1 < PER; ++i) {
                u[i] = u[i + 1];
                s[i] = s[i + 1];
            }
            u[PER - 1] = 0u;
            s[PER - 1] = PER;
        }
    }
    if (R < K) {                                // the first R ranks only: their experts
        if (lane < R) ids_out[lane] = my_e;
        return;
    }
    const float lmax = f32_from_orderable(top);
    const float ex = (lane < K) ? expf(f32_from_orderable(my_u) - lmax) : 0.0f;
    const float den = wave_sum(ex);
    if (lane < K) {
        ids_out[lane] = my_e;
        w_out[lane] = ex / den;
    }
}

// Top-K of one token's E logits by one wave: ids_out[r] is the rank-r expert
// and w_out[r] its softmax weight over the K selected.  With R < K only the
// first R ranks are found (ids only; their ranking is the same as in the
// full call).
__device__ __forceinline__ void topk_wave(const float* L, int E, int K, int32_t* ids_out, float* w_out, int R = -1)
{
    if (R < 0 || R > K) R = K;
    if (E <= 64) topk_wave_t<1>(L, E, K, ids_out, w_out, R);
    else if (E <= 128) topk_wave_t<2>(L, E, K, ids_out, w_out, R);
    else if (E <= 256) topk_wave_t<4>(L, E, K, ids_out, w_out, R);
    else topk_wave_t<8>(L, E, K, ids_out, w_out, R);
}

}  // namespace moe
