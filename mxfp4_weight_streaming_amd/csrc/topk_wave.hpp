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

// The ranks of the selection, in registers: lane r < R ends with the rank-r
// expert (e) and its key (u); top is the largest key (in every lane).
struct TopkRanks {
    int e;
    uint32_t u;
    uint32_t top;
};

// Selection by threshold, one pass.  The lanes form 8 groups of 8 (lanes
// 8g..8g+7, all their entries); each group's largest key is an entry of its
// own, so at least 8 entries are >= T, the smallest of the 8 group maxima, and
// the K <= 8 selected entries (whose keys are >= the K-th largest) are among
// the candidates, the valid entries with key >= T.  The candidates go to LDS
// as 64-bit keys (key << 32 | 0xFFFF - expert: distinct, and larger exactly
// when the logit is larger or, for an equal logit, the expert lower), and each
// candidate's rank is the number of larger candidate keys.  That is the
// canonical order of the rounds below, so both give the same ranks.  Returns
// false, having written nothing, when the candidates do not fit one per lane
// (many equal logits) or are fewer than R; the caller then takes the rounds.
constexpr int kTopkMaxWaves = 16;               // waves in a workgroup of 1024 threads

// This wave's LDS area of the threshold pass: one array for every caller and
// instantiation (a kernel holds it once).
__device__ __forceinline__ uint64_t* topk_lds_wave()
{
    __shared__ __attribute__((aligned(16))) uint64_t tk_lds[kTopkMaxWaves][kWave + kMaxTopK];
    return tk_lds[threadIdx.x >> 6];
}

template <int PER>
__device__ __forceinline__ bool topk_threshold_t(const uint32_t (&u)[PER], const int (&s)[PER], int R,
                                                 TopkRanks& out, uint64_t* c)
{
    const int lane = threadIdx.x & 63;
    uint32_t g = u[0];
#pragma unroll
    for (int i = 1; i < PER; ++i) g = max(g, u[i]);
    g = max(g, dpp_u32<kDppXor1>(g));            // the maximum of each group of 8 lanes
    g = max(g, dpp_u32<kDppXor2>(g));
    g = max(g, dpp_u32<kDppHalfMirror>(g));
    uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)g, 0), top = lo;
#pragma unroll
    for (int q = 1; q < 8; ++q) {
        const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)g, 8 * q);
        lo = min(lo, v);
        top = max(top, v);
    }
    const uint32_t thr = max(lo, 1u);            // key 0 marks entries past E
    uint64_t b[PER];
    int nc = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        b[i] = __ballot(u[i] >= thr);
        nc += __popcll(b[i]);
    }
    if (nc > kWave || nc < R) return false;
    c[lane] = 0;                                 // lanes past the candidates hold key 0
    int base = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (u[i] >= thr) {
            const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b[i] >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)b[i], 0u));
            c[pos] = ((uint64_t)u[i] << 32) | (uint32_t)(0xFFFF - (lane + kWave * s[i]));
        }
        base += __popcll(b[i]);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const uint64_t mine = c[lane];
    int rank = 0;
    // the same addresses in every lane (broadcast reads), 16 keys a step with
    // every read issued before the first compare: one LDS round trip per 16
    // candidates (entries past nc hold key 0)
    for (int j = 0; j < nc; j += 16) {
        ulonglong2 kk[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) kk[q] = *reinterpret_cast<const ulonglong2*>(c + j + 2 * q);
#pragma unroll
        for (int q = 0; q < 8; ++q) rank += (kk[q].x > mine ? 1 : 0) + (kk[q].y > mine ? 1 : 0);
    }
    if (lane < nc && rank < R) c[kWave + rank] = mine;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const uint64_t k = c[kWave + min(lane, kMaxTopK - 1)];
    const bool ranked = lane < R;
    out.e = ranked ? (int)(0xFFFFu - (uint32_t)(k & 0xFFFFu)) : 0;
    out.u = ranked ? (uint32_t)(k >> 32) : 0u;
    out.top = top;
    return true;
}

// The R rounds on keys already held by the lanes: lane l holds the keys of
// experts l + 64 s[i] in u[i] (0 for experts past E), s[i] = i.  With THRESH
// the threshold pass above serves whenever it can (in the caller's LDS area
// lds with OWN_LDS, else in topk_lds_wave()); the rounds sort each lane's
// entries first.
template <int PER, bool THRESH = true, bool OWN_LDS = false>
__device__ __forceinline__ TopkRanks topk_rounds_t(uint32_t (&u)[PER], int (&s)[PER], int R,
                                                   uint64_t* lds = nullptr)
{
    const int lane = threadIdx.x & 63;
    if constexpr (THRESH) {
        TopkRanks t;
        uint64_t* c;
        if constexpr (OWN_LDS) c = lds;                // the caller's area
        else c = topk_lds_wave();
        if (topk_threshold_t<PER>(u, s, R, t, c)) return t;
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
    return TopkRanks{my_e, my_u, top};
}

// The softmax weight of lane r's selection (r < K; 0 in the other lanes).
__device__ __forceinline__ float topk_weight(const TopkRanks& t, int K)
{
    const int lane = threadIdx.x & 63;
    const float lmax = f32_from_orderable(t.top);
    const float ex = (lane < K) ? expf(f32_from_orderable(t.u) - lmax) : 0.0f;
    return ex / wave_sum(ex);
}

// The selection: the R rounds, then ids_out[0..R) and, when R == K and w_out
// is not null, the softmax weights w_out[0..K).
template <int PER>
__device__ __forceinline__ void topk_select_t(uint32_t (&u)[PER], int (&s)[PER], int K, int32_t* ids_out,
                                              float* w_out, int R)
{
    const int lane = threadIdx.x & 63;
    const TopkRanks t = topk_rounds_t<PER>(u, s, R);
    if (R < K || w_out == nullptr) {            // the first R ranks only, or no weights: their experts
        if (lane < R) ids_out[lane] = t.e;
        return;
    }
    const float w = topk_weight(t, K);
    if (lane < K) {
        ids_out[lane] = t.e;
        w_out[lane] = w;
    }
}

// The key of a logit: + 0.0f folds -0 into +0; 0 is below every key and
// marks experts past E.
__device__ __forceinline__ uint32_t topk_key(float v, bool valid)
{
    return f32_orderable(v + 0.0f) & (0u - (uint32_t)valid);
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
        // the mask is arithmetic, so the load's result is always used and
        // the compiler cannot move the load into a branch (with a wait of its own)
        u[i] = topk_key(v, e < E);
        s[i] = i;
    }
    topk_select_t<PER>(u, s, K, ids_out, w_out, R);
}

// One token's logits for every E <= 512: lane l loads experts l + 64 i,
// i < 8 (clamped past E), all issued here and none waited for.
struct TopkLogits8 {
    float v[8];
};

__device__ __forceinline__ TopkLogits8 topk_load_logits8(const float* Lg, int E)
{
    const int lane = threadIdx.x & 63;
    const __attribute__((address_space(1))) float* L = (const __attribute__((address_space(1))) float*)Lg;
    TopkLogits8 l;
#pragma unroll
    for (int i = 0; i < 8; ++i) l.v[i] = L[min(lane + kWave * i, E - 1)];
    return l;
}

// Their keys (0 past E), waited for here, together: the empty asm statements
// consume every key, so no load can be moved into a branch of the caller's
// dispatch on E.  (With the loads inside that dispatch the compiler issued
// them in groups along it, each group waited for before the next went out:
// two memory round trips at E = 256 instead of one.)
struct TopkKeys8 {
    uint32_t u[8];
};

__device__ __forceinline__ TopkKeys8 topk_keys8(const TopkLogits8& l, int E)
{
    const int lane = threadIdx.x & 63;
    TopkKeys8 k;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        k.u[i] = topk_key(l.v[i], lane + kWave * i < E);
        asm volatile("" : : "v"(k.u[i]));
    }
    return k;
}

// The first R ranks of one token from its keys, PER = 1, 2, 4 or 8 entries a
// lane (E <= 64 PER), in registers (see TopkRanks).  The threshold pass runs
// in the caller's LDS area lds (wave 0 of the one-token gate/up kernel passes
// routing scratch it leaves unused: the pass's own array compiled into that
// kernel took its LDS from 7 to 16 KB, and the graph-replayed one-token layer
// was slower with it, 16.2 -> 16.4 us).
template <int PER>
__device__ __forceinline__ TopkRanks topk_ranks_keys(const TopkKeys8& k, int R, uint64_t* lds)
{
    uint32_t u[PER];
    int s[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        u[i] = k.u[i];
        s[i] = i;
    }
    return topk_rounds_t<PER, true, true>(u, s, R, lds);
}

// The first R ranks of one token's E logits by one wave (wave-uniform E).
// Inlined: its callers keep the result in registers.  lds: the wave's 576
// bytes (16-byte aligned) for the threshold pass.
__device__ __forceinline__ TopkRanks topk_wave_ranks(const float* L, int E, int R, uint64_t* lds)
{
    const TopkKeys8 k = topk_keys8(topk_load_logits8(L, E), E);
    if (E <= 64) return topk_ranks_keys<1>(k, R, lds);
    if (E <= 128) return topk_ranks_keys<2>(k, R, lds);
    if (E <= 256) return topk_ranks_keys<4>(k, R, lds);
    return topk_ranks_keys<8>(k, R, lds);
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
