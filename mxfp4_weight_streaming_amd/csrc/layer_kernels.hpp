// layer_kernels.hpp -- the W4A8 MoE decode layer (1-8 tokens) as ONE gfx950
// kernel.  Device code only: compiled ahead of time through moe_kernels.hip
// and at run time by hipRTC.
//
// The pages find batch-1 MoE decode bound by reading expert weights ([EN]
// "Why is MoE decoding on DGX Spark memory-bound?").  At one token a layer
// moves 26 MB, about 3.3 us of this chip's HBM time, so every fixed cost on
// the layer's dependent chain (router -> top-K -> gate/up -> requantisation
// -> down -> combine) counts.  The layer is one kernel with one workgroup per
// compute unit, all resident at once; the workgroups hand results to each
// other through epoch-tagged 64-bit words (LayerSync) instead of kernel
// boundaries:
//   1. router: workgroup b computes the logits of experts b, b + NB, ... and
//      publishes them; meanwhile it quantises every token to FP8 into LDS;
//   2. routing: each workgroup waits for all logits and runs the top-K
//      (ties to the lower index, softmax over the selection) and the
//      token->expert compaction itself ([EN] "What is Ling 3.0...": 8 routed
//      experts per token, plus one shared expert; [EN] "What are the 3
//      optimizations?", item 3: a 4-token verify touches up to 32 experts);
//   3. the layer's weight stream: gate/up tasks (a wave's rows of one slot)
//      and down tasks (a wave's output rows of one slot) are dealt out in
//      equal contiguous ranges; a wave keeps the next task's loads in flight
//      while it computes the current one, and issues its first down task's
//      loads right after its last gate/up task, before the requantisation
//      waits;
//   4. gate/up: SiLU(gate) * up per (pair, row), published tagged;
//   5. requantisation: each workgroup waits for the h rows of the slots its
//      down tasks cover and requantises them to FP8 in LDS (per (token,
//      expert) scale);
//   6. down: per (pair, row) the router-weighted, s2-scaled dot product,
//      published tagged;
//   7. combine: workgroup b sums, in a fixed order (the token's K selections,
//      then the shared expert), the published down outputs of its share of
//      the output rows.
// Every wait is bounded (LayerArgs::wait_ticks of the 100 MHz real-time
// clock): a wait that runs out sets a sticky error bit in LayerSync::word[1]
// and the workgroup goes on without waiting again, so the kernel always ends.
// The M <= 8 path is a GEMV on the vector ALU (exactly decoded f16 operands,
// dot2 with fp32 accumulation), not the matrix cores.
//   [EN] = "NVIDIA Shows 3 Ways to Speed Up MoE Inference on DGX Spark,
//          Lifting Ling-3.0-flash Throughput 42.5%"
#pragma once

#include "gemv_kernels.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Tagged words: (tag << 32) | fp32 bits, written and read whole by relaxed
// device-scope atomics (one 64-bit store / load each, no fences).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t tag_word(uint32_t ep, float v)
{
    return ((uint64_t)ep << 32) | (uint64_t)__float_as_uint(v);
}
__device__ __forceinline__ void put_tagged(uint64_t* p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get_tagged(const uint64_t* p)
{
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool has_tag(uint64_t v, uint32_t ep) { return (uint32_t)(v >> 32) == ep; }
__device__ __forceinline__ float tagged_value(uint64_t v) { return __uint_as_float((uint32_t)v); }

__device__ __forceinline__ uint64_t realtime() { return __builtin_amdgcn_s_memrealtime(); }

// One wave waits until poll() is true in every lane.  poll() issues its
// loads and tests them; it is called again after a pause until the deadline.
// The pauses double from ~60 ns up to ~0.25 us: many waves re-reading the
// same words back to back would starve the memory traffic of the waves that
// produce them, while a hand-off itself takes ~0.3 us.  Returns false (and
// records `bit`) when the wait ran out; a wave whose workgroup already ran
// out of a wait (failed) does not wait again.
struct WaitBound {
    uint64_t ticks;        // s_memrealtime ticks a wait may take
    uint32_t* err;         // sticky error bits (LayerSync::word + 1)
};

template <typename Poll>
__device__ __forceinline__ bool wave_wait(Poll poll, WaitBound wb, uint32_t bit, bool& failed)
{
    if (__all(poll())) return true;
    if (failed) return false;
    const uint64_t t0 = realtime();
    int naps = 1;
    for (;;) {
        for (int i = 0; i < naps; ++i) __builtin_amdgcn_s_sleep(2);   // 128 clocks each
        if (__all(poll())) return true;
        if (realtime() - t0 > wb.ticks) break;
        naps = naps < 4 ? 2 * naps : 4;
    }
    failed = true;
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_or(wb.err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
}

// Top-K of one token from its tagged logits, by one wave: waits for every
// logit of this call, then the selection of topk_select_t (the same
// arithmetic as topk_wave, so both paths pick the same experts and weights:
// neither the selection nor the weights depend on how the keys are spread
// over the lanes, so one body with 8 keys per lane serves every E <= 512,
// inlined: an out-of-line call would give the kernel a stack).
template <int PER>
__device__ __forceinline__ bool topk_tagged_t(const uint64_t* tl, int E, int K, uint32_t ep, int32_t* ids_out,
                                              float* w_out, WaitBound wb, bool failed)
{
    const int lane = threadIdx.x & 63;
    uint64_t v[PER];
    auto poll = [&]() {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = lane + kWave * i;
            if (e < E) {                        // lanes past E load nothing
                v[i] = get_tagged(tl + e);
                ok &= has_tag(v[i], ep);
            }
        }
        return ok;
    };
    wave_wait(poll, wb, kWaitLogits, failed);
    uint32_t u[PER];
    int s[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        u[i] = topk_key(tagged_value(v[i]), lane + kWave * i < E);
        s[i] = i;
    }
    topk_select_t<PER>(u, s, K, ids_out, w_out, K);
    return failed;
}

__device__ __forceinline__ bool topk_tagged(const uint64_t* tl, int E, int K, uint32_t ep, int32_t* ids_out,
                                            float* w_out, WaitBound wb, bool failed)
{
    static_assert(kMaxExperts <= 8 * kWave, "8 keys per lane");
    return topk_tagged_t<8>(tl, E, K, ep, ids_out, w_out, wb, failed);
}

// Equal contiguous shares of W tasks over NB workgroups (W * NB < 2^31).
__device__ __forceinline__ int share_lo(int W, int b, int NB) { return (int)(((uint32_t)W * (uint32_t)b) / (uint32_t)NB); }

template <int H, int I>
struct LayerGeom {
    // gate/up task: RW row pairs of one slot, LPR lanes per row, CPL blocks each
    static constexpr int CH = H / 32;
    static constexpr int LPR = gate_up_lanes_per_row(H);
    static constexpr int CPL = CH / LPR;
    static constexpr int RW = kWave / LPR;
    static constexpr int GT = layer_gate_up_tasks(H, I);
    // down task: DP passes of RP rows of one slot, LD lanes per row, CD blocks each
    static constexpr int CI = I / 32;
    static constexpr int LD = layer_down_lanes(I);
    static constexpr int CD = layer_down_blocks(I);
    static constexpr int RP = layer_down_rows_per_pass(I);
    static constexpr int DP = layer_down_passes(H, I);
    static constexpr int RD = RP * DP;
    static constexpr int DT = layer_down_tasks(H, I);
    static constexpr int NW = kLayerWaves;
    // block scales of a gate/up row as dwords spread over the row's lanes
    static constexpr bool kScaleDw = LPR % 4 == 0 && CH % 4 == 0;
    static constexpr int NSW = kScaleDw ? (CH / 4 + LPR - 1) / LPR : CPL;
    static_assert(layer_shape_ok(H, I), "unsupported one-kernel layer shape");
    static_assert(GT * RW == I && DT * RD == H, "layer blocking");
};

template <int H, int I, int MT>
__global__ __launch_bounds__(512, 1) void layer_kernel(LayerArgs a)
{
    using G = LayerGeom<H, I>;
    constexpr int CH = G::CH, LPR = G::LPR, CPL = G::CPL, CI = G::CI, LD = G::LD, CD = G::CD, DP = G::DP;
    constexpr int NW = G::NW;
    extern __shared__ u32x4 lds_dyn[];
    u32x4* act = lds_dyn;                      // [MT][4][CH]
    u32x4* q2h = lds_dyn + MT * 4 * CH;        // [pairs of this workgroup's down slots][4][CI]
    __shared__ RouteLds rl;
    __shared__ float act_sl[MT];
    __shared__ float s2l[kMaxPairsExt];
    constexpr int NCH = H / 8, NTR = router_threads(H), NR = NTR / 16;
    __shared__ float red_dot[2][MT][NR], red_max[MT][NR];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int NB = gridDim.x, b = blockIdx.x;
    const int M = a.M, E = a.E, K = a.K, P = M * K;
    const bool routed = a.x != nullptr;
    const WaitBound wb{a.wait_ticks, a.sync.word + 1};
    bool failed = false;

    // 0. this call's tag, and this workgroup's arrival (workgroup 0 moves the
    //    epoch on only once every workgroup has read it).  Each workgroup
    //    reads its own copy of the epoch: 256 workgroups reading one word at
    //    once queue behind each other at its memory channel.
    const uint32_t ep = __hip_atomic_load(a.sync.epochs + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    if (tid == 0) put_tagged(a.sync.arrive + b, tag_word(ep, 0.0f));

    // 1. router rows b, b + NB (one or two per round) and the activations.
    //    Thread c < H/8 holds the 16-byte chunk c of each row and of every
    //    token; the dot products and the per-token maxima reduce on DPP within
    //    rows of 16 lanes and then in LDS in a fixed order (the router
    //    kernel's arithmetic, so both give the same logits).
    if (routed) {
        const bool own = tid < NCH;
        const int c = own ? tid : NCH - 1;
        u32x4 xv[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) xv[t] = *(reinterpret_cast<const u32x4*>(a.x + (size_t)min(t, M - 1) * H) + c);
        bool first = true;
        for (int e0 = b; e0 < E || first; e0 += 2 * NB) {
            const int e1 = e0 + NB;
            const u32x4 w0 = load_stream(reinterpret_cast<const u32x4*>(a.wr + (size_t)min(e0, E - 1) * H) + c);
            const u32x4 w1 = load_stream(reinterpret_cast<const u32x4*>(a.wr + (size_t)min(e1, E - 1) * H) + c);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const float d0 = group_sum<16>(own ? dot_bf16x8(xv[t], w0, 0.0f) : 0.0f);
                const float d1 = group_sum<16>(own ? dot_bf16x8(xv[t], w1, 0.0f) : 0.0f);
                if ((lane & 15) == 0 && tid < NTR) {
                    red_dot[0][t][tid >> 4] = d0;
                    red_dot[1][t][tid >> 4] = d1;
                }
                if (first) {
                    const float m = row16_max(own ? amax_bf16x8(xv[t]) : 0.0f);
                    if ((lane & 15) == 0 && tid < NTR) red_max[t][tid >> 4] = m;
                }
            }
            __syncthreads();
            if (tid < 2 * M) {
                const int t = tid % M, j = tid / M, e = j ? e1 : e0;
                float d = 0.0f;
#pragma unroll
                for (int r = 0; r < NR; ++r) d += red_dot[j][t][r];
                if (e < E) put_tagged(a.sync.logits + (size_t)t * E + e, tag_word(ep, d));
            }
            if (first) {
                // every token's FP8 codes as f16 in LDS: s = amax / 448, codes
                // E4M3(x / s) (the router kernel's quantisation)
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    if (t < M && own) {
                        float m = 0.0f;
#pragma unroll
                        for (int r = 0; r < NR; ++r) m = fmaxf(m, red_max[t][r]);
                        const QuantScale qs = quant_scale(m);
                        const uint32_t vv[4] = {xv[t].x, xv[t].y, xv[t].z, xv[t].w};
                        uint32_t code[2] = {0u, 0u};
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const uint32_t bb = (j & 1) ? (vv[j >> 1] & 0xFFFF0000u) : (vv[j >> 1] << 16);
                            code[j >> 2] |= e4m3_encode(quant_div(__uint_as_float(bb), qs)) << (8 * (j & 3));
                        }
                        act[(t * 4 + (c & 3)) * CH + (c >> 2)] = e4m3x8_to_half8(u32x2{code[0], code[1]});
                        if (c == 0) act_sl[t] = qs.s;
                    }
                }
            }
            first = false;
            __syncthreads();        // red_dot is reused by the next round
        }
    } else {
        // caller-given FP8 activations, scales, ids and weights
        constexpr int NST = (MT * (H / 8) + 511) / 512;
        const int n8 = M * (H / 8);
#pragma unroll
        for (int j = 0; j < NST; ++j) {
            const int idx = tid + 512 * j;
            const u32x2 v = ((const u32x2*)a.act_q)[min(idx, n8 - 1)];
            if (idx < n8) {
                const int t = idx / (H / 8), g8 = idx % (H / 8);
                act[(t * 4 + (g8 & 3)) * CH + (g8 >> 2)] = e4m3x8_to_half8(v);
            }
        }
        if (tid < M) act_sl[tid] = a.act_s[tid];
        if (tid < P) {
            rl.ids[tid] = min(max(a.ids[tid], 0), E - 1);     // clamped, never out of bounds
            rl.w[tid] = a.topk_w[tid];
        }
    }

    // 2. routing: wave t ranks token t from the published logits; wave 0
    //    compacts (slots in ascending expert id, then the shared expert)
    if (routed && wave < M)
        failed = topk_tagged(a.sync.logits + (size_t)wave * E, E, K, ep, rl.ids + wave * K, rl.w + wave * K, wb,
                             failed);
    __syncthreads();
    route_compact(M, K, routed, a.shared, rl);
    __syncthreads();
    if (routed && b == 0 && tid < P) {
        if (a.ids_out != nullptr) a.ids_out[tid] = rl.ids[tid];
        if (a.w_out != nullptr) a.w_out[tid] = rl.w[tid];
    }

    const int n_slots = rl.n_act;
    const int Wg = n_slots * G::GT, Wd = n_slots * G::DT;
    const int g_lo = share_lo(Wg, b, NB), g_hi = share_lo(Wg, b + 1, NB);
    const int d_lo = share_lo(Wd, b, NB), d_hi = share_lo(Wd, b + 1, NB);
    const int ng = g_hi - g_lo > wave ? (g_hi - g_lo - wave + NW - 1) / NW : 0;
    const int nd = d_hi - d_lo > wave ? (d_hi - d_lo - wave + NW - 1) / NW : 0;

    // ---- task loads.  Every issue is unconditional: a task past the wave's
    // last loads a fixed in-bounds row piece (the first expert's first row)
    // that nothing uses, so the count of loads in flight is the same on every
    // path and each wait covers exactly the task in use.
    const int gli = lane % LPR, ggrp = lane / LPR;      // gate/up: lane in row, row in task
    const int dli = lane % LD, dgrp = lane / LD;        // down
    struct StageG {
        u32x4 wg[CPL], wu[CPL];
        uint32_t sg[G::NSW], su[G::NSW];
    };
    struct StageD {
        u32x4 w[DP * CD];
        uint32_t sc[DP * CD];
    };
    // Task loads: buffer loads on a resource spanning one expert's matrix
    // (the expert base in scalar registers), non-temporal for the weights.
    constexpr uint32_t kW13Bytes = 2u * I * (H / 2), kS13Bytes = 2u * I * CH;
    constexpr uint32_t kW2Bytes = (uint32_t)H * (I / 2), kS2Bytes = (uint32_t)H * CI;
    auto rsrc = [](const uint8_t* base, uint32_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)bytes, 0x00020000);
    };
    // a slot's expert (kSharedExpert: the shared expert's own tensors), wave-uniform
    auto slot_expert = [&](int slot) { return __builtin_amdgcn_readfirstlane(rl.act_experts[slot]); };
    auto issue_g = [&](int i, StageG& st) {
        const int task = g_lo + wave + NW * i;
        const int e = slot_expert(task / G::GT);
        const bool sh = e == kSharedExpert;
        const uint8_t* wb = sh ? a.sh.w13 : a.w13 + (size_t)max(e, 0) * kW13Bytes;
        const uint8_t* sb = sh ? a.sh.s13 : a.s13 + (size_t)max(e, 0) * kS13Bytes;
        const uint32_t r = (uint32_t)((task % G::GT) * G::RW + ggrp);
        const auto rw = rsrc(wb, kW13Bytes), rs = rsrc(sb, kS13Bytes);
        const uint32_t go = r * (H / 2) + gli * 16, uo = (r + I) * (H / 2) + gli * 16;
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            st.wg[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, go + LPR * 16 * k, 0, 2));
            st.wu[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, uo + LPR * 16 * k, 0, 2));
        }
        if constexpr (G::kScaleDw) {
#pragma unroll
            for (int j = 0; j < G::NSW; ++j) {
                const uint32_t d = (uint32_t)min(gli + LPR * j, CH / 4 - 1) * 4;
                st.sg[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, r * CH + d, 0, 0);
                st.su[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, (r + I) * CH + d, 0, 0);
            }
        } else {
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const uint32_t d = (uint32_t)(gli + LPR * k);
                st.sg[k] = __builtin_amdgcn_raw_buffer_load_b8(rs, r * CH + d, 0, 0);
                st.su[k] = __builtin_amdgcn_raw_buffer_load_b8(rs, (r + I) * CH + d, 0, 0);
            }
        }
    };
    auto issue_d = [&](int i, StageD& st) {
        const int task = d_lo + wave + NW * i;
        const int e = slot_expert(task / G::DT);
        const bool sh = e == kSharedExpert;
        const uint8_t* wb = sh ? a.sh.w2 : a.w2 + (size_t)max(e, 0) * kW2Bytes;
        const uint8_t* sb = sh ? a.sh.s2 : a.sw2 + (size_t)max(e, 0) * kS2Bytes;
        const uint32_t n = (uint32_t)((task % G::DT) * G::RD + dgrp);
        const auto rw = rsrc(wb, kW2Bytes), rs = rsrc(sb, kS2Bytes);
#pragma unroll
        for (int h = 0; h < DP; ++h)
#pragma unroll
            for (int k = 0; k < CD; ++k)
                st.w[h * CD + k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    rw, (n + h * G::RP) * (I / 2) + (uint32_t)(dli + LD * k) * 16, 0, 2));
#pragma unroll
        for (int h = 0; h < DP; ++h)
#pragma unroll
            for (int k = 0; k < CD; ++k)
                st.sc[h * CD + k] =
                    __builtin_amdgcn_raw_buffer_load_b8(rs, (n + h * G::RP) * CI + (uint32_t)(dli + LD * k), 0, 0);
        __builtin_amdgcn_sched_barrier(0);   // the task's loads go out here, not next to their uses
    };
    // A wave's n tasks with the next task's loads in flight while one
    // computes, on two stage buffers used in turn.  Only existing tasks are
    // loaded, and every wait is exact: the loop body and each tail path hold
    // a fixed number of newer loads at each compute.  started: task 0 is
    // already in flight in A.
    auto run = [&](int n, auto& A, auto& B, auto issue, auto compute, bool started) {
        if (n <= 0) return;
        if (!started) issue(0, A);
        int i = 0;
        for (; i + 2 < n; i += 2) {
            issue(i + 1, B);
            compute(i, A);
            issue(i + 2, A);
            compute(i + 1, B);
        }
        if (i + 1 < n) {
            issue(i + 1, B);
            compute(i, A);
            compute(i + 1, B);
        } else {
            compute(i, A);
        }
    };

    // the block scale code of block gli + LPR k of this lane's gate/up row
    auto scale_of = [&](const uint32_t* sw, int k) -> uint32_t {
        if constexpr (G::kScaleDw) {
            const int src = LPR * ggrp + ((LPR / 4) * k + gli / 4) % LPR;
            const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute(src * 4, (int)sw[k / 4]);
            return (v >> (8 * (gli & 3))) & 0xFFu;
        } else {
            return sw[k];
        }
    };

    // 4. gate/up of one task: for each pair of the slot (MT at a time) the
    //    gate and up dot products of this lane's rows, SiLU(g) * u, published
    auto compute_g = [&](int i, const StageG& st) {
        const int task = g_lo + wave + NW * i;
        const int slot = task / G::GT;
        const int r = (task % G::GT) * G::RW + ggrp;
        const int p0 = rl.offsets[slot], p1 = rl.offsets[slot + 1];
        uint32_t scg[CPL], scu[CPL];
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            scg[k] = scale_of(st.sg, k);
            scu[k] = scale_of(st.su, k);
        }
        for (int pg = p0; pg < p1; pg += MT) {
            const int nt = min(p1 - pg, MT);
            float accg[MT], accu[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) accg[t] = accu[t] = 0.0f;
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const int c = gli + LPR * k;
                // decoded here, per group of pairs: an empty asm marks the
                // codes as changed, so the decodes of all blocks are not
                // hoisted out of the pair loop (they would hold 32 registers
                // per block for the whole loop)
                u32x4 wg = st.wg[k], wu = st.wu[k];
                asm volatile("" : "+v"(wg), "+v"(wu));
                half2_t hg[16], hu[16];
                e2m1x8_to_half(wg.x, hg + 0);
                e2m1x8_to_half(wg.y, hg + 4);
                e2m1x8_to_half(wg.z, hg + 8);
                e2m1x8_to_half(wg.w, hg + 12);
                e2m1x8_to_half(wu.x, hu + 0);
                e2m1x8_to_half(wu.y, hu + 4);
                e2m1x8_to_half(wu.z, hu + 8);
                e2m1x8_to_half(wu.w, hu + 12);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    if (t < nt) {
                        const int tok = rl.pair_token[pg + t];
                        const u32x4 a0 = act[(tok * 4 + 0) * CH + c], a1 = act[(tok * 4 + 1) * CH + c];
                        const u32x4 a2 = act[(tok * 4 + 2) * CH + c], a3 = act[(tok * 4 + 3) * CH + c];
                        accg[t] += ldexp_e8m0(block_dot(hg, a0, a1, a2, a3), scg[k]);
                        accu[t] += ldexp_e8m0(block_dot(hu, a0, a1, a2, a3), scu[k]);
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t < nt) {
                    const float gs = group_sum<LPR>(accg[t]), us = group_sum<LPR>(accu[t]);
                    const float sc = act_sl[rl.pair_token[pg + t]];
                    const float g = gs * sc, u = us * sc;
                    const float hv = g / (1.0f + expf(-g)) * u;
                    if (gli == 0) {
                        const int p = rl.pair_src[pg + t];
                        put_tagged(a.sync.h + (size_t)p * I + r, tag_word(ep, hv));
                        if (a.h_tap != nullptr) a.h_tap[(size_t)p * I + r] = hv;
                    }
                }
            }
        }
    };

    // the pairs of this workgroup's down slots: [q_lo, q_hi) in compaction order
    const int s_lo = d_hi > d_lo ? d_lo / G::DT : 0, s_hi = d_hi > d_lo ? (d_hi - 1) / G::DT : -1;
    const int q_lo = d_hi > d_lo ? rl.offsets[s_lo] : 0, q_hi = d_hi > d_lo ? rl.offsets[s_hi + 1] : 0;

    // 6. down of one task: for each pair of the slot (MT at a time) the dot
    //    products of this lane's rows with the pair's FP8 intermediate, times
    //    the pair's router weight and s2, published
    auto compute_d = [&](int i, const StageD& st) {
        const int task = d_lo + wave + NW * i;
        const int slot = task / G::DT;
        const int n = (task % G::DT) * G::RD + dgrp;
        const int p0 = rl.offsets[slot], p1 = rl.offsets[slot + 1];
        for (int pg = p0; pg < p1; pg += MT) {
            const int nt = min(p1 - pg, MT);
            float acc[MT][DP];
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int h = 0; h < DP; ++h) acc[t][h] = 0.0f;
#pragma unroll
            for (int k = 0; k < CD; ++k) {
                const int c = dli + LD * k;
                half2_t hw[DP][16];
#pragma unroll
                for (int h = 0; h < DP; ++h) {
                    u32x4 wv = st.w[h * CD + k];
                    asm volatile("" : "+v"(wv));     // decoded per group of pairs (as in gate/up)
                    e2m1x8_to_half(wv.x, hw[h] + 0);
                    e2m1x8_to_half(wv.y, hw[h] + 4);
                    e2m1x8_to_half(wv.z, hw[h] + 8);
                    e2m1x8_to_half(wv.w, hw[h] + 12);
                }
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    if (t < nt) {
                        const int pl = pg + t - q_lo;
                        const u32x4 a0 = q2h[(pl * 4 + 0) * CI + c], a1 = q2h[(pl * 4 + 1) * CI + c];
                        const u32x4 a2 = q2h[(pl * 4 + 2) * CI + c], a3 = q2h[(pl * 4 + 3) * CI + c];
#pragma unroll
                        for (int h = 0; h < DP; ++h)
                            acc[t][h] += ldexp_e8m0(block_dot(hw[h], a0, a1, a2, a3), st.sc[h * CD + k]);
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t < nt) {
                    const int p = rl.pair_src[pg + t];
                    const float coef = (p < P ? rl.w[p] : 1.0f) * s2l[pg + t - q_lo];
#pragma unroll
                    for (int h = 0; h < DP; ++h) {
                        const float d = group_sum<LD>(acc[t][h]);
                        if (dli == 0)
                            put_tagged(a.sync.y + (size_t)p * H + n + h * G::RP, tag_word(ep, coef * d));
                    }
                }
            }
        }
    };

    // 3./4. the wave's gate/up tasks, the next one's loads in flight; then
    //    its first down task's loads go out, to stream during the hand-off
    StageG g0, g1;
    StageD d0, d1;
    run(ng, g0, g1, issue_g, compute_g, false);
    if (nd > 0) issue_d(0, d0);

    // 5. the FP8 intermediate of this workgroup's down slots: a wave per pair
    //    waits for its h row, then requantises it (s2 = amax / 448, codes
    //    E4M3(h * fl32(1 / s2)), the requantisation kernel's arithmetic) into
    //    LDS as f16.  The workgroup that holds a slot's first down task writes
    //    the slot's intermediate taps.
    {
        using R = RequantRow<I>;
        _Float16* q16 = reinterpret_cast<_Float16*>(q2h);
        for (int pos = q_lo + wave; pos < q_hi; pos += NW) {
            const int p = rl.pair_src[pos], pl = pos - q_lo;
            const uint64_t* row = a.sync.h + (size_t)p * I + lane * R::PER;
            R rr;
            // first one word per gate/up task that writes this lane's rows
            // (a task writes G::RW consecutive rows), then the whole segment
            auto sentinels = [&]() {
                bool ok = true;
#pragma unroll
                for (int k = 0; k < R::PER; k += G::RW) ok &= has_tag(get_tagged(row + k), ep);
                return ok;
            };
            auto poll = [&]() {
                bool ok = true;
#pragma unroll
                for (int k = 0; k < R::PER; ++k) {
                    const uint64_t v = get_tagged(row + k);
                    rr.v[k] = tagged_value(v);
                    ok &= has_tag(v, ep);
                }
                return ok;
            };
            wave_wait(sentinels, wb, kWaitH, failed);
            wave_wait(poll, wb, kWaitH, failed);
            const float sc = rr.scale();
            uint32_t codes[R::NCODE];
            rr.encode(sc, codes);
            int slot = s_lo;
            while (slot < s_hi && rl.offsets[slot + 1] <= pos) ++slot;
            const bool tap = d_lo <= slot * G::DT && slot * G::DT < d_hi;
            const int k0 = lane * R::PER;
            if constexpr (R::PER % 4 == 0) {
#pragma unroll
                for (int c4 = 0; c4 < R::NCODE; ++c4) {
                    const int k = k0 + 4 * c4;
                    uint2 hv2;
                    hv2.x = e4m3x2_to_half2<false>(codes[c4]);
                    hv2.y = e4m3x2_to_half2<true>(codes[c4]);
                    *reinterpret_cast<uint2*>(q16 + ((pl * 4 + ((k & 31) >> 3)) * CI + (k >> 5)) * 8 + (k & 7)) = hv2;
                    if (tap && a.q2_tap != nullptr) reinterpret_cast<uint32_t*>(a.q2_tap + (size_t)p * I + k0)[c4] = codes[c4];
                }
            } else {
#pragma unroll
                for (int k1 = 0; k1 < R::NCODE; ++k1) {
                    const int k = k0 + k1;
                    q16[((pl * 4 + ((k & 31) >> 3)) * CI + (k >> 5)) * 8 + (k & 7)] = (_Float16)e4m3_decode(codes[k1]);
                    if (tap && a.q2_tap != nullptr) a.q2_tap[(size_t)p * I + k] = (uint8_t)codes[k1];
                }
            }
            if (lane == 0) {
                s2l[pl] = sc;
                if (tap && a.s2_tap != nullptr) a.s2_tap[p] = sc;
            }
        }
    }
    __syncthreads();

    // 6. the down tasks, the next one's loads in flight (the first is already out)
    run(nd, d0, d1, issue_d, compute_d, true);

    // 7. combine: this workgroup's output rows [n_lo, n_hi) of every token,
    //    the K selections in order, then the shared expert
    {
        const int n_lo = share_lo(H, b, NB), n_hi = share_lo(H, b + 1, NB);
        const int rows = n_hi - n_lo, total = M * rows;
        for (int base = wave * kWave; base < total; base += NW * kWave) {
            const int idx = min(base + lane, total - 1);
            const int t = idx / rows, n = n_lo + idx % rows;
            float v[kMaxTopK + 1];
            auto poll = [&]() {
                bool ok = true;
#pragma unroll
                for (int j = 0; j < kMaxTopK + 1; ++j) {
                    const bool use = j < K || (j == K && a.shared);
                    const int p = j < K ? t * K + j : P + t;
                    if (use) {
                        const uint64_t w = get_tagged(a.sync.y + (size_t)p * H + n);
                        v[j] = tagged_value(w);
                        ok &= has_tag(w, ep);
                    }
                }
                return ok;
            };
            wave_wait(poll, wb, kWaitY, failed);
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < kMaxTopK + 1; ++j)
                if (j < K || (j == K && a.shared)) s += v[j];
            if (base + lane < total) a.out[(size_t)t * H + n] = s;
        }
    }

    // 8. workgroup 0 moves the epoch on once every workgroup has arrived
    //    (so has read it); a later call then tags its words differently
    if (b == 0 && wave == 0) {
        auto poll = [&]() {
            bool ok = true;
            for (int w = lane; w < NB; w += kWave) ok &= has_tag(get_tagged(a.sync.arrive + w), ep);
            return ok;
        };
        wave_wait(poll, wb, kWaitArrive, failed);
        for (int w = lane; w < kMaxLayerBlocks; w += kWave)
            __hip_atomic_store(a.sync.epochs + w, ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) __hip_atomic_store(a.sync.word, ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace moe
