// moe_types.hpp -- constants, kernel argument blocks and shape geometry shared
// by the device code (compiled ahead of time by hipcc and at run time by
// hipRTC) and the host launchers.  Device-compilable under hipRTC: no host
// runtime headers.
#pragma once

#ifndef __HIPCC_RTC__
#include <hip/hip_runtime.h>
#endif
#include <stdint.h>

namespace moe {


// Largest token count of the GEMV path, and largest K / E it supports.
constexpr int kMaxGemvTokens = 8;
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 512;
constexpr int kMaxPairs = kMaxGemvTokens * kMaxTopK;
// With a shared expert every token adds one pair (row P + t of the
// intermediates) in one more slot, whose expert id is kSharedExpert.
constexpr int kMaxPairsExt = kMaxPairs + kMaxGemvTokens;
constexpr int kSharedExpert = -1;
// Largest token count of the chunk path (M > kMaxGemvTokens): its M*K pairs
// are sorted by expert in one workgroup's LDS.
constexpr int kMaxChunkTokens = 2048;
constexpr int kMaxChunkPairs = kMaxChunkTokens * kMaxTopK;

// The shared expert's weights (one expert of the routed layout), or all null.
struct SharedWeights {
    const uint8_t* w13;    // [2I,H/2]
    const uint8_t* s13;    // [2I,H/32]
    const uint8_t* w2;     // [H,I/2]
    const uint8_t* s2;     // [H,I/32]
};

// Token -> expert compaction as published in the workspace.
struct Compaction {
    int32_t* n_act;        // [1]
    int32_t* act_experts;  // [S] ascending expert ids
    int32_t* offsets;      // [S+1]
    int32_t* pair_token;   // [M*K]
    int32_t* pair_src;     // [M*K] original pair index t*K+j
};

struct RouterArgs {
    const uint16_t* x;     // [M,H] bf16
    const uint16_t* wr;    // [E,H] bf16
    int M, E;
    float* logits;         // [M,E]
    uint8_t* act_q;        // [M,H] or nullptr (no quantisation)
    float* act_s;          // [M]
};

// Routing source of a prologue: logits (top-K computed in the workgroup) or
// caller-given ids.
struct RouteSrc {
    int M, E, K;
    const float* logits;   // [M,E] or nullptr
    const int32_t* ids;    // [M,K] used when logits is nullptr
    int shared;            // 1: append the shared expert's slot
};

struct TopkArgs {
    RouteSrc src;
    int32_t* ids_out;      // [M,K]
    float* w_out;          // [M,K] (only with logits)
    Compaction cp;
};

struct GateUpArgs {
    RouteSrc src;          // logits (top-K in every workgroup) or caller ids
    int32_t* ids_out;      // [M,K] published by workgroup 0; may be nullptr
    float* w_out;          // [M,K]; may be nullptr
    Compaction cp;         // published by workgroup 0
    const uint8_t* w13;    // [E,2I,H/2]
    const uint8_t* s13;    // [E,2I,H/32]
    const uint8_t* act_q;  // [M,H]
    const float* act_s;    // [M]
    float* h;              // [M*K (+M),I]
    SharedWeights sh;      // read when the compaction holds the shared slot
    const uint16_t* x;     // [M,H] bf16, or nullptr.  When set (M <= 2; ignored
                           // by the kernels for more tokens), the kernel
                           // quantises x itself and act_q/act_s are unused
};

struct DownArgs {
    int E, M, K;
    const uint8_t* w2;     // [E,H,I/2]
    const uint8_t* sw2;    // [E,H,I/32]
    const float* h;        // [M*K,I] fp32, requantised in the kernel; or nullptr
    const uint8_t* q2;     // [M*K,I] E4M3 intermediate, used when h is nullptr
    const float* s2;       // [M*K]
    uint8_t* q2_out;       // optional: the requantised codes (workgroup 0 writes them)
    float* s2_out;         // optional: their scales
    const float* topk_w;   // [M*K]
    Compaction cp;         // read
    float* out;            // [M,H]
    SharedWeights sh;      // non-null w2: the compaction's last slot is the shared expert (weight 1)
};

struct RequantArgs {
    const float* h;        // [P,I]
    int P;
    uint8_t* q2;           // [P,I]
    float* s2;             // [P]
};

// Chunk path (M > kMaxGemvTokens): grouped contractions over the expert-sorted
// pairs.  "Sorted position" pos indexes the pairs in (expert, pair index)
// order, as in Compaction; pos_of[p] is the sorted position of pair p.
struct ChunkRouterArgs {
    const uint16_t* x;     // [M,H] bf16
    const uint16_t* wr;    // [E,H] bf16
    int M, E;
    float* logits;         // [M,E]
};

// Chunk top-K, and with act_q the tokens' FP8 quantisation too (a token's
// wave holds its whole row: H <= kTopkQuantMaxH).
constexpr int kTopkQuantMaxH = 4096;
struct ChunkTopkArgs {
    const float* logits;   // [M,E]
    int M, E, K;
    int32_t* ids;          // [M,K]
    float* w;              // [M,K]
    const uint16_t* x;     // [M,H] bf16 hidden states (read only with act_q)
    int H;
    uint8_t* act_q;        // [M,H] E4M3 codes, or null: no quantisation here
    float* act_s;          // [M] scales
};

// Work list of the grouped kernels: the sorted rows of each active expert
// as chunks, larger chunks first.  An expert with at most kChunkRows rows is
// one chunk (1-4 tiles of 16 rows); a busier one is cut evenly into chunks of
// at most kBigChunkRows rows, so that a workgroup reads its rows' weights
// once for up to 16 tiles of tokens instead of once per 64 tokens.
constexpr int kChunkRows = 64;
constexpr int kBigChunkRows = 256;

struct ChunkList {
    int32_t* n_chunks;     // [1]
    int4* rec;             // [C] {expert, first sorted position, rows, 0}; rows = 0 past the last chunk
    int C;                 // entries of rec (chunk_bound)
};

// chunks of S active experts over P rows: at most one per expert plus one
// per kChunkRows rows of the busy ones
__host__ __device__ constexpr int chunk_bound(int S, int P) { return S + (P + kChunkRows - 1) / kChunkRows; }

struct SortArgs {
    const int32_t* ids;    // [M,K]; out-of-range ids are clamped into [0, E)
    int M, K, E;
    Compaction cp;         // written
    int32_t* pos_of;       // [M*K (+M)]
    ChunkList chunks;      // written
    int shared;            // 1: the shared expert's M rows follow as one more slot
};

struct ChunkGateUpArgs {
    Compaction cp;         // read
    ChunkList chunks;      // read
    const uint8_t* w13;    // [E,2I,H/2]
    const uint8_t* s13;    // [E,2I,H/32]
    const uint8_t* act_q;  // [M,H]
    const float* act_s;    // [M]
    float* h;              // [M*K (+M),I] in sorted order
    SharedWeights sh;
};

struct ChunkDownArgs {
    Compaction cp;         // read
    ChunkList chunks;      // read
    const uint8_t* w2;     // [E,H,I/2]
    const uint8_t* sw2;    // [E,H,I/32]
    const uint8_t* q2;     // [M*K,I] E4M3 intermediate
    const float* s2;       // [M*K]
    int by_pair;           // 0: q2/s2 rows in sorted order; 1: in pair order
    float* y;              // [M*K (+M),H] expert outputs (s2 applied) in sorted order
    SharedWeights sh;
};

struct CombineArgs {
    const float* y;        // [M*K,H] sorted order
    const int32_t* pos_of; // [M*K]
    const float* w;        // [M*K] router weights in pair order
    int M, K;
    float* out;            // [M,H]
    int shared;            // 1: add the shared expert's row y[pos_of[M*K + t]] (weight 1)
};

// The one-kernel decode layer (M <= kMaxGemvTokens).  Its workgroups hand
// results to each other through epoch-tagged 64-bit words in the workspace:
// the high half holds the tag of the call that wrote the word (the epoch read
// at the call's start, plus one), the low half the fp32 value.  Each word is
// written and read whole by relaxed device-scope atomics, so a reader that
// sees its own call's tag has the value, with no fences.  The region is
// zeroed once by moe_workspace_init; its layout does not depend on M.
struct LayerSync {
    uint32_t* word;        // [0] epoch of the last call, [1] sticky error bits
    uint32_t* epochs;      // [kMaxLayerBlocks] the epoch again, one copy per workgroup slot
    uint64_t* arrive;      // [kMaxLayerBlocks] one word per workgroup
    uint64_t* logits;      // [kMaxGemvTokens, E]
    uint64_t* h;           // [kMaxPairsExt, I] gate/up output, pair order
    uint64_t* y;           // [kMaxPairsExt, H] weighted down output, pair order
};
constexpr int kMaxLayerBlocks = 1024;
// error bits of LayerSync::word[1] (a bounded wait ran out)
enum : uint32_t { kWaitLogits = 1u, kWaitH = 2u, kWaitY = 4u, kWaitArrive = 8u };

struct LayerArgs {
    // routed from x and wr (x != nullptr), or from the caller's ids, weights
    // and FP8 activations
    const uint16_t* x;     // [M,H] bf16
    const uint16_t* wr;    // [E,H] bf16
    const uint8_t* act_q;  // [M,H] E4M3 (x == nullptr)
    const float* act_s;    // [M]
    const int32_t* ids;    // [M,K] (x == nullptr), clamped into [0, E)
    const float* topk_w;   // [M,K]
    int M, E, K, shared;
    const uint8_t* w13;    // [E,2I,H/2]
    const uint8_t* s13;    // [E,2I,H/32]
    const uint8_t* w2;     // [E,H,I/2]
    const uint8_t* sw2;    // [E,H,I/32]
    SharedWeights sh;
    float* out;            // [M,H]
    // optional taps in pair order (rows M*K + t: the shared expert)
    float* h_tap;          // [M*K (+M),I]
    uint8_t* q2_tap;       // [M*K (+M),I]
    float* s2_tap;         // [M*K (+M)]
    int32_t* ids_out;      // [M,K] routed ids (x != nullptr)
    float* w_out;          // [M,K] their weights
    LayerSync sync;
    uint64_t wait_ticks;   // bound of every wait, in s_memrealtime ticks
};

// ---------------------------------------------------------------------------
// Shape geometry, as constexpr functions so that the kernel templates and the
// host launchers (which also launch kernels compiled at run time for shapes
// known only then) compute the same blocking.
// ---------------------------------------------------------------------------
constexpr int kWaveSize = 64;

// Router GEMV: one workgroup per expert row, one thread per 16-byte chunk
// (8 bf16) of the row, rounded up to whole waves.
__host__ __device__ constexpr int router_threads(int H) { return ((H / 8 + kWaveSize - 1) / kWaveSize) * kWaveSize; }

// gate/up GEMV: H/32 chunks of 16 code bytes per row, LPR lanes per row.
__host__ __device__ constexpr int gate_up_lanes_per_row(int H)
{
    return ((H / 32) % 16 == 0) ? 16 : ((H / 32) % 8 == 0) ? 8 : ((H / 32) % 4 == 0) ? 4 : ((H / 32) % 2 == 0) ? 2 : 1;
}
__host__ __device__ constexpr int gate_up_rows_per_block(int H) { return (kWaveSize / gate_up_lanes_per_row(H)) * 4; }

// down GEMV: a workgroup owns RPB output rows.  A wave covers those rows of
// one expert in RP passes of RPW = RPB / RP rows, LPR lanes per row (each lane
// holds I/32/LPR of a row's 32-element blocks per pass), so that one load
// instruction reads LPR * 16 contiguous bytes of each of RPW rows.  The
// workgroups are all resident at once (8 waves each), so the grid H / RPB is
// kept at or below the chip's 256 compute units where the shape allows: a
// grid above it puts two workgroups on some compute units, and those finish
// last.  RPB is the smallest divisor of H giving such a grid for which some
// RP (the smallest) has LPR a multiple of 4 (whole 64-byte pieces per
// instruction, or the whole row), at most 4 blocks per lane and at least half
// the wave busy.  Other shapes take one pass of 64 / LPR rows with the
// largest power-of-two LPR (up to 8) dividing I/32.
constexpr int kComputeUnits = 256;
constexpr int kDownMaxBlocksPerLane = 4;
__host__ __device__ constexpr int down_lanes_for_rows(int I, int rpw)
{
    int l = kWaveSize / rpw;
    while (l > 1 && (I / 32) % l != 0) --l;
    return l;
}
__host__ __device__ constexpr bool down_blocking_ok(int I, int rpb, int rp)
{
    if (rpb % rp != 0 || rpb / rp > kWaveSize) return false;
    const int rpw = rpb / rp, l = down_lanes_for_rows(I, rpw), c = I / 32;
    return (c / l) * rp <= kDownMaxBlocksPerLane && 2 * l * rpw >= kWaveSize && (l % 4 == 0 || l == c);
}
constexpr int kDownMaxPasses = 4;
__host__ __device__ constexpr int down_rows_per_block(int H, int I)
{
    for (int r = (H + kComputeUnits - 1) / kComputeUnits; r <= kWaveSize * kDownMaxPasses; ++r) {
        if (H % r != 0) continue;
        for (int rp = 1; rp <= kDownMaxPasses; ++rp)
            if (down_blocking_ok(I, r, rp)) return r;
    }
    const int c = I / 32;
    return kWaveSize / ((c % 8 == 0) ? 8 : (c % 4 == 0) ? 4 : (c % 2 == 0) ? 2 : 1);
}
__host__ __device__ constexpr int down_row_passes(int H, int I)
{
    const int r = down_rows_per_block(H, I);
    for (int rp = 1; rp <= kDownMaxPasses; ++rp)
        if (down_blocking_ok(I, r, rp)) return rp;
    return 1;
}
__host__ __device__ constexpr int down_lanes_per_row(int H, int I)
{
    return down_lanes_for_rows(I, down_rows_per_block(H, I) / down_row_passes(H, I));
}

// The decode (GEMV) path's kernels exist for (H, I) when these hold (the
// kernels' own static checks repeat them).
__host__ __device__ constexpr bool gemv_shape_ok(int H, int I)
{
    return H >= 256 && H <= 8192 && H % 32 == 0 && I >= 64 && I <= 4096 && I % kWaveSize == 0 &&
           I % gate_up_rows_per_block(H) == 0 && H % down_rows_per_block(H, I) == 0;
}

// One-kernel decode layer blocking.  A gate/up task is one wave's share of
// one slot: 64 / LPR row pairs (gate row r and up row I + r), LPR lanes per
// row, each lane CPL blocks of 32 (the gate/up GEMV geometry above).  A down
// task is one wave's share of one slot: DP passes of 64 / LD output rows, LD
// lanes per row, each lane CD blocks of 32 per pass; LD is the largest power
// of two up to 16 dividing I / 32.  Tasks are dealt out to the workgroups in
// equal contiguous ranges (slot-major), and to a workgroup's 8 waves in turn.
__host__ __device__ constexpr int layer_down_lanes(int I)
{
    return ((I / 32) % 16 == 0) ? 16 : ((I / 32) % 8 == 0) ? 8 : ((I / 32) % 4 == 0) ? 4 : ((I / 32) % 2 == 0) ? 2 : 1;
}
__host__ __device__ constexpr int layer_down_blocks(int I) { return (I / 32) / layer_down_lanes(I); }
__host__ __device__ constexpr int layer_down_rows_per_pass(int I) { return kWaveSize / layer_down_lanes(I); }
__host__ __device__ constexpr int layer_down_passes(int H, int I)
{
    return (layer_down_blocks(I) <= 3 && H % (2 * layer_down_rows_per_pass(I)) == 0) ? 2 : 1;
}
__host__ __device__ constexpr int layer_gate_up_tasks(int H, int I) { return I / (kWaveSize / gate_up_lanes_per_row(H)); }
__host__ __device__ constexpr int layer_down_tasks(int H, int I)
{
    return H / (layer_down_rows_per_pass(I) * layer_down_passes(H, I));
}
constexpr int kLayerWaves = 8;
// Dynamic LDS of the layer kernel: every token's activations as f16, then the
// FP8 intermediate (as f16) of the nq pairs of a workgroup's down slots.
__host__ __device__ constexpr size_t layer_lds_bytes(int H, int I, int mt, int nq)
{
    return (size_t)mt * H * 2 + (size_t)nq * I * 2;
}
// The one-kernel layer exists for (H, I) when its register plan holds: at most
// 5 gate/up blocks and 6 down blocks per lane and task.
__host__ __device__ constexpr bool layer_shape_ok(int H, int I)
{
    return gemv_shape_ok(H, I) && (H / 32) / gate_up_lanes_per_row(H) <= 5 &&
           layer_down_blocks(I) * layer_down_passes(H, I) <= 6 && H % (layer_down_rows_per_pass(I) * layer_down_passes(H, I)) == 0;
}

// Chunk path blocking: 16-row MFMA tiles, chunks of up to 64 rows (256 for a
// busy expert), 32 gate/up rows and
// 256 down rows per workgroup (4 waves x kDnNJ = 4 n-tiles of 16 rows), router
// K slices of H/8.  The chunk path therefore needs H % 256 == 0.
constexpr int kGuNJ = 2;                                // 16-row n-tiles per wave and matrix
constexpr int kGuRows = 16 * kGuNJ;
constexpr int kDnNJ = 4;
constexpr int kDnRows = 4 * 16 * kDnNJ;                 // 4 waves x NJ n-tiles x 16 rows
constexpr int kRouterWaves = 8;

__host__ __device__ constexpr int chunk_k_steps(int H) { return H / 128; }
__host__ __device__ constexpr int chunk_k_split(int H) { return chunk_k_steps(H) >= 4 ? 4 : chunk_k_steps(H); }

__host__ __device__ constexpr bool chunk_shape_ok(int H, int I)
{
    return gemv_shape_ok(H, I) && H % (kRouterWaves * 32) == 0 && H % 128 == 0 &&
           chunk_k_steps(H) % chunk_k_split(H) == 0 && I % kGuRows == 0 && (kGuRows * (H / 32)) % 16 == 0 &&
           H % kDnRows == 0 && I % 32 == 0;
}

// FP8 LM-head GEMV: 16 lanes per row, each taking 16-code chunks; the
// activations of up to 8 tokens stay in LDS (16 H bytes).
__host__ __device__ constexpr bool lm_head_shape_ok(int H) { return H >= 256 && H <= 4096 && H % 256 == 0; }

}  // namespace moe
