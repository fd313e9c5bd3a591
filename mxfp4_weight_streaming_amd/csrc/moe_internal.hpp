// moe_internal.hpp -- kernel argument blocks, workspace layout and launcher
// declarations shared by the kernels (moe_kernels.hip) and the C ABI
// (moe_api.hip).  Not installed; the public interface is include/moe_decode.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
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

struct ChunkTopkArgs {
    const float* logits;   // [M,E]
    int M, E, K;
    int32_t* ids;          // [M,K]
    float* w;              // [M,K]
};

// Work list of the grouped kernels: the sorted rows of each active expert
// cut into chunks of at most kChunkRows rows, larger chunks first.
constexpr int kChunkRows = 64;

struct ChunkList {
    int32_t* n_chunks;     // [1]
    int4* rec;             // [C] {expert, first sorted position, rows, 0}; rows = 0 past the last chunk
    int C;                 // entries of rec (chunk_bound)
};

inline int chunk_bound(int S, int P) { return S + (P + kChunkRows - 1) / kChunkRows; }

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

// Workspace carving.  No state is carried between calls: every call writes
// what it later reads.  pos_of and y exist only for the chunk path.
struct WsLayout {
    size_t logits, ids, w, act_q, act_s, n_act, act_experts, offsets, pair_token, pair_src, h, q2, s2, pos_of, y,
        n_chunks, chunk_rec, total;
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

inline WsLayout ws_layout(int H, int I, int E, int K, int M)
{
    // room for a shared expert is always kept: one more slot and M more pairs
    WsLayout L{};
    const size_t P = (size_t)M * K;
    const size_t Pe = P + (size_t)M;
    const size_t S = (size_t)(E < (int)P ? E : (int)P) + 1;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    L.logits = take((size_t)M * E * 4);
    L.ids = take(P * 4);
    L.w = take(P * 4);
    L.act_q = take((size_t)M * H);
    L.act_s = take((size_t)M * 4);
    L.n_act = take(4);
    L.act_experts = take(S * 4);
    L.offsets = take((S + 1) * 4);
    L.pair_token = take(Pe * 4);
    L.pair_src = take(Pe * 4);
    L.h = take(Pe * I * 4);
    L.q2 = take(Pe * I);
    L.s2 = take(Pe * 4);
    const bool chunk = M > kMaxGemvTokens;
    L.pos_of = take(chunk ? Pe * 4 : 0);
    L.y = take(chunk ? Pe * (size_t)H * 4 : 0);
    const size_t C = chunk ? (size_t)chunk_bound((int)S, (int)Pe) : 0;
    L.n_chunks = take(chunk ? 4 : 0);
    L.chunk_rec = take(C * 16);
    L.total = off;
    return L;
}

// Optional start/stop events of one kernel launch.  When either is set the
// kernel goes through hipExtLaunchKernel, which stamps the events with the
// kernel's own start and end on the GPU (no queueing or dispatch gaps).
struct LaunchEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};

// Launchers (moe_kernels.hip).  Each returns the hipError_t of its launch.
// mt is the token bound the kernels are instantiated for (1, 2, 4 or 8).
bool gemv_shape_supported(int H, int I);
hipError_t launch_router(int H, int mt, const RouterArgs& a, hipStream_t s, const LaunchEvents& ev = {});
hipError_t launch_quant(int H, const uint16_t* x, int M, uint8_t* q, float* sc, hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
hipError_t launch_gate_up(int H, int I, int mt, int S, const GateUpArgs& a, hipStream_t s,
                          const LaunchEvents& ev = {});  // S: slot bound
hipError_t launch_down(int H, int I, int mt, const DownArgs& a, hipStream_t s, const LaunchEvents& ev = {});
hipError_t launch_requant(int I, const RequantArgs& a, hipStream_t s);
hipError_t launch_fp8_encode_range(uint32_t first, int64_t n, uint8_t* q, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s);
const char* kernel_names(int H, int I, int mt);

// Chunk-path launchers (moe_chunk.hip).
bool chunk_shape_supported(int H, int I, int E);
hipError_t launch_chunk_router(int H, const ChunkRouterArgs& a, hipStream_t s, const LaunchEvents& ev = {});
hipError_t launch_chunk_topk(const ChunkTopkArgs& a, hipStream_t s, const LaunchEvents& ev = {});
hipError_t launch_sort_pairs(const SortArgs& a, hipStream_t s, const LaunchEvents& ev = {});
// C is the chunk bound chunk_bound(S, M*K).
hipError_t launch_chunk_gate_up(int H, int I, int C, const ChunkGateUpArgs& a, hipStream_t s,
                                const LaunchEvents& ev = {});
hipError_t launch_chunk_down(int H, int I, int C, const ChunkDownArgs& a, hipStream_t s, const LaunchEvents& ev = {});
hipError_t launch_combine(int H, const CombineArgs& a, hipStream_t s, const LaunchEvents& ev = {});
hipError_t launch_gather_rows(const void* src, void* dst, const int32_t* pos_of, int P, int row_bytes, hipStream_t s);
const char* chunk_kernel_names(int H, int I);

// FP8 LM head (lm_head.hip).  mt is the token bound (1, 2, 4 or 8).
bool lm_head_shape_supported(int H);
hipError_t launch_lm_head_quant(const uint16_t* w, int V, int H, uint8_t* q, float* scale, hipStream_t s);
hipError_t launch_lm_head_gemv(int H, int mt, const uint16_t* x, int M, const uint8_t* q, const float* scale, int V,
                               float* logits, hipStream_t s);

}  // namespace moe
