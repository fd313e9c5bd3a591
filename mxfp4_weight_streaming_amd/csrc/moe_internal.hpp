// moe_internal.hpp -- host side of the library: workspace layout, launch
// events and the launcher declarations shared by the kernels' launch code and
// the C ABI (moe_api.hip).  Not installed; the public interface is
// include/moe_decode.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

#include "moe_types.hpp"

namespace moe {

// Dynamic LDS a kernel may take on gfx950 (160 KiB per compute unit).
constexpr size_t kMaxDynamicLds = 160 * 1024;
// The layer kernel: at least this much LDS, so that a compute unit holds one
// of its workgroups; at most what leaves room for its static LDS.
constexpr size_t kLayerMinLds = 84 * 1024;
constexpr size_t kLayerMaxDynLds = 152 * 1024;

// Workspace carving.  The one-kernel layer's hand-off region (LayerSync)
// comes first and its layout does not depend on M: its epoch and tags carry
// over from call to call (moe_workspace_init zeroes them once).  Everything
// after it is written by a call before that call reads it.  pos_of and y
// exist only for the chunk path.
struct WsLayout {
    size_t sync_word, sync_epochs, sync_arrive, sync_logits, sync_h, sync_y;
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
    L.sync_word = take(256);
    L.sync_epochs = take((size_t)kMaxLayerBlocks * 4);
    L.sync_arrive = take((size_t)kMaxLayerBlocks * 8);
    L.sync_logits = take((size_t)kMaxGemvTokens * E * 8);
    L.sync_h = take((size_t)kMaxPairsExt * I * 8);
    L.sync_y = take((size_t)kMaxPairsExt * H * 8);
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

// Launchers (moe_kernels.hip).  Each returns the hipError_t of its launch
// (hipErrorInvalidDeviceFunction when the shape has no kernel: neither
// compiled in nor loaded at run time).  mt is the token bound the kernels are
// instantiated for (1, 2, 4 or 8).
bool gemv_shape_supported(int H, int I);
hipError_t launch_router(int H, int mt, const RouterArgs& a, hipStream_t s, const LaunchEvents& ev = {});
hipError_t launch_quant(int H, const uint16_t* x, int M, uint8_t* q, float* sc, hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
hipError_t launch_gate_up(int H, int I, int mt, int S, const GateUpArgs& a, hipStream_t s,
                          const LaunchEvents& ev = {});  // S: slot bound
hipError_t launch_down(int H, int I, int mt, const DownArgs& a, hipStream_t s, const LaunchEvents& ev = {});
// The one-kernel layer (M <= 8); a.wait_ticks is filled in here when zero.
bool layer_shape_supported(int H, int I);
hipError_t launch_layer(int H, int I, int mt, LayerArgs a, hipStream_t s, const LaunchEvents& ev = {});
// Bound of the layer kernel's waits, in microseconds (0: the default).
void set_layer_wait_us(uint32_t us);
hipError_t launch_requant(int I, const RequantArgs& a, hipStream_t s);
hipError_t launch_fp8_encode_range(uint32_t first, int64_t n, uint8_t* q, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s);
void kernel_names(int H, int I, char* buf, size_t n);
void layer_kernel_names(int H, int I, char* buf, size_t n);

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
void chunk_kernel_names(int H, int I, char* buf, size_t n);

// FP8 LM head (lm_head.hip).  mt is the token bound (1, 2, 4 or 8).
bool lm_head_shape_supported(int H);
hipError_t launch_lm_head_quant(const uint16_t* w, int V, int H, uint8_t* q, float* scale, hipStream_t s);
hipError_t launch_lm_head_gemv(int H, int mt, const uint16_t* x, int M, const uint8_t* q, const float* scale, int V,
                               float* logits, hipStream_t s);

// Run-time compilation of the shape-templated kernels (jit.hip).
enum class JitStatus { Ok, BadShape, BadArch, CacheIo, Compile, Load };
struct JitReport {
    bool from_cache = false;   // the code object came from the cache file
    bool chunk = false;        // the module holds the chunk-path kernels
    bool lm_head = false;      // ... and the LM-head GEMV for this H
    int kernels = 0;
    double seconds = 0.0;
    char file[1024] = "";
};
// Compile (or find in the cache) the kernels of (H, I) for `arch`; no device needed.
JitStatus jit_build(int H, int I, const char* arch, const char* cache_dir, JitReport* rep, std::string* err);
// The same for the current device, then load them on it.  prefer: use them
// even where a compiled-in kernel exists.
JitStatus jit_load(int H, int I, const char* cache_dir, bool prefer, JitReport* rep, std::string* err);
// Unload (H, I) from the current device; returns the number of modules removed.
int jit_unload(int H, int I);

}  // namespace moe
