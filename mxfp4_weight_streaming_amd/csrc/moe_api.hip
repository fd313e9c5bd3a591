// moe_api.hip -- the C ABI declared in include/moe_decode.h: argument
// validation, workspace carving and launch ordering on the caller's stream.
// Nothing here allocates, frees or synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "moe_decode.h"
#include "moe_internal.hpp"

namespace {

thread_local char g_last_error[4096] = "";

moe_status fail(moe_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status fail(moe_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

moe_status hip_fail(hipError_t err, const char* what)
{
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int token_bound(int M)
{
    int mt = 1;
    while (mt < M) mt <<= 1;
    return mt;
}

// M above the GEMV bound takes the chunk path (grouped MFMA contractions).
bool chunked(int32_t M) { return M > moe::kMaxGemvTokens; }

// Shape checks shared by every entry point.
moe_status check_shape(const moe_shape* s, int32_t M)
{
    if (s == nullptr) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
    if (s->hidden <= 0 || s->inter <= 0 || s->num_experts <= 0 || s->topk <= 0)
        return fail(MOE_ERR_INVALID_ARG, "shape has a non-positive size (H=%d I=%d E=%d K=%d)",
                    s->hidden, s->inter, s->num_experts, s->topk);
    if (s->hidden % 32 != 0 || s->inter % 32 != 0)
        return fail(MOE_ERR_INVALID_ARG, "H (%d) and I (%d) must be multiples of the MX block size 32",
                    s->hidden, s->inter);
    if (s->topk > s->num_experts)
        return fail(MOE_ERR_INVALID_ARG, "K (%d) exceeds E (%d)", s->topk, s->num_experts);
    if (M <= 0) return fail(MOE_ERR_INVALID_ARG, "M (%d) must be positive", M);
    if (s->topk > moe::kMaxTopK)
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "K (%d) above %d is not compiled", s->topk, moe::kMaxTopK);
    if (s->num_experts > moe::kMaxExperts)
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "E (%d) above %d is not compiled", s->num_experts, moe::kMaxExperts);
    if (!moe::gemv_shape_supported(s->hidden, s->inter))
        return fail(MOE_ERR_UNSUPPORTED_SHAPE,
                    "(H=%d, I=%d) has no kernels on this device: compiled in are (256,64) and (2560,768); other "
                    "shapes need moe_jit_load first",
                    s->hidden, s->inter);
    if (M > moe::kMaxChunkTokens)
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "M=%d above %d tokens is not compiled", M, moe::kMaxChunkTokens);
    if (!chunked(M) && (size_t)(M * s->topk + M) * s->inter * 2 > moe::kMaxDynamicLds)
        return fail(MOE_ERR_UNSUPPORTED_SHAPE,
                    "the down kernel holds the %d x %d FP8 intermediate rows of M=%d tokens in LDS as f16 (%zu "
                    "bytes), above the %zu a workgroup can have",
                    M * s->topk + M, s->inter, M, (size_t)(M * s->topk + M) * s->inter * 2, moe::kMaxDynamicLds);
    if (M > moe::kMaxGemvTokens && s->num_experts % 16 != 0)
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "the chunk path (M > %d) needs E %% 16 == 0 (E=%d)",
                    moe::kMaxGemvTokens, s->num_experts);
    if (M > moe::kMaxGemvTokens && !moe::chunk_shape_supported(s->hidden, s->inter, s->num_experts))
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "(H=%d, I=%d) has no chunk-path kernels (M > %d)", s->hidden, s->inter,
                    moe::kMaxGemvTokens);
    return MOE_OK;
}

moe_status check_ws(const moe_shape* s, int32_t M, void* ws, size_t ws_bytes)
{
    if (ws == nullptr) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
    if (((uintptr_t)ws & 255u) != 0) return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    const size_t need = moe::ws_layout(s->hidden, s->inter, s->num_experts, s->topk, M).total;
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed for M=%d", ws_bytes, need, M);
    return MOE_OK;
}

#define CHECK_PTR(p)                                                             \
    do {                                                                         \
        if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", #p);  \
    } while (0)
#define CHECK_ALIGN(p)                                                                         \
    do {                                                                                       \
        if (!aligned16(p)) return fail(MOE_ERR_ALIGNMENT, "%s is not 16-byte aligned", #p);    \
    } while (0)

struct Carved {
    moe::WsLayout L;
    char* base;
    template <typename T> T* at(size_t off) const { return reinterpret_cast<T*>(base + off); }
    moe::Compaction cp() const
    {
        return {at<int32_t>(L.n_act), at<int32_t>(L.act_experts), at<int32_t>(L.offsets),
                at<int32_t>(L.pair_token), at<int32_t>(L.pair_src)};
    }
    // The chunk list's capacity; with a shared expert, one more slot of M rows.
    static int chunk_cap(const moe_shape* s, int32_t M, bool shared)
    {
        const int P = M * s->topk, S = s->num_experts < P ? s->num_experts : P;
        return shared ? moe::chunk_bound(S + 1, P + M) : moe::chunk_bound(S, P);
    }
    moe::ChunkList chunks(const moe_shape* s, int32_t M, bool shared) const
    {
        return {at<int32_t>(L.n_chunks), at<int4>(L.chunk_rec), chunk_cap(s, M, shared)};
    }
    moe::LayerSync sync() const
    {
        return {at<uint32_t>(L.sync_word), at<uint32_t>(L.sync_epochs), at<uint64_t>(L.sync_arrive),
                at<uint64_t>(L.sync_logits), at<uint64_t>(L.sync_h), at<uint64_t>(L.sync_y)};
    }
};

Carved carve(const moe_shape* s, int32_t M, void* ws)
{
    return {moe::ws_layout(s->hidden, s->inter, s->num_experts, s->topk, M), static_cast<char*>(ws)};
}

int num_slots(const moe_shape* s, int32_t M)
{
    const int P = M * s->topk;
    return s->num_experts < P ? s->num_experts : P;
}

// The shared expert's weights as the kernels take them (all null: none).
moe::SharedWeights shared_weights(const moe_shared_expert* sh)
{
    if (sh == nullptr) return {};
    return {sh->w13, sh->w13_scale, sh->w2, sh->w2_scale};
}

bool has_shared(const moe::SharedWeights& sh) { return sh.w13 != nullptr; }

// Intermediate rows of a call: M*K routed pairs, then M shared-expert rows.
int pair_rows(const moe_shape* s, int32_t M, const moe::SharedWeights& sh)
{
    return M * s->topk + (has_shared(sh) ? M : 0);
}

moe_status enqueue_router(const moe_shape* s, int32_t M, const uint16_t* x, const uint16_t* wr, uint8_t* act_q,
                          float* act_s, const Carved& c, hipStream_t st, const moe::LaunchEvents& ev = {})
{
    moe::RouterArgs a{x, wr, M, s->num_experts, c.at<float>(c.L.logits), act_q, act_s};
    hipError_t e = moe::launch_router(s->hidden, token_bound(M), a, st, ev);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "router launch");
}

// Top-K and compaction in one workgroup, from the logits in the workspace or
// from caller-given ids.
moe_status enqueue_topk(const moe_shape* s, int32_t M, bool from_logits, const int32_t* ids, int32_t* ids_out,
                        float* w_out, const Carved& c, hipStream_t st)
{
    moe::TopkArgs a{{M, s->num_experts, s->topk, from_logits ? c.at<float>(c.L.logits) : nullptr, ids}, ids_out,
                    w_out, c.cp()};
    hipError_t e = moe::launch_topk(a, st);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "topk launch");
}

// The gate/up kernel routes from the workspace logits (ids == nullptr) or
// from caller-given ids.
moe_status enqueue_gate_up(const moe_shape* s, int32_t M, const int32_t* ids, int32_t* ids_out, float* w_out,
                           const uint8_t* act_q, const float* act_s, const uint8_t* w13, const uint8_t* s13, float* h,
                           const Carved& c, hipStream_t st, const moe::LaunchEvents& ev = {},
                           const moe::SharedWeights& sh = {}, const uint16_t* x = nullptr)
{
    const int shared = has_shared(sh) ? 1 : 0;
    const moe::RouteSrc src{M, s->num_experts, s->topk, ids == nullptr ? c.at<float>(c.L.logits) : nullptr, ids,
                            shared};
    moe::GateUpArgs a{src, ids_out, w_out, c.cp(), w13, s13, act_q, act_s, h, sh, x};
    hipError_t e = moe::launch_gate_up(s->hidden, s->inter, token_bound(M), num_slots(s, M) + shared, a, st, ev);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "gate_up launch");
}

moe_status enqueue_requant(const moe_shape* s, int32_t rows, const float* h, uint8_t* q2, float* s2, hipStream_t st)
{
    moe::RequantArgs a{h, rows, q2, s2};
    hipError_t e = moe::launch_requant(s->inter, a, st);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "requant launch");
}

// From h (requantised in the kernel; q2_out/s2_out optional taps) or from a
// caller's E4M3 intermediate q2/s2.
moe_status enqueue_down(const moe_shape* s, int32_t M, const float* h, const uint8_t* q2, const float* s2,
                        uint8_t* q2_out, float* s2_out, const float* topk_w, const uint8_t* w2, const uint8_t* sw2,
                        float* out, const Carved& c, hipStream_t st, const moe::LaunchEvents& ev = {},
                        const moe::SharedWeights& sh = {})
{
    moe::DownArgs a{s->num_experts, M, s->topk, w2, sw2, h, q2, s2, q2_out, s2_out, topk_w, c.cp(), out, sh};
    hipError_t e = moe::launch_down(s->hidden, s->inter, token_bound(M), a, st, ev);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "down launch");
}

// ---- chunk path ----------------------------------------------------------
moe_status enqueue_chunk_router(const moe_shape* s, int32_t M, const uint16_t* x, const uint16_t* wr, const Carved& c,
                                hipStream_t st, const moe::LaunchEvents& ev = {})
{
    moe::ChunkRouterArgs a{x, wr, M, s->num_experts, c.at<float>(c.L.logits)};
    hipError_t e = moe::launch_chunk_router(s->hidden, a, st, ev);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "chunk router launch");
}

moe_status enqueue_quant(const moe_shape* s, int32_t M, const uint16_t* x, uint8_t* q, float* sc, hipStream_t st)
{
    hipError_t e = moe::launch_quant(s->hidden, x, M, q, sc, st);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "quant launch");
}

// Top-K of a chunk; with act_q, the tokens' FP8 quantisation in the same
// kernel where a wave holds a token's row (H <= kTopkQuantMaxH), otherwise
// in quant_kernel before it.
moe_status enqueue_chunk_topk(const moe_shape* s, int32_t M, int32_t* ids, float* w, const Carved& c, hipStream_t st,
                              const uint16_t* x = nullptr, uint8_t* act_q = nullptr, float* act_s = nullptr)
{
    const bool fused = act_q != nullptr && s->hidden <= moe::kTopkQuantMaxH;
    if (act_q != nullptr && !fused) {
        const hipError_t e = moe::launch_quant(s->hidden, x, M, act_q, act_s, st);
        if (e != hipSuccess) return hip_fail(e, "quant launch");
    }
    moe::ChunkTopkArgs a{c.at<float>(c.L.logits), M, s->num_experts, s->topk, ids, w,
                         x, s->hidden, fused ? act_q : nullptr, act_s};
    hipError_t e = moe::launch_chunk_topk(a, st);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "chunk topk launch");
}

moe_status enqueue_sort(const moe_shape* s, int32_t M, const int32_t* ids, const Carved& c, hipStream_t st,
                        bool shared = false)
{
    moe::SortArgs a{ids, M, s->topk, s->num_experts, c.cp(), c.at<int32_t>(c.L.pos_of), c.chunks(s, M, shared),
                    shared ? 1 : 0};
    hipError_t e = moe::launch_sort_pairs(a, st);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "pair sort launch");
}

moe_status enqueue_chunk_gate_up(const moe_shape* s, int32_t M, const uint8_t* act_q, const float* act_s,
                                 const uint8_t* w13, const uint8_t* s13, const Carved& c, hipStream_t st,
                                 const moe::LaunchEvents& ev = {}, const moe::SharedWeights& sh = {})
{
    const moe::ChunkList cl = c.chunks(s, M, has_shared(sh));
    moe::ChunkGateUpArgs a{c.cp(), cl, w13, s13, act_q, act_s, c.at<float>(c.L.h), sh};
    hipError_t e = moe::launch_chunk_gate_up(s->hidden, s->inter, cl.C, a, st, ev);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "chunk gate_up launch");
}

moe_status enqueue_chunk_down(const moe_shape* s, int32_t M, const uint8_t* q2, const float* s2, bool by_pair,
                              const uint8_t* w2, const uint8_t* sw2, const Carved& c, hipStream_t st,
                              const moe::LaunchEvents& ev = {}, const moe::SharedWeights& sh = {})
{
    const moe::ChunkList cl = c.chunks(s, M, has_shared(sh));
    moe::ChunkDownArgs a{c.cp(), cl, w2, sw2, q2, s2, by_pair ? 1 : 0, c.at<float>(c.L.y), sh};
    hipError_t e = moe::launch_chunk_down(s->hidden, s->inter, cl.C, a, st, ev);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "chunk down launch");
}

moe_status enqueue_combine(const moe_shape* s, int32_t M, const float* topk_w, float* out, const Carved& c,
                           hipStream_t st, bool shared = false)
{
    moe::CombineArgs a{c.at<float>(c.L.y), c.at<int32_t>(c.L.pos_of), topk_w, M, s->topk, out, shared ? 1 : 0};
    hipError_t e = moe::launch_combine(s->hidden, a, st);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "combine launch");
}

// Rows of a sorted-order intermediate, delivered in pair order.
moe_status gather_out(void* dst, const void* src, int rows, int row_bytes, const Carved& c, hipStream_t st)
{
    if (dst == nullptr) return MOE_OK;
    hipError_t e = moe::launch_gather_rows(src, dst, c.at<int32_t>(c.L.pos_of), rows, row_bytes, st);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "tap gather");
}

// Gate/up -> requantisation -> down -> combine over sorted pairs (the sort
// has run).  h, q2 and s2 stay in the workspace in sorted order.
moe_status enqueue_chunk_experts(const moe_shape* s, int32_t M, const uint8_t* act_q, const float* act_s,
                                 const float* topk_w, const uint8_t* w13, const uint8_t* s13, const uint8_t* w2,
                                 const uint8_t* sw2, float* out, const Carved& c, hipStream_t st,
                                 const moe::LaunchEvents& ev_gate_up = {}, const moe::LaunchEvents& ev_down = {},
                                 const moe::SharedWeights& sh = {})
{
    moe_status r;
    if ((r = enqueue_chunk_gate_up(s, M, act_q, act_s, w13, s13, c, st, ev_gate_up, sh)) != MOE_OK) return r;
    if ((r = enqueue_requant(s, pair_rows(s, M, sh), c.at<float>(c.L.h), c.at<uint8_t>(c.L.q2),
                             c.at<float>(c.L.s2), st)) != MOE_OK)
        return r;
    if ((r = enqueue_chunk_down(s, M, c.at<uint8_t>(c.L.q2), c.at<float>(c.L.s2), false, w2, sw2, c, st, ev_down,
                                sh)) != MOE_OK)
        return r;
    return enqueue_combine(s, M, topk_w, out, c, st, has_shared(sh));
}

// The M <= 8 path chosen by moe_set_decode_path (three kernels by default).
std::atomic<int32_t> g_decode_path{MOE_PATH_THREE_KERNELS};

// M <= 8 runs as one kernel when that path is selected, its kernels exist for
// (H, I) and its LDS plan fits; otherwise as the three kernels router ->
// gate/up -> down.  moe_path_info names the choice.
bool use_layer(const moe_shape* s, int32_t M, bool shared)
{
    if (g_decode_path.load(std::memory_order_relaxed) != MOE_PATH_ONE_KERNEL) return false;
    if (chunked(M) || !moe::layer_shape_supported(s->hidden, s->inter)) return false;
    const int pe = M * s->topk + (shared ? M : 0);
    return moe::layer_lds_bytes(s->hidden, s->inter, token_bound(M), pe) <= moe::kLayerMaxDynLds;
}

moe::LayerArgs layer_args(const moe_shape* s, int32_t M, const uint8_t* w13, const uint8_t* w13_scale,
                          const uint8_t* w2, const uint8_t* w2_scale, const moe::SharedWeights& sh, float* out,
                          const Carved& c)
{
    moe::LayerArgs a{};
    a.M = M;
    a.E = s->num_experts;
    a.K = s->topk;
    a.shared = has_shared(sh) ? 1 : 0;
    a.w13 = w13;
    a.s13 = w13_scale;
    a.w2 = w2;
    a.sw2 = w2_scale;
    a.sh = sh;
    a.out = out;
    a.sync = c.sync();
    return a;
}

// A shared expert's four tensors: all given, 16-byte aligned codes.
moe_status check_shared(const moe_shared_expert* sh)
{
    if (sh == nullptr) return MOE_OK;
    if (sh->w13 == nullptr || sh->w13_scale == nullptr || sh->w2 == nullptr || sh->w2_scale == nullptr)
        return fail(MOE_ERR_INVALID_ARG, "shared expert: w13, w13_scale, w2 and w2_scale must all be given");
    if (!aligned16(sh->w13) || !aligned16(sh->w2))
        return fail(MOE_ERR_ALIGNMENT, "shared expert: w13 and w2 must be 16-byte aligned");
    return MOE_OK;
}

moe_status copy_out(void* dst, const void* src, size_t bytes, hipStream_t st)
{
    if (dst == nullptr || bytes == 0) return MOE_OK;
    hipError_t e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "tap copy");
}

moe_status decode_forward(const moe_shape* shape, int32_t M, const uint16_t* hidden, const uint16_t* router_w,
                          const uint8_t* w13, const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale,
                          const moe_shared_expert* shared, float* out, void* ws, size_t ws_bytes, void* stream,
                          void* const* events)
{
    moe_status st = check_shape(shape, M);
    if (st != MOE_OK) return st;
    CHECK_PTR(hidden); CHECK_PTR(router_w); CHECK_PTR(w13); CHECK_PTR(w13_scale);
    CHECK_PTR(w2); CHECK_PTR(w2_scale); CHECK_PTR(out);
    CHECK_ALIGN(hidden); CHECK_ALIGN(router_w); CHECK_ALIGN(w13); CHECK_ALIGN(w2); CHECK_ALIGN(out);
    if ((st = check_shared(shared)) != MOE_OK) return st;
    if ((st = check_ws(shape, M, ws, ws_bytes)) != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto ev = [&](int k) -> moe::LaunchEvents {
        if (events == nullptr) return {};
        return {static_cast<hipEvent_t>(events[2 * k]), static_cast<hipEvent_t>(events[2 * k + 1])};
    };
    const moe::SharedWeights sh = shared_weights(shared);
    const Carved c = carve(shape, M, ws);
    int32_t* ids = c.at<int32_t>(c.L.ids);
    float* w = c.at<float>(c.L.w);
    uint8_t* q = c.at<uint8_t>(c.L.act_q);
    float* sc = c.at<float>(c.L.act_s);
    float* h = c.at<float>(c.L.h);
    if (use_layer(shape, M, has_shared(sh))) {
        moe::LayerArgs a = layer_args(shape, M, w13, w13_scale, w2, w2_scale, sh, out, c);
        a.x = hidden;
        a.wr = router_w;
        hipError_t e = moe::launch_layer(shape->hidden, shape->inter, token_bound(M), a, s, ev(0));
        return e == hipSuccess ? MOE_OK : hip_fail(e, "layer launch");
    }
    if (chunked(M)) {
        if ((st = enqueue_chunk_router(shape, M, hidden, router_w, c, s, ev(0))) != MOE_OK) return st;
        if ((st = enqueue_chunk_topk(shape, M, ids, w, c, s, hidden, q, sc)) != MOE_OK) return st;
        if ((st = enqueue_sort(shape, M, ids, c, s, has_shared(sh))) != MOE_OK) return st;
        return enqueue_chunk_experts(shape, M, q, sc, w, w13, w13_scale, w2, w2_scale, out, c, s, ev(1), ev(2), sh);
    }
    // One or two tokens: the gate/up kernel quantises the activations itself
    // (its waves that derive no routing do it during the routing prologue),
    // so the router only computes logits.  More tokens: the router quantises
    // them, a slice per workgroup.  (The router quantising one token too
    // makes gate_up 0.4 us shorter but the graph-replayed layer 0.3 us
    // longer, measured.)
    const bool one = M <= 2;
    if ((st = enqueue_router(shape, M, hidden, router_w, one ? nullptr : q, one ? nullptr : sc, c, s, ev(0))) !=
        MOE_OK)
        return st;
    if ((st = enqueue_gate_up(shape, M, nullptr, ids, w, q, sc, w13, w13_scale, h, c, s, ev(1), sh,
                              one ? hidden : nullptr)) != MOE_OK)
        return st;
    return enqueue_down(shape, M, h, nullptr, nullptr, nullptr, nullptr, w, w2, w2_scale, out, c, s, ev(2), sh);
}

moe_status experts_forward(const moe_shape* shape, int32_t M, const uint8_t* act_fp8, const float* act_scale,
                           const int32_t* topk_ids, const float* topk_w, const uint8_t* w13,
                           const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale,
                           const moe_shared_expert* shared, float* out, const moe_expert_taps* taps, void* ws,
                           size_t ws_bytes, void* stream)
{
    moe_status st = check_shape(shape, M);
    if (st != MOE_OK) return st;
    CHECK_PTR(act_fp8); CHECK_PTR(act_scale); CHECK_PTR(topk_ids); CHECK_PTR(topk_w);
    CHECK_PTR(w13); CHECK_PTR(w13_scale); CHECK_PTR(w2); CHECK_PTR(w2_scale); CHECK_PTR(out);
    CHECK_ALIGN(act_fp8); CHECK_ALIGN(w13); CHECK_ALIGN(w2); CHECK_ALIGN(out);
    if ((st = check_shared(shared)) != MOE_OK) return st;
    if ((st = check_ws(shape, M, ws, ws_bytes)) != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const moe::SharedWeights sh = shared_weights(shared);
    const Carved c = carve(shape, M, ws);
    if (chunked(M)) {
        if ((st = enqueue_sort(shape, M, topk_ids, c, s, has_shared(sh))) != MOE_OK) return st;
        if ((st = enqueue_chunk_experts(shape, M, act_fp8, act_scale, topk_w, w13, w13_scale, w2, w2_scale, out, c,
                                        s, {}, {}, sh)) != MOE_OK)
            return st;
        if (taps == nullptr) return MOE_OK;
        const int I = shape->inter, R = pair_rows(shape, M, sh);
        if ((st = gather_out(taps->h, c.at<void>(c.L.h), R, I * 4, c, s)) != MOE_OK) return st;
        if ((st = gather_out(taps->inter_fp8, c.at<void>(c.L.q2), R, I, c, s)) != MOE_OK) return st;
        return gather_out(taps->inter_scale, c.at<void>(c.L.s2), R, 4, c, s);
    }
    if (use_layer(shape, M, has_shared(sh))) {
        moe::LayerArgs a = layer_args(shape, M, w13, w13_scale, w2, w2_scale, sh, out, c);
        a.act_q = act_fp8;
        a.act_s = act_scale;
        a.ids = topk_ids;
        a.topk_w = topk_w;
        if (taps != nullptr) {
            a.h_tap = taps->h;
            a.q2_tap = taps->inter_fp8;
            a.s2_tap = taps->inter_scale;
        }
        hipError_t e = moe::launch_layer(shape->hidden, shape->inter, token_bound(M), a, s);
        return e == hipSuccess ? MOE_OK : hip_fail(e, "layer launch");
    }
    float* h = (taps && taps->h) ? taps->h : c.at<float>(c.L.h);
    uint8_t* q2_tap = taps ? taps->inter_fp8 : nullptr;
    float* s2_tap = taps ? taps->inter_scale : nullptr;
    if ((st = enqueue_gate_up(shape, M, topk_ids, nullptr, nullptr, act_fp8, act_scale, w13, w13_scale, h, c, s, {},
                              sh)) != MOE_OK)
        return st;
    return enqueue_down(shape, M, h, nullptr, nullptr, q2_tap, s2_tap, topk_w, w2, w2_scale, out, c, s, {}, sh);
}

// ---- the entry point that allocates nothing --------------------------------
// A workspace that lives in the library itself: one file-scope device array,
// of which every GPU that loads the library holds its own copy until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in): the device address of the current device's
// copy comes from hipGetSymbolAddress, once per device, and is kept.
constexpr size_t kScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// The current device's scratch address.  At its first use on a device the
// array is zeroed by a fill kernel on `stream` (the workspace-init state).
moe_status scratch_for_device(hipStream_t stream, void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kScratchDevices)
        return fail(MOE_ERR_HIP, "device %d is beyond the %d devices the static scratch serves", dev, kScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (p == nullptr || ((uintptr_t)p & 255u) != 0) return fail(MOE_ERR_HIP, "static scratch is not 256-byte aligned");
        e = moe::launch_fill_u32(static_cast<uint32_t*>(p), kScratchBytes / 4, 0u, stream);
        if (e != hipSuccess) return hip_fail(e, "static scratch init");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {


size_t moe_workspace_bytes(const moe_shape* shape, int32_t max_tokens)
{
    if (check_shape(shape, max_tokens) != MOE_OK) return 0;
    return moe::ws_layout(shape->hidden, shape->inter, shape->num_experts, shape->topk, max_tokens).total;
}

moe_status moe_workspace_init(void* ws, size_t ws_bytes, void* stream)
{
    if (ws == nullptr || ws_bytes < 256) return fail(MOE_ERR_WORKSPACE, "workspace is NULL or below 256 bytes");
    if (((uintptr_t)ws & 255u) != 0) return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    // no call reads what an earlier call left; zeroing makes a never-written
    // compaction read as "no active expert"
    hipError_t e = moe::launch_fill_u32(static_cast<uint32_t*>(ws), ws_bytes / 4, 0u, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "workspace init");
}

moe_status moe_decode_forward_events(const moe_shape* shape, int32_t M, const uint16_t* hidden,
                                     const uint16_t* router_w, const uint8_t* w13, const uint8_t* w13_scale,
                                     const uint8_t* w2, const uint8_t* w2_scale, float* out, void* ws,
                                     size_t ws_bytes, void* stream, void* const* events)
{
    return decode_forward(shape, M, hidden, router_w, w13, w13_scale, w2, w2_scale, nullptr, out, ws, ws_bytes,
                          stream, events);
}

moe_status moe_decode_forward_shared(const moe_shape* shape, int32_t M, const uint16_t* hidden,
                                     const uint16_t* router_w, const uint8_t* w13, const uint8_t* w13_scale,
                                     const uint8_t* w2, const uint8_t* w2_scale, const moe_shared_expert* shared,
                                     float* out, void* ws, size_t ws_bytes, void* stream, void* const* events)
{
    return decode_forward(shape, M, hidden, router_w, w13, w13_scale, w2, w2_scale, shared, out, ws, ws_bytes,
                          stream, events);
}

moe_status moe_decode_forward(const moe_shape* shape, int32_t M, const uint16_t* hidden, const uint16_t* router_w,
                              const uint8_t* w13, const uint8_t* w13_scale, const uint8_t* w2,
                              const uint8_t* w2_scale, float* out, void* ws, size_t ws_bytes, void* stream)
{
    return moe_decode_forward_events(shape, M, hidden, router_w, w13, w13_scale, w2, w2_scale, out, ws, ws_bytes,
                                     stream, nullptr);
}

moe_status moe_decode_forward_noalloc(const moe_shape* shape, int32_t M, const uint16_t* hidden,
                                      const uint16_t* router_w, const uint8_t* w13, const uint8_t* w13_scale,
                                      const uint8_t* w2, const uint8_t* w2_scale, float* out, void* stream)
{
    // everything is checked before anything (the scratch's first-use fill
    // included) is enqueued
    moe_status st = check_shape(shape, M);
    if (st != MOE_OK) return st;
    CHECK_PTR(hidden); CHECK_PTR(router_w); CHECK_PTR(w13); CHECK_PTR(w13_scale);
    CHECK_PTR(w2); CHECK_PTR(w2_scale); CHECK_PTR(out);
    CHECK_ALIGN(hidden); CHECK_ALIGN(router_w); CHECK_ALIGN(w13); CHECK_ALIGN(w2); CHECK_ALIGN(out);
    const size_t need = moe::ws_layout(shape->hidden, shape->inter, shape->num_experts, shape->topk, M).total;
    if (need > kScratchBytes)
        return fail(MOE_ERR_UNSUPPORTED_SHAPE,
                    "M=%d needs %zu bytes of scratch; the library's static scratch holds %zu (use moe_decode_forward "
                    "with a workspace)",
                    M, need, kScratchBytes);
    void* ws = nullptr;
    if ((st = scratch_for_device(static_cast<hipStream_t>(stream), &ws)) != MOE_OK) return st;
    return decode_forward(shape, M, hidden, router_w, w13, w13_scale, w2, w2_scale, nullptr, out, ws, kScratchBytes,
                          stream, nullptr);
}

moe_status moe_route(const moe_shape* shape, int32_t M, const uint16_t* hidden, const uint16_t* router_w,
                     int32_t* topk_ids, float* topk_w, const moe_route_taps* taps, void* ws, size_t ws_bytes,
                     void* stream)
{
    moe_status st = check_shape(shape, M);
    if (st != MOE_OK) return st;
    CHECK_PTR(hidden); CHECK_PTR(router_w); CHECK_PTR(topk_ids); CHECK_PTR(topk_w);
    CHECK_ALIGN(hidden); CHECK_ALIGN(router_w);
    if ((st = check_ws(shape, M, ws, ws_bytes)) != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Carved c = carve(shape, M, ws);
    uint8_t* act_q = taps ? taps->act_fp8 : nullptr;
    float* act_s = taps ? taps->act_scale : nullptr;
    if ((act_q == nullptr) != (act_s == nullptr))
        return fail(MOE_ERR_INVALID_ARG, "taps act_fp8 and act_scale must be given together");
    if (chunked(M)) {
        if ((st = enqueue_chunk_router(shape, M, hidden, router_w, c, s)) != MOE_OK) return st;
        if ((st = enqueue_chunk_topk(shape, M, topk_ids, topk_w, c, s, hidden, act_q, act_s)) != MOE_OK) return st;
        if ((st = enqueue_sort(shape, M, topk_ids, c, s)) != MOE_OK) return st;
    } else {
        if ((st = enqueue_router(shape, M, hidden, router_w, act_q, act_s, c, s)) != MOE_OK) return st;
        if ((st = enqueue_topk(shape, M, true, nullptr, topk_ids, topk_w, c, s)) != MOE_OK) return st;
    }
    if (taps == nullptr) return MOE_OK;
    const size_t P = (size_t)M * shape->topk, S = (size_t)num_slots(shape, M);
    if ((st = copy_out(taps->logits, c.at<void>(c.L.logits), (size_t)M * shape->num_experts * 4, s)) != MOE_OK) return st;
    if ((st = copy_out(taps->n_active, c.at<void>(c.L.n_act), 4, s)) != MOE_OK) return st;
    if ((st = copy_out(taps->act_experts, c.at<void>(c.L.act_experts), S * 4, s)) != MOE_OK) return st;
    if ((st = copy_out(taps->offsets, c.at<void>(c.L.offsets), (S + 1) * 4, s)) != MOE_OK) return st;
    if ((st = copy_out(taps->pair_token, c.at<void>(c.L.pair_token), P * 4, s)) != MOE_OK) return st;
    return copy_out(taps->pair_src, c.at<void>(c.L.pair_src), P * 4, s);
}

moe_status moe_quant_act(const moe_shape* shape, int32_t M, const uint16_t* hidden, uint8_t* act_fp8,
                         float* act_scale, void* stream)
{
    moe_status st = check_shape(shape, M);
    if (st != MOE_OK) return st;
    CHECK_PTR(hidden); CHECK_PTR(act_fp8); CHECK_PTR(act_scale);
    hipError_t e = moe::launch_quant(shape->hidden, hidden, M, act_fp8, act_scale, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "quant launch");
}

moe_status moe_experts_forward(const moe_shape* shape, int32_t M, const uint8_t* act_fp8, const float* act_scale,
                               const int32_t* topk_ids, const float* topk_w, const uint8_t* w13,
                               const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale, float* out,
                               const moe_expert_taps* taps, void* ws, size_t ws_bytes, void* stream)
{
    return experts_forward(shape, M, act_fp8, act_scale, topk_ids, topk_w, w13, w13_scale, w2, w2_scale, nullptr, out,
                           taps, ws, ws_bytes, stream);
}

moe_status moe_experts_forward_shared(const moe_shape* shape, int32_t M, const uint8_t* act_fp8,
                                      const float* act_scale, const int32_t* topk_ids, const float* topk_w,
                                      const uint8_t* w13, const uint8_t* w13_scale, const uint8_t* w2,
                                      const uint8_t* w2_scale, const moe_shared_expert* shared, float* out,
                                      const moe_expert_taps* taps, void* ws, size_t ws_bytes, void* stream)
{
    return experts_forward(shape, M, act_fp8, act_scale, topk_ids, topk_w, w13, w13_scale, w2, w2_scale, shared, out,
                           taps, ws, ws_bytes, stream);
}

moe_status moe_gate_up(const moe_shape* shape, int32_t M, const uint8_t* act_fp8, const float* act_scale,
                       const int32_t* topk_ids, const uint8_t* w13, const uint8_t* w13_scale, float* h,
                       uint8_t* inter_fp8, float* inter_scale, void* ws, size_t ws_bytes, void* stream)
{
    moe_status st = check_shape(shape, M);
    if (st != MOE_OK) return st;
    CHECK_PTR(act_fp8); CHECK_PTR(act_scale); CHECK_PTR(topk_ids); CHECK_PTR(w13); CHECK_PTR(w13_scale);
    CHECK_PTR(h); CHECK_PTR(inter_fp8); CHECK_PTR(inter_scale);
    CHECK_ALIGN(act_fp8); CHECK_ALIGN(w13);
    if ((st = check_ws(shape, M, ws, ws_bytes)) != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Carved c = carve(shape, M, ws);
    if (chunked(M)) {
        if ((st = enqueue_sort(shape, M, topk_ids, c, s)) != MOE_OK) return st;
        if ((st = enqueue_chunk_gate_up(shape, M, act_fp8, act_scale, w13, w13_scale, c, s)) != MOE_OK) return st;
        const int I = shape->inter, P = M * shape->topk;
        if ((st = enqueue_requant(shape, P, c.at<float>(c.L.h), c.at<uint8_t>(c.L.q2), c.at<float>(c.L.s2), s)) !=
            MOE_OK)
            return st;
        if ((st = gather_out(h, c.at<void>(c.L.h), P, I * 4, c, s)) != MOE_OK) return st;
        if ((st = gather_out(inter_fp8, c.at<void>(c.L.q2), P, I, c, s)) != MOE_OK) return st;
        return gather_out(inter_scale, c.at<void>(c.L.s2), P, 4, c, s);
    }
    if ((st = enqueue_gate_up(shape, M, topk_ids, nullptr, nullptr, act_fp8, act_scale, w13, w13_scale, h, c, s)) !=
        MOE_OK)
        return st;
    return enqueue_requant(shape, M * shape->topk, h, inter_fp8, inter_scale, s);
}

moe_status moe_down_combine(const moe_shape* shape, int32_t M, const uint8_t* inter_fp8, const float* inter_scale,
                            const int32_t* topk_ids, const float* topk_w, const uint8_t* w2, const uint8_t* w2_scale,
                            float* out, void* ws, size_t ws_bytes, void* stream)
{
    moe_status st = check_shape(shape, M);
    if (st != MOE_OK) return st;
    CHECK_PTR(inter_fp8); CHECK_PTR(inter_scale); CHECK_PTR(topk_ids); CHECK_PTR(topk_w);
    CHECK_PTR(w2); CHECK_PTR(w2_scale); CHECK_PTR(out);
    CHECK_ALIGN(inter_fp8); CHECK_ALIGN(w2); CHECK_ALIGN(out);
    if ((st = check_ws(shape, M, ws, ws_bytes)) != MOE_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Carved c = carve(shape, M, ws);
    if (chunked(M)) {
        if ((st = enqueue_sort(shape, M, topk_ids, c, s)) != MOE_OK) return st;
        if ((st = enqueue_chunk_down(shape, M, inter_fp8, inter_scale, true, w2, w2_scale, c, s)) != MOE_OK)
            return st;
        return enqueue_combine(shape, M, topk_w, out, c, s);
    }
    if ((st = enqueue_topk(shape, M, false, topk_ids, nullptr, nullptr, c, s)) != MOE_OK) return st;
    return enqueue_down(shape, M, nullptr, inter_fp8, inter_scale, nullptr, nullptr, topk_w, w2, w2_scale, out, c, s);
}

moe_status moe_lm_head_quantize(const uint16_t* w_bf16, int32_t vocab, int32_t hidden, uint8_t* q, float* scale,
                                void* stream)
{
    CHECK_PTR(w_bf16); CHECK_PTR(q); CHECK_PTR(scale);
    CHECK_ALIGN(w_bf16); CHECK_ALIGN(q);
    if (vocab <= 0 || hidden <= 0) return fail(MOE_ERR_INVALID_ARG, "vocab (%d) and hidden (%d) must be positive", vocab, hidden);
    if (hidden % 8 != 0) return fail(MOE_ERR_INVALID_ARG, "hidden (%d) must be a multiple of 8", hidden);
    hipError_t e = moe::launch_lm_head_quant(w_bf16, vocab, hidden, q, scale, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "lm-head quantisation launch");
}

moe_status moe_lm_head_forward(const uint16_t* x_bf16, int32_t M, const uint8_t* q, const float* scale,
                               int32_t vocab, int32_t hidden, float* logits, void* stream)
{
    CHECK_PTR(x_bf16); CHECK_PTR(q); CHECK_PTR(scale); CHECK_PTR(logits);
    CHECK_ALIGN(x_bf16); CHECK_ALIGN(q);
    if (vocab <= 0) return fail(MOE_ERR_INVALID_ARG, "vocab (%d) must be positive", vocab);
    if (M <= 0) return fail(MOE_ERR_INVALID_ARG, "M (%d) must be positive", M);
    if (M > moe::kMaxGemvTokens)
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "the LM-head GEMV is compiled for up to %d tokens (M=%d)",
                    moe::kMaxGemvTokens, M);
    if (!moe::lm_head_shape_supported(hidden))
        return fail(MOE_ERR_UNSUPPORTED_SHAPE,
                    "hidden %d has no LM-head kernel on this device: compiled in are 512 and 2560; other sizes "
                    "(multiples of 256 up to 4096) need moe_jit_load of a layer shape with that hidden size first",
                    hidden);
    hipError_t e = moe::launch_lm_head_gemv(hidden, token_bound(M), x_bf16, M, q, scale, vocab, logits,
                                            static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "lm-head GEMV launch");
}

moe_status moe_fp8_encode_range(uint32_t first_bits, int64_t n, uint8_t* q, void* stream)
{
    if (q == nullptr) return fail(MOE_ERR_INVALID_ARG, "q is NULL");
    if (n < 0) return fail(MOE_ERR_INVALID_ARG, "n (%lld) is negative", (long long)n);
    hipError_t e = moe::launch_fp8_encode_range(first_bits, n, q, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "fp8 encode launch");
}

moe_status moe_path_info(const moe_shape* shape, int32_t M, char* buf, size_t len)
{
    moe_status st = check_shape(shape, M);
    if (buf != nullptr && len > 0) {
        char names[1024];
        if (st != MOE_OK) {
            snprintf(buf, len, "unsupported: %s", g_last_error);
        } else if (chunked(M)) {
            moe::chunk_kernel_names(shape->hidden, shape->inter, names, sizeof names);
            snprintf(buf, len, "chunk path, M=%d, E=%d, K=%d: %s", M, shape->num_experts, shape->topk, names);
        } else if (use_layer(shape, M, false)) {
            moe::layer_kernel_names(shape->hidden, shape->inter, names, sizeof names);
            snprintf(buf, len, "one-kernel gemv path, M=%d (token bound %d), E=%d, K=%d: %s", M, token_bound(M),
                     shape->num_experts, shape->topk, names);
        } else {
            moe::kernel_names(shape->hidden, shape->inter, names, sizeof names);
            snprintf(buf, len, "gemv path, M=%d (token bound %d), E=%d, K=%d: %s", M, token_bound(M),
                     shape->num_experts, shape->topk, names);
        }
    }
    return st;
}

static moe_status jit_status(moe::JitStatus st, const std::string& err)
{
    switch (st) {
        case moe::JitStatus::Ok: return MOE_OK;
        case moe::JitStatus::BadShape:
        case moe::JitStatus::BadArch: return fail(MOE_ERR_UNSUPPORTED_SHAPE, "%s", err.c_str());
        case moe::JitStatus::CacheIo:
        case moe::JitStatus::Compile: return fail(MOE_ERR_JIT, "%s", err.c_str());
        case moe::JitStatus::Load: return fail(MOE_ERR_HIP, "%s", err.c_str());
    }
    return fail(MOE_ERR_JIT, "%s", err.c_str());
}

static void fill_report(moe_jit_report* r, const moe::JitReport& j)
{
    if (r == nullptr) return;
    r->from_cache = j.from_cache ? 1 : 0;
    r->has_chunk_path = j.chunk ? 1 : 0;
    r->has_lm_head = j.lm_head ? 1 : 0;
    r->num_kernels = j.kernels;
    r->seconds = j.seconds;
    snprintf(r->cache_file, sizeof r->cache_file, "%s", j.file);
}

moe_status moe_jit_build(const moe_shape* shape, const char* arch, const char* cache_dir, moe_jit_report* report)
{
    if (shape == nullptr) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
    if (arch == nullptr) return fail(MOE_ERR_INVALID_ARG, "arch is NULL");
    moe::JitReport j;
    std::string err;
    const moe::JitStatus st = moe::jit_build(shape->hidden, shape->inter, arch, cache_dir, &j, &err);
    fill_report(report, j);
    return jit_status(st, err);
}

moe_status moe_jit_load(const moe_shape* shape, const char* cache_dir, int32_t prefer, moe_jit_report* report)
{
    if (shape == nullptr) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
    moe::JitReport j;
    std::string err;
    const moe::JitStatus st = moe::jit_load(shape->hidden, shape->inter, cache_dir, prefer != 0, &j, &err);
    fill_report(report, j);
    return jit_status(st, err);
}

int32_t moe_jit_unload(const moe_shape* shape)
{
    if (shape == nullptr) return 0;
    return moe::jit_unload(shape->hidden, shape->inter);
}

const char* moe_status_string(moe_status status)
{
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
        case MOE_ERR_ALIGNMENT: return "misaligned pointer";
        case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case MOE_ERR_HIP: return "HIP error";
        case MOE_ERR_JIT: return "run-time compilation or its cache failed";
    }
    return "unknown status";
}

const char* moe_last_error(void) { return g_last_error; }

moe_status moe_workspace_sync_status(const void* ws, size_t ws_bytes, uint32_t* status, void* stream)
{
    if (ws == nullptr || ws_bytes < 256) return fail(MOE_ERR_WORKSPACE, "workspace is NULL or below 256 bytes");
    if (((uintptr_t)ws & 255u) != 0) return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (status == nullptr) return fail(MOE_ERR_INVALID_ARG, "status is NULL");
    // the error word follows the epoch at the start of the workspace
    hipError_t e = hipMemcpyAsync(status, static_cast<const uint32_t*>(ws) + 1, 4, hipMemcpyDeviceToDevice,
                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "sync status copy");
}

void moe_set_wait_limit_us(uint32_t us) { moe::set_layer_wait_us(us); }

moe_status moe_set_decode_path(int32_t path)
{
    if (path != MOE_PATH_THREE_KERNELS && path != MOE_PATH_ONE_KERNEL)
        return fail(MOE_ERR_INVALID_ARG, "decode path %d is neither 0 (three kernels) nor 1 (one kernel)", path);
    g_decode_path.store(path, std::memory_order_relaxed);
    return MOE_OK;
}

}  // extern "C"
