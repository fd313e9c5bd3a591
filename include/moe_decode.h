/*
 * moe_decode.h -- C ABI of the MI355X (gfx950) W4A8 mixture-of-experts decode layer.
 *
 * What the layer computes.  The pages behind this library describe decode of
 * a Ling-3.0-flash-shaped MoE model at batch size 1 and find it bound by
 * reading weights; the two largest readers are the MoE experts and the LM
 * head ([EN] "Why is MoE decoding on DGX Spark memory-bound?"; [ZH]
 * "三项优化分别做了什么").  The model routes every token to 8 routed experts
 * ([EN] "What is Ling 3.0, and why does it suit DGX Spark?"), its expert
 * layer is 768 wide ([EN] "What are the 3 optimizations?", item 1), its hidden
 * state is 2,560 wide (same section, item 2), the experts are stored as MXFP4
 * with FP8 activations (the W4A8 recipe, [EN] "Why is MoE decoding...") and a
 * speculative-decoding verify step runs 4 token positions through the layer at
 * once, touching up to 32 experts ([EN] "What are the 3 optimizations?",
 * item 3; [ZH] "合成负载与真实评测的差距").
 *   [EN] = "NVIDIA Shows 3 Ways to Speed Up MoE Inference on DGX Spark,
 *          Lifting Ling-3.0-flash Throughput 42.5%"
 *   [ZH] = "NVIDIA博客:DGX Spark上三项优化使Ling-3.0-flash解码吞吐提升 42.5%"
 *
 * For M tokens x[M,H] (bf16), E experts and top-K routing:
 *   logits = x Wr^T (fp32); ids = the K largest logits per token (ties -> lower
 *   expert index); w = softmax restricted to the K selected logits.
 *   q, s   = per-token FP8 E4M3 quantisation: s = amax/448 (1 if amax == 0),
 *            q = E4M3_RNE_satfinite(x / s) with a correctly rounded fp32 division.
 *   for each (token t, rank j), expert e = ids[t,j], pair p = t*K + j:
 *     g, u = rows [0,I) and [I,2I) of W13[e] times A = E4M3(q[t]) * s[t]
 *     h[p] = SiLU(g) * u                         (fp32; SiLU(z) = z * sigmoid(z))
 *     s2[p] = max|h[p]| / 448 (1 if 0); q2[p] = E4M3_RNE_satfinite(h[p] / s2[p])
 *   out[t] = sum_j w[t,j] * s2[p] * (W2[e] times E4M3(q2[p]))   (fp32, overwritten)
 * where an MXFP4 matrix element is E2M1(code) * 2^(E8M0 block scale - 127).
 * No residual is added.  The *_shared entry points add the model's shared
 * expert: each Ling MoE layer sends every token to one shared expert besides
 * its 8 routed ones ([EN] "What is Ling 3.0, and why does it suit DGX
 * Spark?").  It is one more expert of the routed layout, taken by every token
 * with weight 1 through the same steps (gate/up on E4M3(q[t]) * s[t], SiLU*up,
 * FP8 requantisation, down); its term is added after the K routed terms:
 *   out[t] = sum_j w[t,j] * y[t*K+j] + y_shared[t]
 * and its intermediate is row M*K + t of the tapped intermediates.
 *
 * Storage layout (every tensor dense, row-major, no padding):
 *   hidden      bf16 bits  [M, H]
 *   router_w    bf16 bits  [E, H]
 *   w13         u8         [E, 2I, H/2]   E2M1 codes; element 2i in bits 3:0 of
 *                                          byte i, element 2i+1 in bits 7:4;
 *                                          rows [0,I) gate, rows [I,2I) up
 *   w13_scale   u8 (E8M0)  [E, 2I, H/32]  one scale per 32 consecutive elements
 *   w2          u8         [E, H, I/2]    same nibble order
 *   w2_scale    u8 (E8M0)  [E, H, I/32]
 *   out         fp32       [M, H]
 *   act_fp8     u8 (E4M3)  [M, H],  act_scale fp32 [M]
 *   topk_ids    int32      [M, K],  topk_w    fp32 [M, K]   (pair p = t*K + j)
 *   inter_fp8   u8 (E4M3)  [M*K, I], inter_scale fp32 [M*K], h fp32 [M*K, I]
 *
 * Ownership and execution.  Every tensor pointer is device memory owned by
 * the caller.  The library never allocates, frees or synchronises: each call
 * validates its arguments on the host, enqueues its kernels on `stream`
 * (a hipStream_t; NULL is the default stream) and returns.  The caller keeps
 * every buffer alive until the stream has passed the call.  Inputs are only
 * read.  A workspace serves one call in flight at a time; calls with distinct
 * workspaces may run concurrently.  The library keeps no other global state
 * except a thread-local copy of the last error message and the registry of
 * modules loaded by moe_jit_load.
 *
 * Errors.  Every argument is checked before anything is enqueued; on any
 * error nothing is enqueued and the status says why.  No C++ exception
 * crosses this interface.  A shape with no kernels on the current device
 * (neither compiled in nor loaded by moe_jit_load) is
 * MOE_ERR_UNSUPPORTED_SHAPE -- there is never a silent fallback to a slower
 * or different kernel (the pages warn that a silent fallback made a draft
 * model misread FP8 weights as BF16: [EN] "What are the 3 optimizations?",
 * "The integration trap"; [ZH] "叠加时的配置陷阱").  moe_path_info() names the
 * kernels a call would run so that callers can check at startup that the path
 * they expect is active, as the pages advise.  Non-finite inputs are not
 * detected; results for them are unspecified.  Caller-given topk_ids must
 * lie in [0, E).  A token may name one expert more than once on the chunk
 * path (M > 8) and on the one-kernel path (moe_experts_forward at M <= 8
 * with MOE_PATH_ONE_KERNEL selected): each (token, j) pair is then computed
 * and weighted on its own.  On the three-kernel M <= 8 path and in
 * moe_gate_up / moe_down_combine at M <= 8 the ids of a token must be
 * distinct.  Other ids give unspecified results (they are clamped on the
 * device, never read or written out of bounds).
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,       /* null pointer, non-positive size, K > E ... */
    MOE_ERR_UNSUPPORTED_SHAPE = -2, /* (H, I, E, K, M) outside the compiled set  */
    MOE_ERR_ALIGNMENT = -3,         /* a tensor base is not 16-byte aligned       */
    MOE_ERR_WORKSPACE = -4,         /* workspace missing, misaligned or too small */
    MOE_ERR_HIP = -5,               /* a HIP launch or copy failed                */
    MOE_ERR_JIT = -6                /* run-time compilation or its cache failed   */
} moe_status;

/* H = hidden, I = expert intermediate, E = routed experts, K = experts per token. */
typedef struct {
    int32_t hidden;
    int32_t inter;
    int32_t num_experts;
    int32_t topk;
} moe_shape;

/* Optional device outputs of moe_route for checking the routing stages.
 * Any member may be NULL.  Sizes use S = min(E, M*K). */
typedef struct {
    float*   logits;       /* [M, E] fp32 router logits                              */
    int32_t* n_active;     /* [1] number of distinct selected experts                */
    int32_t* act_experts;  /* [S] distinct selected experts, ascending id            */
    int32_t* offsets;      /* [S+1] start of each expert's pair list                 */
    int32_t* pair_token;   /* [M*K] token of each compacted pair                     */
    int32_t* pair_src;     /* [M*K] pair index t*K+j of each compacted pair          */
    uint8_t* act_fp8;      /* [M, H] E4M3 activations, as the router kernel makes them */
    float*   act_scale;    /* [M] their fp32 scales                                   */
} moe_route_taps;

/* Optional device outputs of the expert stages.  Any member may be NULL. */
typedef struct {
    float*   h;            /* [M*K, I] fp32 SiLU(g)*u before requantisation          */
    uint8_t* inter_fp8;    /* [M*K, I] E4M3 intermediate                              */
    float*   inter_scale;  /* [M*K] fp32 intermediate scale                           */
} moe_expert_taps;

/* The shared expert: one expert of the routed layout (no leading E axis).
 * All four pointers are device memory owned by the caller; w13 and w2 must be
 * 16-byte aligned. */
typedef struct {
    const uint8_t* w13;        /* [2I, H/2]  E2M1 codes, rows [0,I) gate, [I,2I) up */
    const uint8_t* w13_scale;  /* [2I, H/32] E8M0                                    */
    const uint8_t* w2;         /* [H, I/2]   E2M1 codes                              */
    const uint8_t* w2_scale;   /* [H, I/32]  E8M0                                    */
} moe_shared_expert;

/* Bytes of workspace needed for calls with up to max_tokens tokens; 0 if the
 * shape or max_tokens is invalid or unsupported.  The requirement is
 * non-decreasing in max_tokens, so one workspace sized for max_tokens serves
 * every smaller M, with or without a shared expert. */
size_t moe_workspace_bytes(const moe_shape* shape, int32_t max_tokens);

/* How M <= 8 runs (chunk-path calls, M > 8, are not affected).
 * MOE_PATH_THREE_KERNELS (the default): router, gate/up and down kernels in
 * stream order.  MOE_PATH_ONE_KERNEL: the whole layer as one kernel
 * (layer_kernel) with one workgroup per compute unit, whose workgroups hand
 * logits, intermediate rows and down outputs to each other through
 * epoch-tagged words in the workspace instead of kernel boundaries; shapes
 * outside its LDS plan keep the three kernels.  At Ling-3.0-flash's shape on
 * MI355X the one-kernel layer measures slower (the hand-offs cost more under
 * 256-way polling than a kernel boundary), so it is opt-in. */
typedef enum {
    MOE_PATH_THREE_KERNELS = 0,
    MOE_PATH_ONE_KERNEL = 1
} moe_decode_path;

/* Selects the M <= 8 path for later calls from any thread (a process-wide
 * setting, like moe_set_wait_limit_us).  MOE_ERR_INVALID_ARG for any other
 * value.  moe_path_info reports the selection. */
moe_status moe_set_decode_path(int32_t path);

/* Zero the workspace (a fill kernel on `stream`; the caller orders later
 * calls on other streams after it).  Required once for a new workspace before
 * its first call: on the one-kernel path the layer's workgroups hand results
 * to each other through epoch-tagged words kept at the start of the
 * workspace, and the epoch carries over from call to call (zeroing again
 * later is allowed; it clears the sticky wait-error bits as well).  ws must
 * be 256-byte aligned. */
moe_status moe_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Copies (on `stream`, device to device) the workspace's sticky wait-error
 * bits into *status, a caller device word: 0 when every call of the one-kernel
 * layer since moe_workspace_init completed its hand-offs.  The layer kernel's
 * workgroups wait for each other (they are all resident at once: one per
 * compute unit); every such wait is bounded (0.2 s by default), and a wait
 * that runs out sets bit 1 (router logits), 2 (intermediate rows), 4 (down
 * outputs) or 8 (arrivals) and lets the kernel finish with an undefined
 * result.  A wait can only run out when another kernel occupies compute units
 * for longer than the bound, e.g. more than one of these layers running
 * concurrently on one GPU. */
moe_status moe_workspace_sync_status(const void* ws, size_t ws_bytes, uint32_t* status, void* stream);

/* Sets the bound of every wait of the one-kernel layer, in microseconds, for
 * later launches from any thread (0 restores the default, 0.2 s).  For tests
 * of the wait-error path. */
void moe_set_wait_limit_us(uint32_t us);

/* The whole layer for M tokens: route -> quantise -> compact -> gate/up ->
 * requantise -> down + combine.  out[M,H] fp32 is overwritten.  M <= 8 runs
 * as three kernels (router, gate/up, down), or as one (layer_kernel) when
 * moe_set_decode_path selected it and its LDS plan fits; M > 8 runs the chunk
 * path.  moe_path_info names the kernels. */
moe_status moe_decode_forward(const moe_shape* shape, int32_t M,
                              const uint16_t* hidden, const uint16_t* router_w,
                              const uint8_t* w13, const uint8_t* w13_scale,
                              const uint8_t* w2, const uint8_t* w2_scale,
                              float* out, void* ws, size_t ws_bytes, void* stream);

/* moe_decode_forward with per-kernel timing: `events` is an array of 6
 * caller-created hipEvent_t (timing enabled), start/stop pairs for the router
 * (0, 1), gate/up (2, 3) and down (4, 5) kernels; on the one-kernel path the
 * pair (0, 1) times layer_kernel and the other events are not used.  Each pair is stamped by the
 * kernel's own launch (hipExtLaunchKernel), so hipEventElapsedTime of a pair
 * is that kernel's execution time on the GPU, without queueing or dispatch
 * gaps.  `events` may be NULL (then this is moe_decode_forward); a NULL pair
 * launches that kernel without stamps.  Not for use under stream capture. */
moe_status moe_decode_forward_events(const moe_shape* shape, int32_t M,
                                     const uint16_t* hidden, const uint16_t* router_w,
                                     const uint8_t* w13, const uint8_t* w13_scale,
                                     const uint8_t* w2, const uint8_t* w2_scale,
                                     float* out, void* ws, size_t ws_bytes, void* stream,
                                     void* const* events);

/* moe_decode_forward_events plus the shared expert (see the layer definition
 * above).  `shared` may be NULL: then this is moe_decode_forward_events.
 * Its slot runs in the same gate/up and down kernels as the routed experts
 * (after them in slot order), so the layer stays three kernels at M <= 8.
 * MOE_ERR_INVALID_ARG if a member of *shared is NULL, MOE_ERR_ALIGNMENT if
 * its w13 or w2 is not 16-byte aligned. */
moe_status moe_decode_forward_shared(const moe_shape* shape, int32_t M,
                                     const uint16_t* hidden, const uint16_t* router_w,
                                     const uint8_t* w13, const uint8_t* w13_scale,
                                     const uint8_t* w2, const uint8_t* w2_scale,
                                     const moe_shared_expert* shared,
                                     float* out, void* ws, size_t ws_bytes, void* stream,
                                     void* const* events);

/* moe_decode_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a static device array
 * inside the library (4 MiB; every GPU that runs the library holds its own
 * copy until the process ends); the call itself allocates nothing.  At the
 * first call on a device the array is zeroed by a fill kernel on `stream`.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (other streams, other host threads) race and give undefined results, so
 * order them.  A call whose workspace would exceed the array
 * (moe_workspace_bytes(shape, M) > 4 MiB, e.g. large M on the chunk path) is
 * MOE_ERR_UNSUPPORTED_SHAPE; otherwise arguments and errors are those of
 * moe_decode_forward. */
moe_status moe_decode_forward_noalloc(const moe_shape* shape, int32_t M,
                                      const uint16_t* hidden, const uint16_t* router_w,
                                      const uint8_t* w13, const uint8_t* w13_scale,
                                      const uint8_t* w2, const uint8_t* w2_scale,
                                      float* out, void* stream);

/* Router, top-K, renormalised weights and compaction (the first kernel of
 * moe_decode_forward; it also quantises the activations when the taps ask
 * for them).  topk_ids/topk_w [M,K] are written in canonical order (logit
 * descending, expert index ascending).  taps may be NULL. */
moe_status moe_route(const moe_shape* shape, int32_t M,
                     const uint16_t* hidden, const uint16_t* router_w,
                     int32_t* topk_ids, float* topk_w, const moe_route_taps* taps,
                     void* ws, size_t ws_bytes, void* stream);

/* Per-token FP8 E4M3 activation quantisation as a kernel of its own (the
 * router kernel produces the same bytes; see moe_route_taps).  No workspace. */
moe_status moe_quant_act(const moe_shape* shape, int32_t M, const uint16_t* hidden,
                         uint8_t* act_fp8, float* act_scale, void* stream);

/* Everything after routing, on caller-given routing (e.g. an oracle's ids and
 * weights for tokens whose K-th and (K+1)-th logits are too close to call):
 * compaction -> gate/up -> requantise -> down + combine, with the same
 * kernels as moe_decode_forward.  taps may be NULL. */
moe_status moe_experts_forward(const moe_shape* shape, int32_t M,
                               const uint8_t* act_fp8, const float* act_scale,
                               const int32_t* topk_ids, const float* topk_w,
                               const uint8_t* w13, const uint8_t* w13_scale,
                               const uint8_t* w2, const uint8_t* w2_scale,
                               float* out, const moe_expert_taps* taps,
                               void* ws, size_t ws_bytes, void* stream);

/* moe_experts_forward plus the shared expert (`shared` may be NULL).  With a
 * shared expert the taps hold M*K + M rows: the M*K routed pairs, then the
 * shared expert's row for token t at M*K + t. */
moe_status moe_experts_forward_shared(const moe_shape* shape, int32_t M,
                                      const uint8_t* act_fp8, const float* act_scale,
                                      const int32_t* topk_ids, const float* topk_w,
                                      const uint8_t* w13, const uint8_t* w13_scale,
                                      const uint8_t* w2, const uint8_t* w2_scale,
                                      const moe_shared_expert* shared,
                                      float* out, const moe_expert_taps* taps,
                                      void* ws, size_t ws_bytes, void* stream);

/* Compaction and the fused gate/up kernel, then the per-(token, expert) FP8
 * requantisation as a kernel of its own (moe_decode_forward does the same
 * arithmetic inside its down kernel): writes h, the E4M3 intermediate and its
 * scales.  All three outputs are required. */
moe_status moe_gate_up(const moe_shape* shape, int32_t M,
                       const uint8_t* act_fp8, const float* act_scale,
                       const int32_t* topk_ids,
                       const uint8_t* w13, const uint8_t* w13_scale,
                       float* h, uint8_t* inter_fp8, float* inter_scale,
                       void* ws, size_t ws_bytes, void* stream);

/* Compaction and the down-projection + combine kernel alone, on a
 * caller-given E4M3 intermediate [M*K, I] and scales [M*K]. */
moe_status moe_down_combine(const moe_shape* shape, int32_t M,
                            const uint8_t* inter_fp8, const float* inter_scale,
                            const int32_t* topk_ids, const float* topk_w,
                            const uint8_t* w2, const uint8_t* w2_scale,
                            float* out, void* ws, size_t ws_bytes, void* stream);

/* The E4M3 encoder the quantisation kernels use, applied to the n binary32
 * values whose bit patterns are first_bits, first_bits+1, ... (wrapping at
 * 2^32): q[i] = E4M3_RNE_satfinite(bits_as_float(first_bits + i)).  For
 * exhaustive checks of the encoder. */
moe_status moe_fp8_encode_range(uint32_t first_bits, int64_t n, uint8_t* q, void* stream);

/* ---- FP8 LM head ----------------------------------------------------------
 * The output projection (hidden 2,560 -> vocabulary 157,184 on the pages) is
 * stored in BF16 and read in full for every token; it is quantised to FP8
 * once at load time so that those reads halve ([EN] "What are the 3
 * optimizations?", item 2).  Reading taken: one fp32 scale per vocabulary row,
 * s_v = amax_k |W[v,k]| / 448 (1 for an all-zero row), codes
 * E4M3_RNE_sat(W[v,k] / s_v) (correctly rounded fp32 divisions: the
 * activation scheme of moe_quant_act applied to weight rows); activations stay
 * bf16. */

/* Load-time quantisation.  w_bf16 [vocab, hidden] row-major (16-byte
 * aligned); q [vocab, hidden] E4M3 codes (16-byte aligned); scale [vocab].
 * hidden % 8 == 0.  Any vocab > 0.  Caller-owned device memory; asynchronous
 * on `stream`; nothing is enqueued on an error. */
moe_status moe_lm_head_quantize(const uint16_t* w_bf16, int32_t vocab, int32_t hidden,
                                uint8_t* q, float* scale, void* stream);

/* Decode GEMV over the FP8 rows: logits[t, v] = scale[v] * sum_k
 * E4M3(q[v,k]) * x[t,k], fp32 accumulation of exact products, for M = 1..8
 * tokens.  x_bf16 [M, hidden] (16-byte aligned); logits [M, vocab] fp32,
 * overwritten.  Compiled hidden sizes: 512 and 2560 (others return
 * MOE_ERR_UNSUPPORTED_SHAPE); any vocab > 0. */
moe_status moe_lm_head_forward(const uint16_t* x_bf16, int32_t M, const uint8_t* q,
                               const float* scale, int32_t vocab, int32_t hidden,
                               float* logits, void* stream);

/* Writes a one-line description of the kernels a call with this shape and M
 * would run (NUL-terminated, truncated to len).  Returns the same status the
 * call's shape validation would. */
moe_status moe_path_info(const moe_shape* shape, int32_t M, char* buf, size_t len);

/* Static description of a status code. */
const char* moe_status_string(moe_status status);

/* The last error message recorded on this thread ("" if none). */
const char* moe_last_error(void);

/* ---- Run-time compilation for other layer shapes --------------------------
 *
 * The kernels above are compiled into this library for (H, I) = (256, 64) and
 * (2560, 768), and the LM-head GEMV for hidden 512 and 2560.  Other shapes get
 * the same kernels compiled at run time with hipRTC for their (H, I) and the
 * GPU, the way the pages' MoE backend compiles per shape and caches the
 * binaries ([EN] "What are the 3 optimizations?", item 1; [ZH]
 * "三项优化分别做了什么").  One module per (H, I) holds the decode-path kernels
 * (M <= 8), the chunk-path kernels where their blocking fits (H % 256 == 0,
 * I % 32 == 0) and the LM-head GEMV for hidden H where it fits (H % 256 == 0,
 * H <= 4096).  Compiled code objects are kept in a cache directory (cache_dir;
 * NULL or "" means $MOE_JIT_CACHE_DIR, else $XDG_CACHE_HOME/moe_decode_jit, else
 * $HOME/.cache/moe_decode_jit), one file per shape named by a 64-bit hash of
 * the kernel sources, compile options, compiler version, target and shape;
 * a file whose header, kernel list or checksum does not match is rebuilt.
 * Files are written to a temporary name and renamed, so concurrent builders
 * never see a partial file.
 *
 * Nothing is compiled implicitly: a call with a shape that has no kernels on
 * the current device fails with MOE_ERR_UNSUPPORTED_SHAPE.  These calls
 * allocate host memory and (load) device code; they are set-up calls, not for
 * stream capture.  The library's module registry is process-wide and
 * thread-safe. */
typedef struct {
    int32_t from_cache;      /* 1: the code object came from the cache file; 0: compiled by this call */
    int32_t has_chunk_path;  /* the module holds the chunk-path kernels (M > 8)                    */
    int32_t has_lm_head;     /* the module holds the LM-head GEMV for hidden H                    */
    int32_t num_kernels;     /* kernels in the module                                              */
    double  seconds;         /* wall time of the call                                              */
    char    cache_file[1024];
} moe_jit_report;

/* Compile the kernels of shape->hidden, shape->inter for `arch` ("gfx950",
 * optionally with ":feature" suffixes) into the cache, or find them there.
 * Needs no GPU (a build farm can fill a cache for later use).  report may be
 * NULL.  MOE_ERR_UNSUPPORTED_SHAPE for a shape without kernel geometry or
 * another target; MOE_ERR_JIT with the compiler log for a failed compile or
 * an unusable cache directory. */
moe_status moe_jit_build(const moe_shape* shape, const char* arch, const char* cache_dir,
                         moe_jit_report* report);

/* moe_jit_build for the current device, then load the module on it; later
 * calls on this device with this (H, I) run its kernels.  prefer != 0 makes
 * them win over compiled-in kernels of the same shape (to check that the two
 * agree); otherwise compiled-in kernels are used where they exist.  Loading a
 * shape again replaces its earlier module on this device (no work using the
 * old one may be pending).  MOE_ERR_HIP if the code object does not load. */
moe_status moe_jit_load(const moe_shape* shape, const char* cache_dir, int32_t prefer,
                        moe_jit_report* report);

/* Unload the module of (H, I) from the current device; returns the number of
 * modules removed (0 or 1).  No work using it may be pending. */
int32_t moe_jit_unload(const moe_shape* shape);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DECODE_H */
