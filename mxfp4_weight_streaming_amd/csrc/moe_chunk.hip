// moe_chunk.hip -- host launchers of the chunk-path kernels in
// chunk_kernels.hpp (9..2048 tokens).
#include <hip/hip_ext.h>
#include <stdio.h>

#include "chunk_kernels.hpp"
#include "kernel_table.hpp"
#include "moe_internal.hpp"

namespace moe {

size_t sort_lds_bytes(int M, int K, int E)
{
    const int P = M * K;
    int NP = 64;
    while (NP < P) NP <<= 1;
    const size_t mask_words = (size_t)E * (((M + 31) / 32) | 1);   // odd row stride (sort_pairs_kernel)
    return 4 * (mask_words > (size_t)NP ? mask_words : (size_t)NP);
}

// ---------------------------------------------------------------------------
// Ahead-of-time instantiations: (H, I) in {(256, 64), (2560, 768)}.  Other
// shapes run kernels compiled at run time.
// ---------------------------------------------------------------------------
#define MOE_CHUNK_SHAPE(H, I)                                                                    \
    {key_chunk_router(H), (const void*)chunk_router_kernel<H>},                                 \
    {key_chunk_gate_up(H, I), (const void*)chunk_gate_up_kernel<H, I>},                         \
    {key_chunk_down(H, I, false), (const void*)chunk_down_kernel<H, I, false>},                 \
    {key_chunk_down(H, I, true), (const void*)chunk_down_kernel<H, I, true>},                   \
    {key_combine(H), (const void*)combine_kernel<H>},

const AotKernel kChunkAot[] = {MOE_CHUNK_SHAPE(256, 64) MOE_CHUNK_SHAPE(2560, 768)};
const int kChunkAotCount = (int)(sizeof(kChunkAot) / sizeof(kChunkAot[0]));
#undef MOE_CHUNK_SHAPE

template <typename F, typename... Args>
static hipError_t launch(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s, const LaunchEvents& ev,
                         Args... args)
{
    if (ev.start != nullptr || ev.stop != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, block, lds, s, ev.start, ev.stop, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
    return hipGetLastError();
}

// The chunk path has kernels for (H, I) (compiled in, or loaded at run time)
// and E splits into 16-expert router tiles.
bool chunk_shape_supported(int H, int I, int E)
{
    return chunk_shape_ok(H, I) && E % 16 == 0 && find_kernel(key_chunk_gate_up(H, I)).ok();
}

hipError_t launch_chunk_router(int H, const ChunkRouterArgs& a, hipStream_t s, const LaunchEvents& ev)
{
    const Kern k = find_kernel(key_chunk_router(H));
    if (!k.ok()) return hipErrorInvalidDeviceFunction;
    const dim3 grid((unsigned)(((a.M + 15) / 16) * (a.E / 16)));
    return launch_kern(k, grid, dim3(kRouterWaves * kWave), 0, s, ev, a);
}

hipError_t launch_chunk_topk(const ChunkTopkArgs& a, hipStream_t s, const LaunchEvents& ev)
{
    if (a.act_q != nullptr) {
        if (a.H > kTopkQuantMaxH || a.H % 8 != 0) return hipErrorInvalidValue;
        return launch(chunk_topk_kernel<true>, dim3((a.M + 3) / 4), dim3(256), 0, s, ev, a);
    }
    return launch(chunk_topk_kernel<false>, dim3((a.M + 3) / 4), dim3(256), 0, s, ev, a);
}

hipError_t launch_sort_pairs(const SortArgs& a, hipStream_t s, const LaunchEvents& ev)
{
    if (a.M * a.K > kMaxChunkPairs || a.E > kMaxExperts || a.M > kMaxChunkTokens) return hipErrorInvalidValue;
    const size_t lds = sort_lds_bytes(a.M, a.K, a.E);
    if (lds > 64 * 1024) {   // above the default dynamic-LDS limit (gfx950 has 160 KiB per CU)
        const hipError_t err = hipFuncSetAttribute((const void*)sort_pairs_kernel,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
    }
    return launch(sort_pairs_kernel, dim3(1), dim3(kSortThreads), (uint32_t)lds, s, ev, a);
}

hipError_t launch_chunk_gate_up(int H, int I, int C, const ChunkGateUpArgs& a, hipStream_t s, const LaunchEvents& ev)
{
    const Kern k = find_kernel(key_chunk_gate_up(H, I));
    if (!k.ok()) return hipErrorInvalidDeviceFunction;
    return launch_kern(k, dim3((unsigned)(C * (I / kGuRows))), dim3(256), 0, s, ev, a);
}

hipError_t launch_chunk_down(int H, int I, int C, const ChunkDownArgs& a, hipStream_t s, const LaunchEvents& ev)
{
    const Kern k = find_kernel(key_chunk_down(H, I, a.by_pair != 0));
    if (!k.ok()) return hipErrorInvalidDeviceFunction;
    return launch_kern(k, dim3((unsigned)(C * (H / kDnRows))), dim3(256), 0, s, ev, a);
}

hipError_t launch_combine(int H, const CombineArgs& a, hipStream_t s, const LaunchEvents& ev)
{
    const Kern k = find_kernel(key_combine(H));
    if (!k.ok()) return hipErrorInvalidDeviceFunction;
    const int total = a.M * (H / 4);
    const int blocks = (total + 255) / 256;
    return launch_kern(k, dim3((unsigned)(blocks < 2048 ? blocks : 2048)), dim3(256), 0, s, ev, a);
}

hipError_t launch_gather_rows(const void* src, void* dst, const int32_t* pos_of, int P, int row_bytes, hipStream_t s)
{
    if (P <= 0 || row_bytes <= 0) return hipSuccess;
    if (row_bytes % 4 != 0) return hipErrorInvalidValue;
    const int words = row_bytes / 4;
    const int64_t total = (int64_t)P * words;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s,
                       static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), pos_of, P, words);
    return hipGetLastError();
}

void chunk_kernel_names(int H, int I, char* buf, size_t n)
{
    const Kern k = find_kernel(key_chunk_gate_up(H, I));
    snprintf(buf, n,
             "chunk_router_kernel<H=%d> (bf16 MFMA 16x16x32) -> %s -> "
             "sort_pairs_kernel (1 workgroup: token bitmasks in LDS) -> chunk_gate_up_kernel<%d,%d> (scaled FP8xFP4 "
             "MFMA 16x16x128, %d workgroups per 64-token chunk, K split over %d waves) -> requant_kernel<%d> -> "
             "chunk_down_kernel<%d,%d> (scaled FP8xFP4 MFMA, %d workgroups per chunk) -> combine_kernel<%d>%s",
             H, H <= kTopkQuantMaxH ? "chunk_topk_kernel (top-K + FP8 quantisation)" : "quant_kernel -> chunk_topk_kernel",
             H, I, I / kGuRows, chunk_k_split(H), I, H, I, H / kDnRows, H,
             k.jit != nullptr ? " [compiled at run time]" : "");
}

}  // namespace moe
