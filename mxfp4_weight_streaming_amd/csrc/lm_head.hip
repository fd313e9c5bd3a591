// lm_head.hip -- host launchers of the FP8 LM-head kernels in
// lm_head_kernels.hpp.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kernel_table.hpp"
#include "lm_head_kernels.hpp"
#include "moe_internal.hpp"

namespace moe {

// Ahead-of-time instantiations: hidden 512 and 2560, token bounds 1, 2, 4, 8.
#define MOE_LMH_SHAPE(H)                                                                                   \
    {key_lm_head(H, 1), (const void*)lm_head_gemv_kernel<H, 1>}, {key_lm_head(H, 2), (const void*)lm_head_gemv_kernel<H, 2>}, \
    {key_lm_head(H, 4), (const void*)lm_head_gemv_kernel<H, 4>}, {key_lm_head(H, 8), (const void*)lm_head_gemv_kernel<H, 8>},

const AotKernel kLmHeadAot[] = {MOE_LMH_SHAPE(512) MOE_LMH_SHAPE(2560)};
const int kLmHeadAotCount = (int)(sizeof(kLmHeadAot) / sizeof(kLmHeadAot[0]));
#undef MOE_LMH_SHAPE

// The GEMV exists for hidden size H: compiled in, or loaded at run time.
bool lm_head_shape_supported(int H) { return lm_head_shape_ok(H) && find_kernel(key_lm_head(H, 1)).ok(); }

hipError_t launch_lm_head_quant(const uint16_t* w, int V, int H, uint8_t* q, float* scale, hipStream_t s)
{
    if (V <= 0) return hipSuccess;
    hipLaunchKernelGGL(lm_head_quant_kernel, dim3((unsigned)((V + 3) / 4)), dim3(256), 0, s, w, V, H, q, scale);
    return hipGetLastError();
}

hipError_t launch_lm_head_gemv(int H, int mt, const uint16_t* x, int M, const uint8_t* q, const float* scale, int V,
                               float* logits, hipStream_t s)
{
    const Kern k = find_kernel(key_lm_head(H, mt));
    if (!k.ok()) return hipErrorInvalidDeviceFunction;
    // as many workgroups as are resident at once (every one striding over the
    // row blocks): a workgroup queued behind a full compute unit would start
    // only when another ends, and the last ones would run alone
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = k.aot != nullptr ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k.aot, 256, 0)
                             : hipModuleOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k.jit, 256, 0);
    if (e != hipSuccess) return e;
    const int blocks = (V + 15) / 16, resident = std::max(per_cu, 1) * std::max(cus, 1);
    const int grid = blocks < resident ? blocks : resident;
    return launch_kern(k, dim3(grid), dim3(256), 0, s, {}, x, M, q, scale, V, logits);
}

}  // namespace moe
