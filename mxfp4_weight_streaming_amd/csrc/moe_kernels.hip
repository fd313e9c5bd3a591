// moe_kernels.hip -- host launchers of the decode-path kernels in
// gemv_kernels.hpp: grid geometry, the dynamic-LDS sizes and the choice of the
// ahead-of-time instantiation or a kernel compiled at run time.
#include <hip/hip_ext.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "gemv_kernels.hpp"
#include "layer_kernels.hpp"
#include "kernel_table.hpp"
#include "moe_internal.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Ahead-of-time instantiations: (H, I) in {(256, 64), (2560, 768)} with token
// bounds 1, 2, 4 and 8.  Other shapes run kernels compiled at run time.
// ---------------------------------------------------------------------------
#define MOE_GEMV_MT(H, I, MT)                                                                    \
    {key_router(H, MT), (const void*)router_kernel<H, MT>},                                     \
    {key_gate_up(H, I, MT), (const void*)gate_up_kernel<H, I, MT>},                             \
    {key_down(H, I, MT, true), (const void*)down_kernel<H, I, MT, true>},                       \
    {key_down(H, I, MT, false), (const void*)down_kernel<H, I, MT, false>},
#define MOE_LAYER_MT(H, I, MT) {key_layer(H, I, MT), (const void*)layer_kernel<H, I, MT>},
#define MOE_GEMV_SHAPE(H, I)                                                                     \
    {key_quant(H), (const void*)quant_kernel<H>}, {key_requant(I), (const void*)requant_kernel<I>}, \
    MOE_GEMV_MT(H, I, 1) MOE_GEMV_MT(H, I, 2) MOE_GEMV_MT(H, I, 4) MOE_GEMV_MT(H, I, 8)          \
    MOE_LAYER_MT(H, I, 1) MOE_LAYER_MT(H, I, 2) MOE_LAYER_MT(H, I, 4) MOE_LAYER_MT(H, I, 8)

const AotKernel kGemvAot[] = {MOE_GEMV_SHAPE(256, 64) MOE_GEMV_SHAPE(2560, 768)};
const int kGemvAotCount = (int)(sizeof(kGemvAot) / sizeof(kGemvAot[0]));
#undef MOE_GEMV_SHAPE
#undef MOE_GEMV_MT
#undef MOE_LAYER_MT

// The decode path has kernels for (H, I): compiled in, or loaded at run time.
bool gemv_shape_supported(int H, int I)
{
    return gemv_shape_ok(H, I) && find_kernel(key_gate_up(H, I, 1)).ok();
}

hipError_t launch_router(int H, int mt, const RouterArgs& a, hipStream_t s, const LaunchEvents& ev)
{
    const Kern k = find_kernel(key_router(H, mt));
    if (!k.ok()) return hipErrorInvalidDeviceFunction;
    // one workgroup per expert row, one thread per 16-byte chunk of it
    return launch_kern(k, dim3(a.E), dim3(router_threads(H)), 0, s, ev, a);
}

hipError_t launch_quant(int H, const uint16_t* x, int M, uint8_t* q, float* sc, hipStream_t s)
{
    const Kern k = find_kernel(key_quant(H));
    if (!k.ok()) return hipErrorInvalidDeviceFunction;
    return launch_kern(k, dim3(M), dim3(256), 0, s, {}, x, q, sc);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s)
{
    hipLaunchKernelGGL(topk_kernel, dim3(1), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gate_up(int H, int I, int mt, int S, const GateUpArgs& a, hipStream_t s, const LaunchEvents& ev)
{
    const Kern k = find_kernel(key_gate_up(H, I, mt));
    if (!k.ok()) return hipErrorInvalidDeviceFunction;
    // one workgroup per (expert, row block) up to two per CU; beyond that the
    // workgroups loop over their items with the next item's loads in flight
    const int items = S * (I / gate_up_rows_per_block(H));
    const int grid = items < 512 ? items : 512;
    return launch_kern(k, dim3(grid), dim3(256), 0, s, ev, a);
}

hipError_t launch_down(int H, int I, int mt, const DownArgs& a, hipStream_t s, const LaunchEvents& ev)
{
    // the shared expert's rows come only from h (the caller-given q2 path is routed-only)
    if (a.sh.w2 != nullptr && a.h == nullptr) return hipErrorInvalidValue;
    const Kern k = find_kernel(key_down(H, I, mt, a.h != nullptr));
    if (!k.ok()) return hipErrorInvalidDeviceFunction;
    // the intermediate as f16, and afterwards the lanes' sums (8 waves x mt tokens x row passes x 64 lanes)
    const size_t lds = std::max((size_t)(a.M * a.K + (a.sh.w2 != nullptr ? a.M : 0)) * I * 2,
                                (size_t)8 * mt * down_row_passes(H, I) * kWaveSize * sizeof(float));
    if (lds > kMaxDynamicLds) return hipErrorInvalidValue;
    if (lds > 64 * 1024 && k.aot != nullptr) {   // above the default dynamic-LDS limit of a compiled kernel
        hipError_t err = hipFuncSetAttribute(k.aot, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
    }
    return launch_kern(k, dim3(H / down_rows_per_block(H, I)), dim3(512), (uint32_t)lds, s, ev, a);
}

// ---------------------------------------------------------------------------
// The one-kernel layer.
// ---------------------------------------------------------------------------
bool layer_shape_supported(int H, int I)
{
    return layer_shape_ok(H, I) && find_kernel(key_layer(H, I, 1)).ok();
}

namespace {
std::atomic<uint32_t> g_layer_wait_us{0};
constexpr uint32_t kDefaultLayerWaitUs = 200000;   // 0.2 s: far above any real wait

struct DeviceFacts {
    int cus = 0;
    uint64_t wall_khz = 0;
};
std::mutex g_facts_mu;
DeviceFacts g_facts[64];

hipError_t device_facts(DeviceFacts* out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_facts_mu);
    DeviceFacts& f = g_facts[dev];
    if (f.cus == 0) {
        int cus = 0, khz = 0;
        if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        if ((e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev)) != hipSuccess) return e;
        f.wall_khz = khz > 0 ? (uint64_t)khz : 100000;
        f.cus = cus > 0 ? cus : 1;
    }
    *out = f;
    return hipSuccess;
}
}  // namespace

void set_layer_wait_us(uint32_t us) { g_layer_wait_us.store(us); }

hipError_t launch_layer(int H, int I, int mt, LayerArgs a, hipStream_t s, const LaunchEvents& ev)
{
    const Kern k = find_kernel(key_layer(H, I, mt));
    if (!k.ok()) return hipErrorInvalidDeviceFunction;
    DeviceFacts d;
    hipError_t e = device_facts(&d);
    if (e != hipSuccess) return e;
    const uint32_t us = g_layer_wait_us.load();
    if (a.wait_ticks == 0) a.wait_ticks = (uint64_t)(us ? us : kDefaultLayerWaitUs) * d.wall_khz / 1000u;
    // one workgroup per compute unit (all resident at once: the workgroups
    // wait for each other), and no more than the work has tasks for
    const int slots = std::min(a.E, a.M * a.K) + (a.shared ? 1 : 0);
    const int need = std::max({slots * layer_gate_up_tasks(H, I), slots * layer_down_tasks(H, I), a.E, 1});
    const int nb = std::min({d.cus, need, kMaxLayerBlocks});
    // the LDS request keeps one workgroup per compute unit
    const int pe = a.M * a.K + (a.shared ? a.M : 0);
    const size_t lds = std::max(layer_lds_bytes(H, I, mt, pe), kLayerMinLds);
    if (lds > kLayerMaxDynLds) return hipErrorInvalidValue;
    if (lds > 64 * 1024 && k.aot != nullptr) {
        e = hipFuncSetAttribute(k.aot, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    return launch_kern(k, dim3(nb), dim3(512), (uint32_t)lds, s, ev, a);
}

hipError_t launch_requant(int I, const RequantArgs& a, hipStream_t s)
{
    if (a.P <= 0) return hipSuccess;
    const Kern k = find_kernel(key_requant(I));
    if (!k.ok()) return hipErrorInvalidDeviceFunction;
    return launch_kern(k, dim3((a.P + 3) / 4), dim3(256), 0, s, {}, a);
}

hipError_t launch_fp8_encode_range(uint32_t first, int64_t n, uint8_t* q, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    const int64_t blocks64 = (n + 255) / 256;
    const int blocks = (int)(blocks64 < 16384 ? blocks64 : 16384);
    hipLaunchKernelGGL(fp8_encode_range_kernel, dim3(blocks), dim3(256), 0, s, first, n, q);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s)
{
    if (n == 0) return hipSuccess;
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

void layer_kernel_names(int H, int I, char* buf, size_t n)
{
    const Kern k = find_kernel(key_layer(H, I, 1));
    DeviceFacts d;
    const int cus = device_facts(&d) == hipSuccess ? d.cus : 0;
    snprintf(buf, n,
             "layer_kernel<H=%d,I=%d> (one kernel: router, top-K, FP8 quantisation, compaction, gate/up, "
             "requantisation, down, combine; up to %d workgroups of 512 threads, one per compute unit, handing off "
             "through epoch-tagged words; gate/up tasks of %d row pairs, down tasks of %d rows)%s",
             H, I, cus, kWaveSize / gate_up_lanes_per_row(H), layer_down_rows_per_pass(I) * layer_down_passes(H, I),
             k.jit != nullptr ? " [compiled at run time]" : "");
}

void kernel_names(int H, int I, char* buf, size_t n)
{
    const Kern k = find_kernel(key_gate_up(H, I, 1));
    const int lg = gate_up_lanes_per_row(H), ld = down_lanes_per_row(H, I);
    snprintf(buf, n,
             "router_kernel<H=%d> -> gate_up_kernel<H=%d,I=%d> (routing prologue; %d lanes/row, %d row-pairs per "
             "item, %d items/expert, up to 512 WGs) -> down_kernel<H=%d,I=%d> (FP8 requantisation prologue; %d "
             "lanes/row, %d rows/WG in %d passes, %d WGs)%s",
             H, H, I, lg, gate_up_rows_per_block(H), I / gate_up_rows_per_block(H), H, I, ld, down_rows_per_block(H, I),
             down_row_passes(H, I), H / down_rows_per_block(H, I), k.jit != nullptr ? " [compiled at run time]" : "");
}

}  // namespace moe
