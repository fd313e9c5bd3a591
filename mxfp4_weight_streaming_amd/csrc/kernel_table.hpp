// kernel_table.hpp -- the kernels templated on the layer shape, looked up by
// kind and template arguments.  A kernel is either an instantiation compiled
// ahead of time into this library or one compiled at run time for a shape
// (jit.hip) and loaded on a device; both come from the same device headers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>

#include "moe_internal.hpp"

namespace moe {

enum class KernelKind : int {
    Quant = 0,    // quant_kernel<H>
    Router,       // router_kernel<H, MT>                    v = MT
    GateUp,       // gate_up_kernel<H, I, MT>                v = MT
    Down,         // down_kernel<H, I, MT, FROM_H>           v = 2 MT + FROM_H
    Requant,      // requant_kernel<I>
    ChunkRouter,  // chunk_router_kernel<H>
    ChunkGateUp,  // chunk_gate_up_kernel<H, I>
    ChunkDown,    // chunk_down_kernel<H, I, BY_PAIR>        v = BY_PAIR
    Combine,      // combine_kernel<H>
    LmHead,       // lm_head_gemv_kernel<H, MT>              v = MT
    Layer,        // layer_kernel<H, I, MT>                  v = MT
};

// H or I is 0 for a kernel templated on the other one only.
struct KernelKey {
    KernelKind kind;
    int H, I, v;
};

inline bool same_key(const KernelKey& a, const KernelKey& b)
{
    return a.kind == b.kind && a.H == b.H && a.I == b.I && a.v == b.v;
}

inline KernelKey key_quant(int H) { return {KernelKind::Quant, H, 0, 0}; }
inline KernelKey key_router(int H, int mt) { return {KernelKind::Router, H, 0, mt}; }
inline KernelKey key_gate_up(int H, int I, int mt) { return {KernelKind::GateUp, H, I, mt}; }
inline KernelKey key_down(int H, int I, int mt, bool from_h) { return {KernelKind::Down, H, I, 2 * mt + (from_h ? 1 : 0)}; }
inline KernelKey key_requant(int I) { return {KernelKind::Requant, 0, I, 0}; }
inline KernelKey key_chunk_router(int H) { return {KernelKind::ChunkRouter, H, 0, 0}; }
inline KernelKey key_chunk_gate_up(int H, int I) { return {KernelKind::ChunkGateUp, H, I, 0}; }
inline KernelKey key_chunk_down(int H, int I, bool by_pair) { return {KernelKind::ChunkDown, H, I, by_pair ? 1 : 0}; }
inline KernelKey key_combine(int H) { return {KernelKind::Combine, H, 0, 0}; }
inline KernelKey key_lm_head(int H, int mt) { return {KernelKind::LmHead, H, 0, mt}; }
inline KernelKey key_layer(int H, int I, int mt) { return {KernelKind::Layer, H, I, mt}; }

// The kernel's qualified template-id, e.g. "moe::gate_up_kernel<2560, 768, 1>"
// (the name expression hipRTC resolves).  Returns false for an unknown kind.
bool kernel_expr(const KernelKey& k, char* buf, size_t n);

struct AotKernel {
    KernelKey key;
    const void* fn;   // host stub of the ahead-of-time instantiation
};

// The ahead-of-time instantiations of each translation unit.
extern const AotKernel kGemvAot[];
extern const int kGemvAotCount;
extern const AotKernel kChunkAot[];
extern const int kChunkAotCount;
extern const AotKernel kLmHeadAot[];
extern const int kLmHeadAotCount;

struct Kern {
    const void* aot = nullptr;
    hipFunction_t jit = nullptr;
    bool ok() const { return aot != nullptr || jit != nullptr; }
};

// A module loaded with preference on the current device, else the
// ahead-of-time instantiation, else a module loaded on the current device;
// an empty Kern when none has it.
Kern find_kernel(const KernelKey& k);

// Launch with by-value arguments whose types are exactly the kernel's
// parameter types.  With start/stop events the launch stamps them with the
// kernel's own execution interval.
template <typename... A>
hipError_t launch_kern(const Kern& k, dim3 grid, dim3 block, uint32_t lds, hipStream_t s, const LaunchEvents& ev,
                       A... args)
{
    void* argv[] = {static_cast<void*>(&args)...};
    const bool timed = ev.start != nullptr || ev.stop != nullptr;
    if (k.jit != nullptr) {
        if (timed)
            return hipExtModuleLaunchKernel(k.jit, grid.x * block.x, grid.y * block.y, grid.z * block.z, block.x,
                                            block.y, block.z, lds, s, argv, nullptr, ev.start, ev.stop, 0);
        return hipModuleLaunchKernel(k.jit, grid.x, grid.y, grid.z, block.x, block.y, block.z, lds, s, argv, nullptr);
    }
    if (k.aot == nullptr) return hipErrorInvalidDeviceFunction;
    if (timed) return hipExtLaunchKernel(k.aot, grid, block, argv, lds, s, ev.start, ev.stop, 0);
    return hipLaunchKernel(k.aot, grid, block, argv, lds, s);
}

}  // namespace moe
