// device_common.hpp -- number formats and wave helpers shared by the gfx950 kernels.
//
// Formats (the pages name MXFP4 weights and FP8 activations but do not define
// them; these follow the OCP MX v1.0 and OCP OFP8 definitions):
//   E2M1  : decoded by the gfx950 scaled-conversion instruction
//           (v_cvt_scalef32_pk_f16_fp4), two codes per byte, low nibble first.
//   E8M0  : 2^(code-127), applied to fp32 block sums with v_ldexp_f32 (exact).
//   E4M3  : OCP "FN" variant (bias 7, no infinity, max 448), encoded here with
//           integer round-to-nearest-even and saturation to 448.
#pragma once

#ifndef __HIPCC_RTC__
#include <hip/hip_runtime.h>
#endif
#include <stdint.h>

namespace moe {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// E4M3 encode: nearest finite value, ties to the even code, |y| > 448 -> 448,
// sign kept (-0 -> 0x80); NaN -> 0x7F.  gfx950's v_cvt_pk_fp8_f32 converts to
// OCP E4M3 with round-to-nearest-even; clamping to +-448 first (v_med3) gives
// the saturating behaviour.
__device__ __forceinline__ uint32_t e4m3_encode(float y)
{
    if (y != y) return 0x7Fu;
    const float c = __builtin_amdgcn_fmed3f(y, -448.0f, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}

// fl32(x / s) as far as its E4M3 code goes, for the activation quantisation
// (s = fl32(amax / 448) of a token, r = fl32(1 / s), both once per token):
// the product q0 = x * r corrected once by its residual, fma(x - q0 s, r, q0).
// For every bf16 amax >= 2^-64 and every bf16 x with |x| <= amax the E4M3
// code of this value equals that of the correctly rounded quotient (checked
// on the host over all such pairs; a negative x mirrors a positive one).
// Below that amax (fast false, one decision per token) the residual can lose
// bits, and the division is taken.  The quotient has the sign of x (s > 0):
// copying it keeps -0 (fma(+0, r, -0) is +0).
struct QuantScale {
    float s, r;
    bool fast;
};

__device__ __forceinline__ QuantScale quant_scale(float amax)
{
    const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
    return QuantScale{s, 1.0f / s, !(amax > 0.0f && amax < 0x1p-64f)};
}

__device__ __forceinline__ float quant_div(float x, const QuantScale& q)
{
#pragma clang fp contract(off)
    if (!q.fast) return x / q.s;
    const float q0 = x * q.r;
    return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, q.s, x), q.r, q0), x);
}

// Four values -> four E4M3 codes in one dword (byte i = value i), same
// rounding and saturation (NaN inputs are not expected here).
__device__ __forceinline__ uint32_t e4m3x4_encode(float a, float b, float c, float d)
{
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
    d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Two E4M3 codes (bytes 0,1 when HI is false, 2,3 when true) -> their exact
// values as half2.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_half2(uint32_t codes)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)codes, 1.0f, HI));
}

// 8 E4M3 codes (little-endian in a u32x2) -> 8 halves in a u32x4 (exact).
__device__ __forceinline__ u32x4 e4m3x8_to_half8(u32x2 c)
{
    u32x4 r;
    r.x = e4m3x2_to_half2<false>(c.x);
    r.y = e4m3x2_to_half2<true>(c.x);
    r.z = e4m3x2_to_half2<false>(c.y);
    r.w = e4m3x2_to_half2<true>(c.y);
    return r;
}

// E4M3 code -> fp32 value (exact).
__device__ __forceinline__ float e4m3_decode(uint32_t c)
{
    const uint32_t em = c & 0x7Fu;
    const float mag = (em >= 8u) ? __uint_as_float((em + (120u << 3)) << 20)
                                 : (float)em * 0.001953125f;          // m * 2^-9
    return __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
}

__device__ __forceinline__ half2_t as_half2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// One dword of 8 E2M1 codes -> 4 half2 (true values, elements 2b and 2b+1 of byte b).
__device__ __forceinline__ void e2m1x8_to_half(uint32_t d, half2_t* o)
{
    o[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0);
    o[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1);
    o[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2);
    o[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3);
}

// Dot product of one 32-element MXFP4 block (16 bytes of codes, decoded) with
// 32 f16 activations held as four u32x4 (8 halves each), in fp32.  Two
// accumulators shorten the dependent chain.
__device__ __forceinline__ float block_dot(const half2_t* w, u32x4 a0, u32x4 a1, u32x4 a2, u32x4 a3)
{
    float s0 = 0.0f, s1 = 0.0f;
    s0 = __builtin_amdgcn_fdot2(w[0], as_half2(a0.x), s0, false);
    s1 = __builtin_amdgcn_fdot2(w[1], as_half2(a0.y), s1, false);
    s0 = __builtin_amdgcn_fdot2(w[2], as_half2(a0.z), s0, false);
    s1 = __builtin_amdgcn_fdot2(w[3], as_half2(a0.w), s1, false);
    s0 = __builtin_amdgcn_fdot2(w[4], as_half2(a1.x), s0, false);
    s1 = __builtin_amdgcn_fdot2(w[5], as_half2(a1.y), s1, false);
    s0 = __builtin_amdgcn_fdot2(w[6], as_half2(a1.z), s0, false);
    s1 = __builtin_amdgcn_fdot2(w[7], as_half2(a1.w), s1, false);
    s0 = __builtin_amdgcn_fdot2(w[8], as_half2(a2.x), s0, false);
    s1 = __builtin_amdgcn_fdot2(w[9], as_half2(a2.y), s1, false);
    s0 = __builtin_amdgcn_fdot2(w[10], as_half2(a2.z), s0, false);
    s1 = __builtin_amdgcn_fdot2(w[11], as_half2(a2.w), s1, false);
    s0 = __builtin_amdgcn_fdot2(w[12], as_half2(a3.x), s0, false);
    s1 = __builtin_amdgcn_fdot2(w[13], as_half2(a3.y), s1, false);
    s0 = __builtin_amdgcn_fdot2(w[14], as_half2(a3.z), s0, false);
    s1 = __builtin_amdgcn_fdot2(w[15], as_half2(a3.w), s1, false);
    return s0 + s1;
}

__device__ __forceinline__ float ldexp_e8m0(float v, uint32_t code)
{
    return __builtin_amdgcn_ldexpf(v, (int)code - 127);
}

template <typename T>
__device__ __forceinline__ T load_stream(const T* p)
{
    return __builtin_nontemporal_load(p);   // weights are read once per call
}

// Workgroup barrier for data handed over in LDS only.  __syncthreads also
// releases global memory: with a global store in flight it waits for the
// whole vector-memory counter, which on gfx950 counts loads and stores in
// issue order, so it waits for every load in flight as well (the next tile's
// operands, say).  Here only this wave's LDS operations are waited for.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Cross-lane helpers on DPP (no LDS round trip): four steps reduce each row of
// 16 lanes (xor 1, xor 2, half-row mirror, row mirror), then the four row
// results are read as scalars and combined in a fixed order, so every lane
// gets the same, deterministic result.
enum : int { kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140 };

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

__device__ __forceinline__ float row_lane(float v, int lane)
{
    return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), lane));
}

__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    v += dpp_f32<kDppHalfMirror>(v);
    v += dpp_f32<kDppMirror>(v);
    return (row_lane(v, 0) + row_lane(v, 16)) + (row_lane(v, 32) + row_lane(v, 48));
}

__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp_f32<kDppXor1>(v));
    v = fmaxf(v, dpp_f32<kDppXor2>(v));
    v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f32<kDppMirror>(v));
    return fmaxf(fmaxf(row_lane(v, 0), row_lane(v, 16)), fmaxf(row_lane(v, 32), row_lane(v, 48)));
}

// Sum over aligned groups of N lanes (N = 1, 2, 4, 8 or 16); every lane of a
// group gets the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group of 1..16 lanes");
    if constexpr (N >= 2) v += dpp_f32<kDppXor1>(v);
    if constexpr (N >= 4) v += dpp_f32<kDppXor2>(v);
    if constexpr (N >= 8) v += dpp_f32<kDppHalfMirror>(v);
    if constexpr (N >= 16) v += dpp_f32<kDppMirror>(v);
    return v;
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v)
{
    return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}

__device__ __forceinline__ uint64_t read_lane_u64(uint64_t v, int lane)
{
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// The row results of a 32-bit reduction are combined across rows on DPP as
// well: row_bcast:15 gives rows 1 and 3 the combination with the row before,
// row_bcast:31 gives rows 2 and 3 the combination with rows 0-1, so lane 63
// ends with the whole wave's result (one readlane instead of four).
enum : int { kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143 };

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32_rows(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWS, 0xF, false);
}

// Wave-wide maximum of an unsigned 32-bit value (uniform result).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u32<kDppXor1>(v));
    v = max(v, dpp_u32<kDppXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    v = max(v, dpp_u32<kDppMirror>(v));
    v = max(v, dpp_u32_rows<kDppRowBcast15, 0xA>(v));
    v = max(v, dpp_u32_rows<kDppRowBcast31, 0xC>(v));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Wave-wide minimum of an unsigned 32-bit value (uniform result).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
    v = min(v, dpp_u32<kDppXor1>(v));
    v = min(v, dpp_u32<kDppXor2>(v));
    v = min(v, dpp_u32<kDppHalfMirror>(v));
    v = min(v, dpp_u32<kDppMirror>(v));
    v = min(v, dpp_u32_rows<kDppRowBcast15, 0xA>(v));
    v = min(v, dpp_u32_rows<kDppRowBcast31, 0xC>(v));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Wave-wide maximum of a 64-bit key; the result is uniform across the wave.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    v = max_u64(v, dpp_u64<kDppXor1>(v));
    v = max_u64(v, dpp_u64<kDppXor2>(v));
    v = max_u64(v, dpp_u64<kDppHalfMirror>(v));
    v = max_u64(v, dpp_u64<kDppMirror>(v));
    return max_u64(max_u64(read_lane_u64(v, 0), read_lane_u64(v, 16)),
                   max_u64(read_lane_u64(v, 32), read_lane_u64(v, 48)));
}

}  // namespace moe
