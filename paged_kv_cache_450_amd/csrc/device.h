// Device helpers for gfx950 (wave64): DPP row reductions, 16-bit and FP8
// conversions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pagedkv.h"

namespace pkv {
namespace dev {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- DPP reductions inside groups of N lanes (N in {1,2,4,8,16}) --------
// quad_perm [1,0,3,2] and [2,3,0,1] pair lanes inside a quad; row_half_mirror
// pairs the two quads of an 8-lane half row; row_mirror pairs the two halves of
// a 16-lane row. After log2(N) steps every lane of the group holds the sum.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, true));
}

template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group size");
    if constexpr (N >= 2) x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
    if constexpr (N >= 4) x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
    if constexpr (N >= 8) x += dpp_f32<0x141>(x);  // row_half_mirror
    if constexpr (N >= 16) x += dpp_f32<0x140>(x); // row_mirror
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- 16-bit conversions ---------------------------------------------------
__device__ __forceinline__ float f16_lo(uint32_t w) {
    return static_cast<float>(__builtin_bit_cast(half2_t, w).x);
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
    return static_cast<float>(__builtin_bit_cast(half2_t, w).y);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
    return __builtin_bit_cast(float, w & 0xFFFF0000u);
}

// fp32 -> fp16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// ---- FP8 E4M3 ("fn": bias 7, max 448, NaN = S.1111.111, no inf) ----------
// Two codes (bytes 0,1 or 2,3 of w) to fp32 with the hardware converter; on
// gfx950 the FP8 conversions use the OCP E4M3 format.
__device__ __forceinline__ float2_t e4m3x2_lo(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
}
__device__ __forceinline__ float2_t e4m3x2_hi(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
}

// fp32 -> E4M3 code: nearest finite value, ties to even mantissa, magnitudes
// at or above 448 saturate to 448, sign kept (so tiny negatives give 0x80).
// Written from the format definition with integer operations, so it does not
// depend on the hardware converter's saturation mode.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t mag = u & 0x7FFFFFFFu;
    if (mag > 0x7F800000u) return sign | 0x7Fu;                 // NaN in, NaN out
    const float a = __builtin_bit_cast(float, mag);
    if (a >= 448.0f) return sign | 0x7Eu;                       // saturate (inf too)
    uint32_t code;
    if (a >= 0.015625f) {                                       // normal: a >= 2^-6
        // Keep 3 of 23 mantissa bits, round half to even at bit 20.
        const uint32_t r = mag + 0x7FFFFu + ((mag >> 20) & 1u);
        code = (r >> 20) - (120u << 3);                         // rebias 127 -> 7
    } else {                                                    // subnormal: m * 2^-9
        code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));  // exact scaling, RNE
    }
    return sign | code;
}

// Eight 16-bit source elements (one 16-byte chunk, element e in bytes 2e,
// 2e+1) to eight E4M3 codes (byte e): code = e4m3(fp32(x) / scale), the
// quotient correctly rounded. SRC is PKV_F16 or PKV_BF16.
template <int SRC>
__device__ __forceinline__ uint2 quant_e4m3x8(const uint4& x, float scale) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = (SRC == PKV_F16) ? f16_lo(w[i]) : bf16_lo(w[i]);
        const float b = (SRC == PKV_F16) ? f16_hi(w[i]) : bf16_hi(w[i]);
        const uint32_t ca = f32_to_e4m3(a / scale);
        const uint32_t cb = f32_to_e4m3(b / scale);
        out[i >> 1] |= (ca | (cb << 8)) << ((i & 1) * 16);
    }
    return make_uint2(out[0], out[1]);
}

}  // namespace dev
}  // namespace pkv
