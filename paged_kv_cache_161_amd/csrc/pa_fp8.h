// pa_fp8.h -- the OCP FP8 E4M3 encoder shared by the cache writes (append, and the
// decode that appends its own new row).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// fp32 -> E4M3 code by bit arithmetic on the binary32 encoding: round the 23-bit
// fraction to 3 bits (nearest, ties to even) and rebias the exponent 127 -> 7; below
// 2^-6 the code counts steps of 2^-9; NaN stays NaN, |x| >= 448 gives +-448.
__device__ __forceinline__ uint32_t e4m3_code(float x)
{
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u)
        return sign | 0x7Fu;                              // NaN
    if (a >= 0x43E00000u)
        return sign | 0x7Eu;                              // >= 448 (and inf): 448
    if (a < 0x3C800000u)                                  // < 2^-6: subnormal codes
        return sign | (uint32_t)rintf(__uint_as_float(a) * 512.0f);
    const uint32_t rounded = a + 0x7FFFFu + ((a >> 20) & 1u);
    return sign | ((rounded >> 20) - (120u << 3));
}

// E4M3 code of x / scale, the division in IEEE fp32; a scale that is not finite and
// > 0 (a bad per-head scale) gives the NaN code.
__device__ __forceinline__ uint32_t e4m3_scaled(float x, float scale)
{
    return (scale > 0.f && scale <= 3.402823466e38f) ? e4m3_code(__fdiv_rn(x, scale)) : 0x7Fu;
}

// A 16-bit activation element (bf16 bits when bf16, else f16 bits) -> E4M3 code of
// x / scale.
__device__ __forceinline__ uint32_t e4m3_of_16(uint32_t bits, bool bf16, float scale)
{
    const float x = bf16 ? __uint_as_float(bits << 16)
                         : (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
    return e4m3_scaled(x, scale);
}

}  // namespace pa
