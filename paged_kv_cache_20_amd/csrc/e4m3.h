// e4m3.h -- the OCP E4M3 ("E4M3FN") codec shared by the kernels that write
// fp8 pages: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
// infinities, S.1111.111 is NaN, exponent 0 is subnormal m * 2^-9.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Nearest E4M3 code, ties to even, |y| > 448 -> +-448, NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_code(float y)
{
    const uint32_t bits = __float_as_uint(y);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const float a = __builtin_fabsf(y);
    if (a != a)
        return 0x7Fu;
    if (a > 448.f)
        return sign | 0x7Eu;
    if (a < 0.015625f)  // below 2^-6: subnormal codes m * 2^-9, m = 0..8
        return sign | (uint32_t)__builtin_rintf(a * 512.f);
    // Normal: keep 3 mantissa bits with round-to-nearest-even on the fp32
    // pattern, then rebias the exponent from 127 to 7.
    const uint32_t ab = __float_as_uint(a);
    const uint32_t r = (ab + 0x7FFFFu + ((ab >> 20) & 1u)) >> 20;
    return sign | (r - (120u << 3));
}

// Value of an E4M3 code (exact in fp32); NaN for the two NaN codes.
__device__ __forceinline__ float e4m3_value(uint32_t c)
{
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    if ((c & 0x7Fu) == 0x7Fu)
        return __builtin_nanf("");
    const float v = e == 0 ? (float)m * 0.001953125f  // m * 2^-9
                           : __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (c & 0x80u) ? -v : v;
}

}  // namespace pa
