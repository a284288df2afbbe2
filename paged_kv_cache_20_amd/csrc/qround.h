// qround.h -- a query vector rounded to E4M3 for the fp8 QK^T of a prefill
// chunk ("Radiance Architecture Plugins -- declaring a model", section
// "Declare: the metadata": the prefill_fp8 bits handed to the attention op).
//
// The vector (one row, one head) is scaled by the smallest power of two 2^e
// with max|q| <= 448 * 2^e (448 = 0.875 * 2^9), e >= -117, and each d-value
// q / 2^e (exact) is rounded to the nearest E4M3 value, ties to even.  The
// lanes n, n + 16, n + 32, n + 48 of a wave hold one vector: lane group kb
// holds d = 128 st + 32 kb + 0..31 of k-step st, byte i of its operand being
// d = 128 st + 32 kb + i (the B operand layout of
// v_mfma_scale_f32_16x16x128_f8f6f4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {
namespace qround {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// q: the vector's bf16 values (null-safe: valid = false reads nothing and
// gives zeros).  Returns 2^e; qf receives the codes.
template <int QS>
__device__ __forceinline__ float round_q(const uint16_t* q, bool valid, int kb, i32x8 (&qf)[QS])
{
    u32x4 raw[QS][4];
    float amax = 0.f;
#pragma unroll
    for (int st = 0; st < QS; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            raw[st][j] = valid ? *(const u32x4*)(q + 128 * st + 32 * kb + 8 * j)
                               : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int w = 0; w < 4; ++w)
                amax = fmaxf(amax, fmaxf(fabsf(lo(raw[st][j][w])), fabsf(hi(raw[st][j][w]))));
        }
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    int e = -117;
    if (amax > 0.f) {
        int ex;
        const float mt = frexpf(amax, &ex);
        e = max(mt <= 0.875f ? ex - 9 : ex - 8, -117);
    }
#pragma unroll
    for (int st = 0; st < QS; ++st)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t w0 = raw[st][j][2 * h], w1 = raw[st][j][2 * h + 1];
                int c = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(lo(w0), -e), ldexpf(hi(w0), -e), 0,
                                                        false);
                c = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(lo(w1), -e), ldexpf(hi(w1), -e), c,
                                                    true);
                qf[st][2 * j + h] = c;
            }
    return ldexpf(1.f, e);
}

}  // namespace qround
}  // namespace pa
