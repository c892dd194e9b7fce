// OCP E4M3 (FP8) codes on gfx950: the conversions the FP8 pool kernels use.
//
// A code is 1 sign bit, 4 exponent bits (bias 7) and 3 mantissa bits; there
// are no infinities, 0x7F / 0xFF are NaN and the largest finite value is 448.
// Every E4M3 value is also a bfloat16 value (8 exponent bits, 7 mantissa
// bits), so widening a code to bfloat16 is exact and the pool's codes can be
// fed to the bf16 matrix-core instructions unchanged in value; the per-block
// scale is applied outside the products.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvp {

constexpr float kE4M3Max = 448.0f;

// Two codes, bytes 2*kHi and 2*kHi + 1 of w, to a packed bfloat16 pair (the
// first byte in the low half).  v_cvt_scalef32_pk_bf16_fp8 with a scale of
// 1.0: exact.
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi));
}

// fp32 -> E4M3 code: round to the nearest E4M3 value, ties to the even code;
// |x| >= 448 saturates to +-448 (0x7E / 0xFE); NaN gives 0x7F.  Written from
// the format's bit fields: above 2^-6 the fp32 exponent is re-biased and the
// mantissa rounded from 23 to 3 bits (a carry out of the mantissa moves to
// the next binade, which is the next code); below 2^-6 the values are the
// multiples of 2^-9, so the code is x * 2^9 rounded to an integer.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return 0x7Fu;               // NaN
    if (a >= 0x43E00000u) return sign | 0x7Eu;       // >= 448
    if (a < 0x3C800000u) {                           // < 2^-6: subnormal codes 0..8
        const float q = __builtin_rintf(__uint_as_float(a) * 512.0f);   // exact scaling, then ties to even
        return sign | (uint32_t)q;
    }
    const uint32_t e = (a >> 23) - 120u;              // E4M3 biased exponent, 1..15
    const uint32_t m = a & 0x7FFFFFu;
    uint32_t code = (e << 3) | (m >> 20);
    const uint32_t rest = m & 0xFFFFFu;               // the 20 dropped mantissa bits
    code += (rest > 0x80000u || (rest == 0x80000u && (code & 1u))) ? 1u : 0u;
    return sign | code;
}

// Quantize a packed bfloat16 pair with a block scale: two codes in the low 16
// bits (the low half's code first).  The division is IEEE fp32 division.
__device__ __forceinline__ uint32_t bf16x2_to_e4m3x2(uint32_t w, float scale) {
    const float lo = __uint_as_float(w << 16);
    const float hi = __uint_as_float(w & 0xFFFF0000u);
    return f32_to_e4m3(lo / scale) | (f32_to_e4m3(hi / scale) << 8);
}

// Block scale from the largest magnitude of the rows that set it.
__device__ __forceinline__ float e4m3_block_scale(float amax) { return amax > 0.0f ? amax / kE4M3Max : 1.0f; }

}  // namespace kvp
