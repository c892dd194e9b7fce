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

#include "device_common.hpp"

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
// multiples of 2^-9, so the code is x * 2^9 rounded to an integer.  Both
// candidates are computed and selected, without branches.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    // below 2^-6: subnormal codes 0..8 (the input clamped so the conversion stays in range)
    const uint32_t sub = (uint32_t)__builtin_rintf(fminf(__uint_as_float(a), 0.015625f) * 512.0f);
    // from 2^-6: biased exponent 1..15 and three mantissa bits, round to nearest even
    const uint32_t m = a & 0x7FFFFFu;
    const uint32_t rest = m & 0xFFFFFu;                // the 20 dropped mantissa bits
    uint32_t code = (((a >> 23) - 120u) << 3) | (m >> 20);
    code += (rest > 0x80000u || (rest == 0x80000u && (code & 1u))) ? 1u : 0u;
    uint32_t r = a < 0x3C800000u ? sub : code;         // 2^-6
    r = a >= 0x43E00000u ? 0x7Eu : r;                  // >= 448
    return a > 0x7F800000u ? 0x7Fu : (sign | r);       // NaN
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

// max(m, |lo|, |hi|) of a packed bfloat16 pair.
__device__ __forceinline__ float abs_max2(uint32_t w, float m) {
    return fmaxf(m, fmaxf(fabsf(bf16_lo(w)), fabsf(bf16_hi(w))));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
    return x;
}

// One wave writes one new head row (128 bf16 values, lane l: dims 2l and
// 2l + 1) into an FP8 pool row `dst` (128 codes).  When the row is row 0 of
// its block (`opens`), it alone sets the block's scale first; otherwise the
// stored scale is used.
__device__ __forceinline__ void fp8_store_row(const uint32_t* __restrict__ src, uint16_t* dst, float* scale,
                                              bool opens, int lane) {
    const uint32_t w = src[lane];
    float s;
    if (opens) {
        s = e4m3_block_scale(wave_max(abs_max2(w, 0.0f)));
        if (lane == 0) *scale = s;
    } else {
        s = *scale;
    }
    dst[lane] = (uint16_t)bf16x2_to_e4m3x2(w, s);
}

}  // namespace kvp
