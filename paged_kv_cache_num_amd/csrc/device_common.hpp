// Device helpers shared by the kvpool kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace kvp {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// ---- bfloat16 <-> fp32 -------------------------------------------------------

// Exact widening of the low / high bfloat16 of a packed pair.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bfloat16, round to nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Two-term bfloat16 dot product with fp32 accumulation: a.lo*b.lo + a.hi*b.hi + c.
// Each product of two bfloat16 values is exact in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---- cross-lane sums ---------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum over aligned groups of W consecutive lanes (W in 1..32, a power of two);
// every lane of a group receives the same bits (each step adds two values in
// an order-independent way, so partners compute identical sums).
template <int W>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (W >= 2) x += dpp_f32<kDppQuadSwap1>(x);
    if constexpr (W >= 4) x += dpp_f32<kDppQuadSwap2>(x);
    if constexpr (W >= 8) x += dpp_f32<kDppRowHalfMirror>(x);   // after the quad steps: the other quad
    if constexpr (W >= 16) x += dpp_f32<kDppRowMirror>(x);      // the other half-row
    if constexpr (W >= 32) x += __shfl_xor(x, 16, kWave);
    static_assert(W <= 32, "group wider than half a wave");
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- streaming loads ---------------------------------------------------------

// Loads of data read once per call, with the nontemporal hint (global_load
// ... nt): the lines are not kept in the caches at the expense of data that is
// reused.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_stream(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint2 load_stream(const uint2* p) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(v.x, v.y);
}

}  // namespace kvp
