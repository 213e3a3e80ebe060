// spa_device.h -- gfx950 device helpers shared by the bf16 kernels.
//
// MFMA operand layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64, lane l,
// half = l / 32, col = l % 32):
//   A (32 x 16): lane l holds A[col][8*half .. 8*half+7]        (8 bf16, one row)
//   B (16 x 32): lane l holds B[8*half .. 8*half+7][col]        (8 bf16, one column)
//   D (32 x 32): lane l holds D[8*g + 4*half + r][col], g, r in 0..3, at index 4*g + r
// Every contraction below is over an index whose order is free, so operands are loaded in
// whatever k-order keeps the loads contiguous, as long as A and B agree on it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spa {

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
// Native vectors for raw 16- and 8-byte moves (copies of HIP's uint4 struct lower to memcpy,
// which keeps arrays of them out of registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x8 as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ uint4 as_uint4(bf16x8 v) { return __builtin_bit_cast(uint4, v); }

__device__ __forceinline__ uint4 load16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// Two floats rounded to nearest-even bf16, packed low/high into one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Two floats rounded to nearest-even fp16, packed low/high into one dword.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a packed bf16 pair, in fp32 (one v_dot2 against (1, 1)).
__device__ __forceinline__ float add_bf16x2(uint32_t packed, float acc) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), ones, acc, false);
}

__device__ __forceinline__ f32x16 f32x16_fill(float x) {
    f32x16 v;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = x;
    return v;
}

// max / sum of x over lanes l and l xor 32, in every lane (one v_permlane32_swap: the two
// results hold the low and the high half-wave's values side by side).
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace spa
