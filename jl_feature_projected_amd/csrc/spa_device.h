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

// The same fp16 MFMA with its result and accumulator in VGPRs. In a kernel that may use
// more than 256 registers the compiler gives every MFMA the AGPR form, and a VALU use of the
// result then needs one v_accvgpr_read per element; this form avoids that for results the
// VALU consumes. The compiler inserts no wait states around inline assembly, so each
// statement carries those it inserts around its own 8-pass MFMAs: two between a VALU write of
// a source and the MFMA (s_nop 1 in front) and, where the accumulator input is a register of
// its own, eight between the issue and a later write of that input (s_nop 7 behind). Next to
// another MFMA these nops overlap the matrix pipe's issue wait. The caller keeps at least three
// MFMAs between this and the first VALU read of the result; a chain on one accumulator needs
// no wait (exact overlap of result and srcC).
__device__ __forceinline__ f32x16 mfma32x32x16_v(f16x8 a, f16x8 b, f32x16 c) {
    f32x16 d;
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %3\n\ts_nop 7" : "=&v"(d) : "v"(a), "v"(b), "v"(c));
#else
    d = c;
#endif
    return d;
}
__device__ __forceinline__ void mfma32x32x16_v_acc(f16x8 a, f16x8 b, f32x16& c) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
#endif
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

// Buffer descriptor over [base, base + bytes): loads past the end return zero. Raw buffer
// (stride 0), 32-bit data format. The fields go through readfirstlane so they are SGPRs
// (the asm operand needs them there) even where the compiler cannot prove them uniform.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    u32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
    r.z = __builtin_amdgcn_readfirstlane(bytes);
    r.w = 0x00020000u;
    return r;
}

// 16 bytes per lane from buffer offset voff straight into LDS at byte address m0 + 16 * lane
// (m0 wave-uniform; readfirstlane keeps it in an SGPR where the compiler cannot prove that).
// Issued as inline assembly so the compiler does not track it: it cannot tell that the LDS
// it writes (another buffer) is disjoint from the LDS the tile loop reads, and would
// otherwise wait for the copy before the first read. The copy's completion is awaited
// explicitly (vmcnt) before the barrier that hands the buffer over. Device pass only: the
// host pass does not parse AMDGPU assembly constraints.
// The copies set M0 themselves and list it as clobbered, which is what tells the compiler
// not to keep a value there across them; clang notes that M0 is a reserved register.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(u32x4 rsrc, uint32_t m0, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(rsrc)
                 : "m0");
#endif
}

// 16-byte chunk swizzles: LDS slot = global chunk ^ swizzle(row), a GF(2)-linear function of
// the row's low bits, chosen so that every operand read touches each LDS bank once per
// service cycle, whether the LDS serves 128 bytes per cycle over 32 banks or 256 bytes over
// 64 (the K-tile tables were found by exhaustive search over such functions):
//   K tile (rows of MP*2 bytes), score operand: 8 or 16 consecutive rows, one chunk each
//   (the backward's tiles of rows of R*2 bytes, R in {16, 32, 64, 128}, are read the same
//   way and use kswz<R>);
//   V^T tile (rows of 128 bytes = 64 keys), PV operand: 8 or 16 consecutive rows, one chunk
//   each. Rows r and r+8 share their position in a 256-byte bank row pair only if they differ
//   in bit 0 after the swizzle, hence the extra bit-3 term.
template <int MP>
__device__ __forceinline__ int kswz(int row) {
    constexpr int b0 = MP == 16 ? 0 : MP == 32 ? 0 : 1;
    constexpr int b1 = MP == 16 ? 0 : MP == 32 ? 1 : 2;
    constexpr int b2 = MP == 16 ? 1 : MP == 32 ? 2 : 4;
    constexpr int b3 = MP == 16 ? 1 : MP == 32 ? 1 : MP == 64 ? 1 : 8;
    return (row & 1 ? b0 : 0) ^ (row & 2 ? b1 : 0) ^ (row & 4 ? b2 : 0) ^ (row & 8 ? b3 : 0);
}
__device__ __forceinline__ int vtswz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
// Row-major V tile (rows of 256 bytes), transposing PV operand read: a 16-lane group takes 32
// bytes of each of 4 consecutive rows, two groups 64 bytes of the same rows. Byte offsets in
// row r are XORed with vxswz(r % 4) (it moves whole 32-byte blocks), which sends the 4 rows to
// 4 distinct quarters of 128 bytes and of 256 bytes alike.
__device__ __forceinline__ int vxswz(int r3) { return 64 * r3 + 32 * (r3 >> 1); }

// As copy16_to_lds, 4 bytes per lane, to m0 + 4 * lane.
__device__ __forceinline__ void copy4_to_lds(u32x4 rsrc, uint32_t m0, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(rsrc)
                 : "m0");
#endif
}
#pragma clang diagnostic pop

// s_waitcnt immediate that waits until at most n vector-memory operations are outstanding
// (expcnt and lgkmcnt left at their maxima, i.e. not waited on).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// LDS byte address of a __shared__ array's first byte (wave-uniform).
__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p);
}

}  // namespace spa
