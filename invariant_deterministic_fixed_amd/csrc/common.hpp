// common.hpp -- small device helpers shared by the libbinv kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace binv {

typedef uint16_t bf16_t;                                          // raw bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));        // MFMA operand
typedef float f32x4 __attribute__((ext_vector_type(4)));          // 16x16 MFMA accumulator
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));       // 16-byte load / store
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));       // 8-byte load / store

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN
// (bits 31..16 with the quiet bit set).  gfx950 converts in one instruction
// (v_cvt_pk_bf16_f32, two values at a time), which gives exactly those bits for
// all 2^32 inputs (a GPU test checks it exhaustively against the integer rule
// u + 0x7fff + ((u >> 16) & 1), NaNs included).  The integer form
// cost up to seven vector instructions per value and, written with an early
// return for NaN, a branch with exec-mask save / restore around each one.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// two fp32 -> packed pair of bf16 (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D = A(16x32) * B(32x16) + C on the bf16 matrix cores, fp32 accumulate.
// Lane l supplies A row (l % 16) and B column (l % 16), each with the 8 k
// values of group l / 16; the result element (row 4*(l/16)+i, column l%16)
// is returned in component i.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

}  // namespace binv
