// Shared device helpers for the gfx950 kernels of the TTT layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vggt3 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// bf16 bit patterns are handled as uint16_t in memory.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// Low / high bf16 of a packed pair -> fp32 (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
// Two fp32 -> packed bf16 pair (lo = a, hi = b), round to nearest even, as one
// v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 32x32x16 bf16 MFMA, fp32 accumulate.
//   A operand: lane l holds A[row = l%32][k = 8*(l/32) + j], j = 0..7
//   B operand: lane l holds B[k = 8*(l/32) + j][col = l%32]
//   C/D:       lane l, register r holds C[row = 8*(r/4) + 4*(l/32) + r%4][col = l%32]
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Logistic sigmoid via the hardware exp2 and reciprocal: 1 / (1 + 2^(-x log2 e)).
__device__ __forceinline__ float sigmoid_fast(float x) {
  const float e = __builtin_amdgcn_exp2f(x * -1.4426950408889634f);
  return __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace vggt3
