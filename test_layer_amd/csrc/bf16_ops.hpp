// bf16 tile helpers for the MFMA kernels: LDS/global vector access, operand
// packing and the gfx950 LDS transpose read.
#pragma once

#include "common.hpp"

namespace vggt3 {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(void* p, const u32x2& v) { *reinterpret_cast<u32x2*>(p) = v; }

// 8 consecutive bf16 of one LDS row as an MFMA operand (one ds_read_b128).
__device__ __forceinline__ bf16x8 ld_op(const uint16_t* p) { return as_bf16x8(ld16(p)); }

// LDS transpose read (ds_read_b64_tr_b16). Within each group of 16 lanes, lane
// s = 4j + q supplies the address of 4 consecutive bf16 (columns c0+4q..c0+4q+3
// of some row R_j); lane i of the group receives, as element j = 0..3, the
// value at (row R_j, column c0 + i). I.e. the group reads a 4 x 16 block
// row-wise and every lane gets one column of it.
__device__ __forceinline__ u32x2 lds_tr16(const uint16_t* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uint16_t*)p);
  return __builtin_bit_cast(u32x2, v);
}

// MFMA operand from two transpose reads (k-slots 0..3 from p0, 4..7 from p1).
__device__ __forceinline__ bf16x8 tr_op(const uint16_t* p0, const uint16_t* p1) {
  const u32x2 a = lds_tr16(p0), b = lds_tr16(p1);
  return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
}

// MFMA operand from two 4-element LDS runs (ds_read_b64 x 2).
__device__ __forceinline__ bf16x8 pair_op(const uint16_t* p0, const uint16_t* p1) {
  const u32x2 a = ld8(p0), b = ld8(p1);
  return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
}

__device__ __forceinline__ bf16x8 pack8(const float* v) {
  u32x4 q;
  q[0] = pack_bf16x2(v[0], v[1]);
  q[1] = pack_bf16x2(v[2], v[3]);
  q[2] = pack_bf16x2(v[4], v[5]);
  q[3] = pack_bf16x2(v[6], v[7]);
  return as_bf16x8(q);
}

__device__ __forceinline__ u32x4 as_u32x4(const bf16x8& v) { return __builtin_bit_cast(u32x4, v); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace vggt3
