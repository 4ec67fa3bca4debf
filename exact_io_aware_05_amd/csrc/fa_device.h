// Device-side building blocks shared by the attention kernels (gfx950).
//
// Matrix-core operand layouts used throughout (v_mfma_f32_32x32x16_bf16, one
// wave of 64 lanes, h = lane / 32, col = lane % 32):
//   A (32 x 16):  lane holds A[row = col][k = 8h .. 8h+7]      (8 bf16)
//   B (16 x 32):  lane holds B[k = 8h .. 8h+7][col]            (8 bf16)
//   C (32 x 32):  lane holds C[row = 8(r/4) + 4h + r%4][col], r = 0..15
// Scores are computed transposed, S^T = K Q^T, so that one lane owns one
// query (column) and 16 of its 32 keys; the other 16 sit in lane col + 32.
// Row reductions are then 16 in-lane steps plus one exchange between the
// two wave halves (v_permlane32_swap).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max / sum of x over lanes (l, l ^ 32).  Both lanes of a pair get the same
// value, computed in the same order (low-half operand first).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// two fp32 -> packed bf16x2, round to nearest even
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a packed bf16 pair, accumulated in fp32
// (v_dot2c_f32_bf16 against (1, 1)).
__device__ __forceinline__ float add_bf16x2(uint32_t pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                         __builtin_bit_cast(bf16x2, 0x3F803F80u),
                                         acc, false);
}

// Eight fp32 (elements [base, base + 8) of a C fragment) -> a bf16x8
// operand.
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& c, int base) {
  u32x4 u;
  u[0] = pack_bf16x2(c[base + 0], c[base + 1]);
  u[1] = pack_bf16x2(c[base + 2], c[base + 3]);
  u[2] = pack_bf16x2(c[base + 4], c[base + 5]);
  u[3] = pack_bf16x2(c[base + 6], c[base + 7]);
  return __builtin_bit_cast(bf16x8, u);
}

// Maps the launch index of a workgroup to a logical work item so that each
// of the 8 XCDs (which receive workgroups round-robin) gets one contiguous
// range of logical items, in logical order.  Bijective on [0, n).
__device__ __forceinline__ int xcd_contiguous(int w, int n) {
  const int x = w & 7, s = w >> 3;
  const int base = n >> 3, rem = n & 7;
  return x * base + (x < rem ? x : rem) + s;
}

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Buffer resource over [base, base + bytes): loads at byte offsets >= bytes
// return zeros (the hardware range check), which is how the kernels read
// past the end of a sequence without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base,
                                                              uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)bytes, 0x00020000);
}

}  // namespace fa
