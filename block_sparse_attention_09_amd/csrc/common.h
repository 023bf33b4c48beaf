// Internal helpers shared by the gfx950 kernels of libabatt.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace abatt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  return (u & 0x7fffffffu) > 0x7f800000u ? ((u >> 16) | 0x40u) : rne;
}

// Two floats -> packed fp16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16_rne(float lo, float hi) {
  f16x2 v;
  v[0] = (_Float16)lo;
  v[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Two floats -> packed fp16 pair, round toward zero.  Exact for values that
// came from bfloat16 and lie in fp16's normal range (8 <= 11 mantissa bits).
__device__ __forceinline__ uint32_t pack_f16_rtz(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f16_32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Work-group id -> work item so that consecutive items land on one XCD.
// The dispatcher hands work-group i to XCD i % 8; this mapping gives XCD x a
// contiguous range of items (a bijection on [0, n)).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, rem = n & 7;
  const int x = bid & 7, k = bid >> 3;
  return x * q + (x < rem ? x : rem) + k;
}

// Exchanges between lane groups through the register file (gfx950
// v_permlane32_swap / v_permlane16_swap) in place of LDS-routed shuffles.
// permlane32_swap(a, b) returns {a of lanes 0-31 | b of lanes 0-31} and
// {a of lanes 32-63 | b of lanes 32-63} (in the lower | upper half), so with
// a = b = v every lane receives v of lanes l & ~32 and l | 32, in that order;
// permlane16_swap does the same for the 16-lane rows 0,1 and 2,3.  Results
// are identical in both lanes of a pair, which keeps pairwise sums in the same
// order everywhere.
__device__ __forceinline__ f32x2 pair_x32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ f32x2 pair_x16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ int sum_x32(int v) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
  return (int)(r[0] + r[1]);
}
__device__ __forceinline__ int sum_x16(int v) {
  const auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
  return (int)(r[0] + r[1]);
}
// {a, b} -> lower half gets a of both halves, upper half gets b of both halves
__device__ __forceinline__ f32x2 cross_x32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace abatt
