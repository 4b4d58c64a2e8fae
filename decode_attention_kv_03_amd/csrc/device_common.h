// Device-side helpers shared by the decode-attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvattn {

// Register types of the gfx950 bf16 matrix-core builtins.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x on the hardware exp unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max over lanes {l, l^16, l^32, l^48}: the gfx950 row swaps exchange
// 16-lane rows (odd <-> even) and 32-lane halves on the VALU, so each pair
// of results holds a lane's own value and its partner's.
__device__ __forceinline__ float max_over_row_groups(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(v);
  const auto c = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

__device__ __forceinline__ float sum_over_row_groups(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t w = __float_as_uint(v);
  const auto c = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Max and sum over lanes {l, l^32}: the two lane halves that hold the two
// row groups of a 32x32 matrix-core result.
__device__ __forceinline__ float max_over_halves(float v) {
  const uint32_t w = __float_as_uint(v);
  const auto c = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

__device__ __forceinline__ float sum_over_halves(float v) {
  const uint32_t w = __float_as_uint(v);
  const auto c = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Two floats -> packed bfloat16 pair (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// Sum of the two bfloat16 values of a packed pair, added to acc in fp32.
__device__ __forceinline__ float add_bf16x2(uint32_t packed, float acc) {
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), ones, acc, false);
}

// Full 64-lane reductions.
__device__ __forceinline__ float wave_reduce_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ __forceinline__ float wave_reduce_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Sliding window ("One dial, four settings", the full ladder's SWA row and
// the sliding-window question): a sequence of `len` tokens attends to its
// last `window` tokens (window 0: all of them).  First attended token, and
// the 64-aligned token the splits start from (tiles keep their alignment;
// tokens below the first attended one are masked).
__device__ __forceinline__ int window_first(int len, int window) { return window > 0 && len > window ? len - window : 0; }
__device__ __forceinline__ int window_base(int len, int window) { return window_first(len, window) & ~63; }

// Clamp a device-side sequence length into [0, cap].
__device__ __forceinline__ int clamp_len(int len, int cap) { return len < 0 ? 0 : (len > cap ? cap : len); }

}  // namespace kvattn
