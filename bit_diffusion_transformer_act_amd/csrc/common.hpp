// Shared device-side types and helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace svdq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float lane_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, kWave));
}

__device__ __forceinline__ float lane_sum_xor(float v, int mask) {
  return v + __shfl_xor(v, mask, kWave);
}

// max over lanes l and l ^ 32, and over lanes l and l ^ 16, with gfx950's lane
// swaps: v_permlane32_swap exchanges the upper 32 lanes of its first operand
// with the lower 32 of its second (so with two copies of v each lane ends up
// holding v[l] and v[l ^ 32]); v_permlane16_swap does the same between the odd
// and even 16-lane rows (v[l] and v[l ^ 16]). All 64 lanes must be active.
__device__ __forceinline__ float lane_max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Sum over each 16-lane row with DPP (mirror, half-mirror, then the two quad
// exchanges); every lane of the row gets the same total.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  return v;
}

__device__ __forceinline__ float lane_max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// GELU, tanh form, in fp32: y/2 * (1 + tanh(u)), u = sqrt(2/pi) (y + 0.044715 y^3).
// Uses 1 + tanh(u) = 2 / (1 + exp(-2u)), so the value is y / (1 + 2^(-2u log2 e))
// with the hardware exp2 and reciprocal (about 1 ulp each): far below the fp16
// rounding of the result. The exponent -2u log2 e is formed as y (c0 + c1 y^2).
// Large |y| saturates to y or -0 exactly.
__device__ __forceinline__ float gelu_tanh_f32(float y) {
  const float c0 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float c1 = c0 * 0.044715f;
  const float e = __builtin_amdgcn_exp2f(y * fmaf(c1, y * y, c0));
  return y * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace svdq
