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

// GELU, tanh form, in fp32: y/2 * (1 + tanh(sqrt(2/pi) * (y + 0.044715 y^3))).
__device__ __forceinline__ float gelu_tanh_f32(float y) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  const float k1 = 0.044715f;
  float u = k0 * (y + k1 * y * y * y);
  return 0.5f * y * (1.0f + tanhf(u));
}

}  // namespace svdq
