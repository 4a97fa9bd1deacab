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
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// The 16-bit type of activations, the low-rank branch, biases, norm weights and
// outputs (the layer's compute dtype): IO 0 = fp16, IO 1 = bf16. Conversions to
// 16 bits round to nearest, ties to even; the low-rank products run on the
// matching MFMA with fp32 accumulation. Operands are passed as raw bits.
template <int IO> struct Io;
template <> struct Io<0> {
  static __device__ __forceinline__ float to_f(uint16_t b) { return __half2float(__ushort_as_half(b)); }
  static __device__ __forceinline__ uint16_t from_f(float v) { return __half_as_ushort(__float2half_rn(v)); }
  static __device__ __forceinline__ v4f mma16x16x16(uint2 a, uint2 b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v4h, a), __builtin_bit_cast(v4h, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ v4f mma16x16x32(uint4 a, uint4 b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ v16f mma32x32x16(uint4 a, uint4 b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  }
};
template <> struct Io<1> {
  static __device__ __forceinline__ float to_f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
  // gfx950's v_cvt_pk_bf16_f32: round to nearest even, NaN -> quiet NaN with
  // the upper payload bits kept, denormals kept; equal bit for bit, over all
  // 2^32 inputs, to (u + 0x7FFF + lsb) >> 16 with NaN -> (u >> 16) | 0x40.
  // One instruction and no branch.
  static __device__ __forceinline__ uint16_t from_f(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
  }
  static __device__ __forceinline__ v4f mma16x16x16(uint2 a, uint2 b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4s, a), __builtin_bit_cast(v4s, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ v4f mma16x16x32(uint4 a, uint4 b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ v16f mma32x32x16(uint4 a, uint4 b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  }
};

// lora_act is fp32; the low-rank up-projection runs on the 16-bit matrix
// instructions, so each value v enters as a pair of 16-bit operands hi =
// h16(v), lo = h16(v - hi) (v - hi is exact in fp32) and the pair goes through
// two MFMAs against the same lora_up operand. hi + lo equals v within
// 2^-22 |v| for fp16 (plus 2^-25 absolute where lo is subnormal) and 2^-18 |v|
// for bf16, where one 16-bit value alone would be off by up to 2^-11 |v| or
// 2^-8 |v|.
template <int IO>
__device__ __forceinline__ void split_h16(float v, uint32_t& hi, uint32_t& lo) {
  const uint16_t h = Io<IO>::from_f(v);
  hi = h;
  lo = Io<IO>::from_f(v - Io<IO>::to_f(h));
}
// four consecutive values -> (hi, lo) as two packed 4 x h16 operands
template <int IO>
__device__ __forceinline__ void split4_h16(float4 v, uint2& hi, uint2& lo) {
  uint32_t h[4], l[4];
  split_h16<IO>(v.x, h[0], l[0]);
  split_h16<IO>(v.y, h[1], l[1]);
  split_h16<IO>(v.z, h[2], l[2]);
  split_h16<IO>(v.w, h[3], l[3]);
  hi = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  lo = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
}
// eight consecutive values -> (hi, lo) as two packed 8 x h16 operands
template <int IO>
__device__ __forceinline__ void split8_h16(float4 a, float4 b, uint4& hi, uint4& lo) {
  uint2 h0, l0, h1, l1;
  split4_h16<IO>(a, h0, l0);
  split4_h16<IO>(b, h1, l1);
  hi = make_uint4(h0.x, h0.y, h1.x, h1.y);
  lo = make_uint4(l0.x, l0.y, l1.x, l1.y);
}

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
// For NON-NEGATIVE values only (the group maxima of |x|): their bit patterns
// order as unsigned integers the way the values do, so an integer max takes
// the place of a float max (which would canonicalize both swapped operands).
__device__ __forceinline__ float lane_max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(max((uint32_t)r[0], (uint32_t)r[1]));
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

// max over the 16 lanes of a DPP row (same exchange pattern as row16_sum), for
// NON-NEGATIVE values (compared as unsigned bit patterns, as in lane_max_xor32)
__device__ __forceinline__ float row16_max(float v) {
  uint32_t u = __float_as_uint(v);
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x140, 0xF, 0xF, false));   // row_mirror
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x141, 0xF, 0xF, false));   // row_half_mirror
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
  u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
  return __uint_as_float(u);
}

__device__ __forceinline__ float lane_max_xor16(float v) {   // non-negative values, as above
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(max((uint32_t)r[0], (uint32_t)r[1]));
}

// fl32(a / 7), correctly rounded, in three instructions: q = RN(a z) with
// z = RN(1/7), the residual r = a - 7 q (exact in one fma), then RN(q + r z).
// Equal to the IEEE quotient for every fp32 a: checked exhaustively over the
// significands of the subnormals and of the lowest 40 and highest 55 binades
// (the sequence scales exactly by powers of two in between).
__device__ __forceinline__ float div7_rn(float a) {
#pragma clang fp contract(off)
  const float z = 0.142857149243354797363281250f;   // RN(1/7) = 0x3E124925
  const float q = a * z;
  return fmaf(fmaf(-7.0f, q, a), z, q);
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
