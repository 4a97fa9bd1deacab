// The fused MLP chain's epilogue on a staged tile: the up-projection's 16-bit
// output U (GELU applied, rounded to the compute dtype exactly as the unfused
// GEMM stores it) sits in LDS, and the down-projection's activation quantizer
// runs on it there (the pages' GELU / MLP fused kernels of the full engine:
// dothoosh.com "How Nunchaku Lite halves diffusion-model VRAM", generic-path
// paragraph). Two parts, each run by all 256 threads of the workgroup:
//
//  - chain_quantize_tile: smoothing x_hat = fl32(U * smooth_inv2), then INT4
//    group-64 codes and fp16 scales of every (row, group) of the tile, stored
//    straight to the down-projection's act_codes / act_scales. The rule is the
//    activation quantizer's, so the codes equal what svdq_quantize_act gives on
//    the stored U, bit for bit.
//  - chain_lowrank_partial: the tile's share of U lora_down2^T (fp32), one
//    slice per tile of columns, summed in a fixed order by the chain's reduce
//    kernel.
//
// Used by the 4-bit float kernels, whose accumulators do not map onto INT4
// groups lane by lane; the INT4 kernel quantizes from its registers instead.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace svdq {

// INT4 codes of 8 values against scale sf (nonzero), rs = rcp(sf); raises
// tmax to the largest |v * rs - q|. The product v * rs is rounded to an integer
// (ties to even) inside fma(v, rs, 1.5 * 2^23) and clamped to +-7 by a med3 in
// that domain; it is within 2^-19 |y| of fl32(v / sf) (rcp is within an ulp),
// so the two round to the same integer unless y lies within 2^-16 of a
// half-integer, which fma(v, rs, -q) shows (one rounding): a group with
// tmax > 0.5 - 2^-16 is recomputed with the IEEE division by the caller.
// Nibbles: even k low.
__device__ __forceinline__ uint32_t chain_int4_codes8(const float* v, float rs, float& tmax) {
  constexpr float kM = 12582912.0f;   // 1.5 * 2^23
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float y = __builtin_amdgcn_fmed3f(fmaf(v[i], rs, kM), kM - 7.0f, kM + 7.0f);
    tmax = __builtin_fmaxf(tmax, fabsf(fmaf(v[i], rs, -(y - kM))));
    w |= (__float_as_uint(y) & 0xFu) << (4 * i);
  }
  return w;
}

__device__ __forceinline__ uint32_t chain_int4_codes8_exact(const float* v, float sf) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q = fminf(fmaxf(rintf(v[i] / sf), -7.0f), 7.0f);   // IEEE division, ties to even
    w |= ((uint32_t)(int)q & 0xFu) << (4 * i);
  }
  return w;
}

// tile: U [BM][TP] in LDS (h16 bits), columns n0 .. n0 + BN of the up-projection's
// output; si: smooth_inv2[n0 .. n0 + BN) in LDS. Thread t of the NT takes the
// (row, group) items t, t + NT, ...; the four (or two) threads of one row write
// its BN / 2 code bytes as consecutive 32-byte pieces.
template <int IO, int BM, int BN, int TP, int NT = 256>
__device__ __forceinline__ void chain_quantize_tile(const uint16_t* tile, const float* si, int m0, int n0, int M,
                                                    int N, const ChainEpilogue& ce, int tid) {
#pragma clang fp contract(off)
  constexpr int G = BN / 64;
  for (int it = tid; it < BM * G; it += NT) {
    const int row = it / G, g = it - row * G;
    if (m0 + row >= M) break;   // items run row by row, so every later one is past M too
    const uint16_t* src = tile + row * TP + g * 64;
    float x[64];
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint4 h = *reinterpret_cast<const uint4*>(src + 8 * c);
      const float4 s0 = *reinterpret_cast<const float4*>(si + g * 64 + 8 * c);
      const float4 s1 = *reinterpret_cast<const float4*>(si + g * 64 + 8 * c + 4);
      const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
      const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint16_t b = (uint16_t)(hw[i >> 1] >> (16 * (i & 1)));
        // x_hat = fl32(u * smooth_inv): one multiply, the -0 addend keeps the sign of zero
        x[8 * c + i] = fmaf(Io<IO>::to_f(b), sv[i], -0.0f);
        amax = fmaxf(amax, fabsf(x[8 * c + i]));
      }
    }
    const __half s16 = __float2half_rn(fminf(div7_rn(amax), 65504.0f));   // fl32(amax / 7), as IEEE division
    const float sf = __half2float(s16);
    uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (sf != 0.0f) {
      const float rs = __builtin_amdgcn_rcpf(sf);
      float tmax = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) w[c] = chain_int4_codes8(x + 8 * c, rs, tmax);
      if (tmax > 0.4999847412109375f) {   // 0.5 - 2^-16
#pragma unroll
        for (int c = 0; c < 8; ++c) w[c] = chain_int4_codes8_exact(x + 8 * c, sf);
      }
    }
    uint8_t* dst = ce.codes + (size_t)(m0 + row) * (N >> 1) + ((n0 + g * 64) >> 1);
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
    reinterpret_cast<__half*>(ce.scales)[(size_t)(m0 + row) * (N >> 6) + (n0 >> 6) + g] = s16;
  }
}

// P[m][j] = sum_n U[m][n] lora_down2[j][n0 + n] over the tile's BN columns, on
// v_mfma_f32_16x16x16 (lane l: row or rank l % 16, k 4 (l / 16) .. +4; result:
// rank l % 16, rows 4 (l / 16) + i). Wave w of the NT / 64 takes rows w WR .. +WR
// (WR = BM / (NT / 64)); the slice `part` ([M][r2] fp32, this tile's) is
// written in full for rows < M.
template <int IO, int BM, int BN, int TP, int NT = 256>
__device__ __forceinline__ void chain_lowrank_partial(const uint16_t* tile, int m0, int n0, int M, int N,
                                                      const ChainEpilogue& ce, float* part, int wave,
                                                      int lane) {
  constexpr int WR = BM / (NT / 64), HB = WR / 16;   // rows per wave, 16-row blocks per wave
  static_assert(WR % 16 == 0, "whole 16-row blocks per wave");
  const int l16 = lane & 15, lq = lane >> 4;
  const uint16_t* ldn = reinterpret_cast<const uint16_t*>(ce.lora_down);
  for (int jb = 0; jb < ce.r; jb += 16) {
    uint2 bw[BN / 16];
#pragma unroll
    for (int k = 0; k < BN / 16; ++k)
      bw[k] = *reinterpret_cast<const uint2*>(ldn + (size_t)(jb + l16) * N + n0 + 16 * k + lq * 4);
    v4f pacc[HB];
#pragma unroll
    for (int h = 0; h < HB; ++h) pacc[h] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < BN / 16; ++k)
#pragma unroll
      for (int h = 0; h < HB; ++h) {
        const uint2 aw =
            *reinterpret_cast<const uint2*>(tile + (wave * WR + h * 16 + l16) * TP + 16 * k + lq * 4);
        pacc[h] = Io<IO>::mma16x16x16(aw, bw[k], pacc[h]);
      }
#pragma unroll
    for (int h = 0; h < HB; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wave * WR + h * 16 + lq * 4 + i;
        if (m < M) part[(size_t)m * ce.r + jb + l16] = pacc[h][i];
      }
  }
}

}  // namespace svdq
