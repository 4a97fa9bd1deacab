// awq_gemv_w4a16: 4-bit weights, 16-bit activations, for the memory-bound
// modulation / adaptive-norm projections (dothoosh.com "How Nunchaku Lite
// halves diffusion-model VRAM", kernel-family list, the awq_w4a16 entry;
// int4 with group size 64 in the quantization_config block).
//
//   y[m,n] = sum_k x[m,k] (q[n,k] - z[n,g]) s[n,g],  g = k / 64
//
// HBM-bound: every weight byte is read once. Dequantization uses the fp16
// bit trick: (word >> 4j) & 0x000F000F | 0x64006400 is the packed fp16 pair
// (1024 + q_j, 1024 + q_{j+4}), exact, and v_dot2_f32_f16 accumulates
// x (1024 + q) in fp32 against x stored as pairs (x_j, x_{j+4}). Per group,
//   sum x (q - z) = sum x (1024 + q) - (1024 + z) sum x,
// with the second term one fma from the precomputed sum of x, so any fp16
// zero point works.
//
// Main kernel (M * ceil(K / 4096) <= 4): one lane owns one 64-wide group of
// every row it visits (two 16-byte code loads, one scale, one zero); its
// x values stay in registers for the whole kernel; a wave handles 8 rows and
// issues all their loads before any arithmetic. Fallback kernel for larger
// M * K: x staged in LDS, a lane owns 16-code chunks.
#include "common.hpp"

namespace svdq {

constexpr int kGemvWaves = 4;

// ----------------------------------------------------------------- main --
template <int MR, int GPL, int RPW>
__global__ __launch_bounds__(256)
void awq_gemv_reg_kernel(const __half* __restrict__ x, const uint8_t* __restrict__ codes,
                         const __half* __restrict__ scales, const __half* __restrict__ zeros,
                         __half* __restrict__ y, int N, int K) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = K >> 6;
  const int nbase = (blockIdx.x * kGemvWaves + wave) * RPW;

  // issue every weight load of the wave's rows first
  uint4 cw[RPW][GPL][2];
  float sv[RPW][GPL], zv[RPW][GPL];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const int n = nbase + rr, g = lane + 64 * j;
      if (n < N && g < G) {
        const uint4* pc = reinterpret_cast<const uint4*>(codes + (size_t)n * (K >> 1) + g * 32);
        cw[rr][j][0] = pc[0];
        cw[rr][j][1] = pc[1];
        sv[rr][j] = __half2float(scales[(size_t)n * G + g]);
        zv[rr][j] = __half2float(zeros[(size_t)n * G + g]);
      } else {
        cw[rr][j][0] = make_uint4(0, 0, 0, 0);
        cw[rr][j][1] = make_uint4(0, 0, 0, 0);
        sv[rr][j] = 0.f;
        zv[rr][j] = 0.f;
      }
    }

  // x of this lane's groups as (x_j, x_{j+4}) pairs, and their sums
  uint32_t xp[MR][GPL][32];
  float xsum[MR][GPL];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const int g = lane + 64 * j;
      float sum = 0.f;
#pragma unroll
      for (int seg = 0; seg < 8; ++seg) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (g < G) v = reinterpret_cast<const uint4*>(x + (size_t)m * K + g * 64)[seg];
        xp[m][j][seg * 4 + 0] = (v.x & 0xFFFFu) | (v.z << 16);
        xp[m][j][seg * 4 + 1] = (v.x >> 16) | (v.z & 0xFFFF0000u);
        xp[m][j][seg * 4 + 2] = (v.y & 0xFFFFu) | (v.w << 16);
        xp[m][j][seg * 4 + 3] = (v.y >> 16) | (v.w & 0xFFFF0000u);
        const v2h one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sum = __builtin_amdgcn_fdot2(__builtin_bit_cast(v2h, xp[m][j][seg * 4 + e]), one, sum, false);
      }
      xsum[m][j] = sum;
    }

#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = 0.f;
#pragma unroll
    for (int j = 0; j < GPL; ++j) {
      const uint32_t w[8] = {cw[rr][j][0].x, cw[rr][j][0].y, cw[rr][j][0].z, cw[rr][j][0].w,
                             cw[rr][j][1].x, cw[rr][j][1].y, cw[rr][j][1].z, cw[rr][j][1].w};
      float part[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) part[m] = 0.f;
#pragma unroll
      for (int wi = 0; wi < 8; ++wi)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const uint32_t hb = ((w[wi] >> (4 * jj)) & 0x000F000Fu) | 0x64006400u;
#pragma unroll
          for (int m = 0; m < MR; ++m)
            part[m] = __builtin_amdgcn_fdot2(__builtin_bit_cast(v2h, hb),
                                             __builtin_bit_cast(v2h, xp[m][j][wi * 4 + jj]), part[m], false);
        }
#pragma unroll
      for (int m = 0; m < MR; ++m)
        acc[m] = fmaf(sv[rr][j], fmaf(-(1024.0f + zv[rr][j]), xsum[m][j], part[m]), acc[m]);
    }
    const int n = nbase + rr;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float v = acc[m];
      v = lane_sum_xor(v, 32);
      v = lane_sum_xor(v, 16);
      v = lane_sum_xor(v, 8);
      v = lane_sum_xor(v, 4);
      v = lane_sum_xor(v, 2);
      v = lane_sum_xor(v, 1);
      if (lane == 0 && n < N) y[(size_t)m * N + n] = __float2half_rn(v);
    }
  }
}

// ------------------------------------------------------------- fallback --
constexpr int kRowsPerWave = 4;

template <int MR>
__global__ __launch_bounds__(256)
void awq_gemv_kernel(const __half* __restrict__ x, const uint8_t* __restrict__ codes,
                     const __half* __restrict__ scales, const __half* __restrict__ zeros,
                     __half* __restrict__ y, int N, int K) {
  extern __shared__ uint32_t xs[];  // [MR][K/8 segments][4 pairs]
  const int segs = K >> 3;
  for (int idx = threadIdx.x; idx < MR * segs; idx += blockDim.x) {
    const int m = idx / segs, sg = idx - m * segs;
    const uint4 v = *reinterpret_cast<const uint4*>(x + (size_t)m * K + sg * 8);
    uint32_t* o = xs + (size_t)idx * 4;
    o[0] = (v.x & 0xFFFFu) | (v.z << 16);
    o[1] = (v.x >> 16) | (v.z & 0xFFFF0000u);
    o[2] = (v.y & 0xFFFFu) | (v.w << 16);
    o[3] = (v.y >> 16) | (v.w & 0xFFFF0000u);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nbase = (blockIdx.x * kGemvWaves + wave) * kRowsPerWave;
  const int chunks = K >> 4;        // 16 codes (8 bytes) per chunk
  const int gstride = K >> 6;
  const v2h one = {(_Float16)1.0f, (_Float16)1.0f};

  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int n = nbase + rr;
    if (n >= N) break;
    const uint8_t* crow = codes + (size_t)n * (K >> 1);
    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = 0.f;
    for (int c = lane; c < chunks; c += 64) {
      const uint2 w = *reinterpret_cast<const uint2*>(crow + (size_t)c * 8);
      const int g = c >> 2;
      const float s = __half2float(scales[(size_t)n * gstride + g]);
      const float zb = 1024.0f + __half2float(zeros[(size_t)n * gstride + g]);
      float part[MR], sum[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) part[m] = sum[m] = 0.f;
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const uint32_t word = d ? w.y : w.x;
        const int sg = 2 * c + d;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t hb = ((word >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            const v2h xp = __builtin_bit_cast(v2h, xs[((size_t)m * segs + sg) * 4 + j]);
            part[m] = __builtin_amdgcn_fdot2(__builtin_bit_cast(v2h, hb), xp, part[m], false);
            sum[m] = __builtin_amdgcn_fdot2(one, xp, sum[m], false);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MR; ++m) acc[m] = fmaf(s, fmaf(-zb, sum[m], part[m]), acc[m]);
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      float v = acc[m];
      v = lane_sum_xor(v, 32);
      v = lane_sum_xor(v, 16);
      v = lane_sum_xor(v, 8);
      v = lane_sum_xor(v, 4);
      v = lane_sum_xor(v, 2);
      v = lane_sum_xor(v, 1);
      if (lane == 0) y[(size_t)m * N + n] = __float2half_rn(v);
    }
  }
}

template <int MR, int GPL>
static hipError_t launch_reg(int N, int K, const void* x, const uint8_t* q, const void* s,
                             const void* z, void* y, hipStream_t st) {
  constexpr int RPW = 8;
  const int rows_per_block = kGemvWaves * RPW;
  const dim3 grid((N + rows_per_block - 1) / rows_per_block), block(64 * kGemvWaves);
  hipLaunchKernelGGL((awq_gemv_reg_kernel<MR, GPL, RPW>), grid, block, 0, st, (const __half*)x, q,
                     (const __half*)s, (const __half*)z, (__half*)y, N, K);
  return hipGetLastError();
}

template <int MR>
static hipError_t launch_lds(int N, int K, const void* x, const uint8_t* q, const void* s,
                             const void* z, void* y, hipStream_t st) {
  const int rows_per_block = kGemvWaves * kRowsPerWave;
  const dim3 grid((N + rows_per_block - 1) / rows_per_block), block(64 * kGemvWaves);
  const size_t lds = (size_t)MR * K * sizeof(__half);
  hipLaunchKernelGGL((awq_gemv_kernel<MR>), grid, block, lds, st, (const __half*)x, q,
                     (const __half*)s, (const __half*)z, (__half*)y, N, K);
  return hipGetLastError();
}

hipError_t launch_awq_gemv(int M, int N, int K, const void* x, const uint8_t* q, const void* s,
                           const void* z, void* y, hipStream_t st) {
  const int gpl = ((K >> 6) + 63) / 64;
  if (M * gpl <= 4) {
#define SVDQ_REG(MR_, GPL_) if (M == MR_ && gpl == GPL_) return launch_reg<MR_, GPL_>(N, K, x, q, s, z, y, st)
    SVDQ_REG(1, 1); SVDQ_REG(1, 2); SVDQ_REG(1, 3); SVDQ_REG(1, 4);
    SVDQ_REG(2, 1); SVDQ_REG(2, 2); SVDQ_REG(3, 1); SVDQ_REG(4, 1);
#undef SVDQ_REG
  }
  switch (M) {
    case 1: return launch_lds<1>(N, K, x, q, s, z, y, st);
    case 2: return launch_lds<2>(N, K, x, q, s, z, y, st);
    case 3: return launch_lds<3>(N, K, x, q, s, z, y, st);
    case 4: return launch_lds<4>(N, K, x, q, s, z, y, st);
    case 5: return launch_lds<5>(N, K, x, q, s, z, y, st);
    case 6: return launch_lds<6>(N, K, x, q, s, z, y, st);
    case 7: return launch_lds<7>(N, K, x, q, s, z, y, st);
    default: return launch_lds<8>(N, K, x, q, s, z, y, st);
  }
}

}  // namespace svdq
