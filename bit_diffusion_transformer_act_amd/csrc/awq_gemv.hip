// awq_gemv_w4a16: 4-bit weights, 16-bit activations, for the memory-bound
// modulation / adaptive-norm projections (dothoosh.com "How Nunchaku Lite
// halves diffusion-model VRAM", kernel-family list, the awq_w4a16 entry;
// int4 with group size 64 in the quantization_config block).
//
//   y[m,n] = sum_k x[m,k] (q[n,k] - z[n,g]) s[n,g],  g = k / 64
//
// HBM-bound: every weight byte is read once, with 8-byte loads from
// consecutive lanes (512 contiguous bytes per wave instruction). x is staged
// once per workgroup in LDS, pre-arranged so that the two fp16 values paired
// with codes k and k+4 of an 8-code word sit in one 32-bit word. Dequant
// uses the fp16 bit trick: (word >> 4j) & 0x000F000F | 0x64006400 is the
// packed pair (1024 + q_j, 1024 + q_{j+4}); subtracting 1024 + z in packed
// fp16 gives q - z exactly, and v_dot2_f32_f16 accumulates x (q - z) in fp32.
#include "common.hpp"

namespace svdq {

constexpr int kGemvWaves = 4;
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
    const uint32_t a[4] = {v.x, v.y, v.z, v.w};  // halves (0,1) (2,3) (4,5) (6,7)
    uint32_t* o = xs + (size_t)idx * 4;
    // pair j = (x_j, x_{j+4})
    o[0] = (a[0] & 0xFFFFu) | (a[2] << 16);
    o[1] = (a[0] >> 16) | (a[2] & 0xFFFF0000u);
    o[2] = (a[1] & 0xFFFFu) | (a[3] << 16);
    o[3] = (a[1] >> 16) | (a[3] & 0xFFFF0000u);
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nbase = (blockIdx.x * kGemvWaves + wave) * kRowsPerWave;
  const int chunks = K >> 4;        // 16 codes (8 bytes) per chunk
  const int gstride = K >> 6;

  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int n = nbase + rr;
    if (n >= N) break;
    const uint8_t* crow = codes + (size_t)n * (K >> 1);
    float acc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[m] = 0.f;
#pragma unroll 4
    for (int c = lane; c < chunks; c += 64) {
      const uint2 w = *reinterpret_cast<const uint2*>(crow + (size_t)c * 8);
      const int g = c >> 2;
      const float s = __half2float(scales[(size_t)n * gstride + g]);
      const _Float16 zb = (_Float16)(-1024.0f) - (_Float16)__half2float(zeros[(size_t)n * gstride + g]);
      const v2h nz = {zb, zb};
      float part[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) part[m] = 0.f;
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const uint32_t word = d ? w.y : w.x;
        const int sg = 2 * c + d;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t hb = ((word >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
          const v2h hz = __builtin_bit_cast(v2h, hb) + nz;   // (q_j - z, q_{j+4} - z), exact
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            const v2h xp = __builtin_bit_cast(v2h, xs[((size_t)m * segs + sg) * 4 + j]);
            part[m] = __builtin_amdgcn_fdot2(hz, xp, part[m], false);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MR; ++m) acc[m] = fmaf(part[m], s, acc[m]);
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

template <int MR>
static hipError_t launch_g(int N, int K, const void* x, const uint8_t* q, const void* s,
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
  switch (M) {
    case 1: return launch_g<1>(N, K, x, q, s, z, y, st);
    case 2: return launch_g<2>(N, K, x, q, s, z, y, st);
    case 3: return launch_g<3>(N, K, x, q, s, z, y, st);
    case 4: return launch_g<4>(N, K, x, q, s, z, y, st);
    case 5: return launch_g<5>(N, K, x, q, s, z, y, st);
    case 6: return launch_g<6>(N, K, x, q, s, z, y, st);
    case 7: return launch_g<7>(N, K, x, q, s, z, y, st);
    default: return launch_g<8>(N, K, x, q, s, z, y, st);
  }
}

}  // namespace svdq
