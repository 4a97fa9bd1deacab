// svdq_gemm_w4a4, FP4 E2M1 / E8M0-b32 format, large-tile kernel.
//
// Same contract as the INT4 path (the 4-bit GEMM with the low-rank
// up-projection, bias and GELU fused, dothoosh.com "How Nunchaku Lite halves
// diffusion-model VRAM", fused-kernel paragraph and kernel-family list, the
// 4-bit float variant of svdq_w4a4), for a format with no per-group VALU work:
// v_mfma_scale_f32_32x32x64_f8f6f4 takes the packed E2M1 codes as they are
// (lane l: row l%32, k 32 (l/32) .. +32) and the E8M0 byte of (row, 32-block)
// as the lane's scale, and accumulates in fp32.
//
// With no VALU work the bound is the matrix core, so the tile is sized for
// operand reuse: 256 x 256 per workgroup, 4 waves of 128 x 128 (4 x 4 blocks
// of 32 x 32, 256 fp32 accumulators per lane held in AGPRs). Per K step of 128
// codes a workgroup moves 34 KB into LDS for 8.4 M MACs (about 33 B/clk per CU
// at the MXFP4 rate, half of what a 128 x 128 tile would need). The ring has 4
// stages of 34 KB (one workgroup per CU); loads are LDS-DMA as in the INT4
// kernel, one barrier per step. This file is built with MFMA results in AGPRs
// (no VGPR-form flag): the accumulators are only touched by MFMAs until the
// epilogue.
#include <atomic>

#include "common.hpp"
#include "pipeline.hpp"

namespace svdq {

namespace fp4big {
constexpr int BM = 256, BN = 256;
constexpr int RB = 4, CB = 4;                 // 32 x 32 blocks per wave
constexpr int A_BYTES = BM * 64, B_BYTES = BN * 64;
constexpr int SC_ROWS = BM + BN;              // one scale word (4 E8M0 bytes) per row
constexpr int STAGE = A_BYTES + B_BYTES + SC_ROWS * 4;
constexpr int STAGES = 4;
constexpr int LDS = STAGES * STAGE;
constexpr int DMA_PER_STEP = BM / 64 + BN / 64 + SC_ROWS / 256;   // per thread
}  // namespace fp4big

template <int EPI>
__global__ __launch_bounds__(256, 1)
void gemm_fp4_big_kernel(const uint8_t* __restrict__ act_codes, const uint8_t* __restrict__ act_scales,
                         const __half* __restrict__ lora_act, const uint8_t* __restrict__ w_codes,
                         const uint8_t* __restrict__ w_scales, const __half* __restrict__ lora_up,
                         const __half* __restrict__ bias, __half* __restrict__ Y,
                         int M, int N, int K, int r) {
  using namespace fp4big;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;

  // XCD-aware grouped tile order (4 M-tiles per group: one 256 x 256 tile per
  // CU, so the ~32 tiles resident on an XCD form a 4 x 8 patch)
  const int ntm = (M + BM - 1) / BM;
  const int ntn = N / BN;
  const int ntiles = ntm * ntn;
  int pid = blockIdx.x;
  if ((ntiles & 7) == 0) pid = (pid & 7) * (ntiles >> 3) + (pid >> 3);
  constexpr int GROUP_M = 4;
  const int gsz = GROUP_M * ntn;
  const int first_m = (pid / gsz) * GROUP_M;
  const int gm = min(ntm - first_m, GROUP_M);
  const int m0 = (first_m + (pid % gsz) % gm) * BM;
  const int n0 = ((pid % gsz) / gm) * BN;
  const int nk = K >> 7;
  const int KB = K >> 1;
  const int sstride = K >> 5;

  // ---- DMA sources: wave w fills rows [64 w, 64 w + 64) of A and of B
  const uint8_t* ga[BM / 64];
  const uint8_t* gb[BN / 64];
  const uint8_t* gs[SC_ROWS / 256];
  uint32_t la_off[BM / 64], lb_off[BN / 64], ls_off[SC_ROWS / 256];
  const uint32_t lds0 = lds_addr(smem);
#pragma unroll
  for (int i = 0; i < BM / 64; ++i) {
    const int rloc = wave * (BM / 4) + 16 * i;
    const int row = rloc + (lane >> 2);
    const int chunk = (lane & 3) ^ swz(row);
    ga[i] = act_codes + (size_t)min(m0 + row, M - 1) * KB + chunk * 16;
    la_off[i] = rloc * 64;
  }
#pragma unroll
  for (int i = 0; i < BN / 64; ++i) {
    const int rloc = wave * (BN / 4) + 16 * i;
    const int row = rloc + (lane >> 2);
    const int chunk = (lane & 3) ^ swz(row);
    gb[i] = w_codes + (size_t)(n0 + row) * KB + chunk * 16;
    lb_off[i] = A_BYTES + rloc * 64;
  }
#pragma unroll
  for (int i = 0; i < SC_ROWS / 256; ++i) {
    const int rloc = (wave * (SC_ROWS / 256) + i) * 64;
    const int row = rloc + lane;
    gs[i] = (row < BM) ? act_scales + (size_t)min(m0 + row, M - 1) * sstride
                       : w_scales + (size_t)(n0 + row - BM) * sstride;
    ls_off[i] = A_BYTES + B_BYTES + rloc * 4;
  }
  auto issue = [&](int ks) {
    const uint32_t base = lds0 + (uint32_t)((ks % STAGES) * STAGE);
#pragma unroll
    for (int i = 0; i < BM / 64; ++i) dma16(ga[i] + ks * 64, base + la_off[i]);
#pragma unroll
    for (int i = 0; i < BN / 64; ++i) dma16(gb[i] + ks * 64, base + lb_off[i]);
#pragma unroll
    for (int i = 0; i < SC_ROWS / 256; ++i) dma4(gs[i] + ks * 4, base + ls_off[i]);
  };
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s);

  // ---- low-rank up-projection initialises the accumulators
  v16f acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  // loads for 32 ranks are issued together so a tile pays one round trip
  for (int j0 = 0; j0 < r; j0 += 32) {
    const int nj = min(r - j0, 32) >> 4;
    uint4 ua[RB][2], ub[CB][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int m = m0 + wm * 128 + rb * 32 + l32;
        ua[rb][h] = (m < M && h < nj)
                        ? *reinterpret_cast<const uint4*>(lora_act + (size_t)m * r + j0 + 16 * h + lh * 8)
                        : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int n = n0 + wn * 128 + cb * 32 + l32;
        ub[cb][h] = (h < nj) ? *reinterpret_cast<const uint4*>(lora_up + (size_t)n * r + j0 + 16 * h + lh * 8)
                             : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, ua[rb][h]),
                                                               __builtin_bit_cast(v8h, ub[cb][h]),
                                                               acc[rb][cb], 0, 0, 0);
  }

  int arow[RB], brow[CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) arow[rb] = wm * 128 + rb * 32 + l32;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) brow[cb] = wn * 128 + cb * 32 + l32;

  for (int ks = 0; ks < nk; ++ks) {
    if (ks + STAGES - 2 < nk) waitvm<DMA_PER_STEP * (STAGES - 2)>();
    else waitvm<0>();
    __syncthreads();
    if (ks + STAGES - 1 < nk) issue(ks + STAGES - 1);

    const uint8_t* st = smem + (ks % STAGES) * STAGE;
    const uint8_t* sA = st;
    const uint8_t* sB = st + A_BYTES;
    const uint32_t* sS = reinterpret_cast<const uint32_t*>(st + A_BYTES + B_BYTES);
    uint32_t ea[RB], eb[CB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) ea[rb] = sS[arow[rb]];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) eb[cb] = sS[BM + brow[cb]];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int sh = 8 * (2 * g + lh);
      v8i av[RB], bv[CB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int rr = arow[rb];
        const uint4 ap = *reinterpret_cast<const uint4*>(sA + rr * 64 + (((g * 2 + lh) ^ swz(rr)) << 4));
        av[rb] = v8i{(int)ap.x, (int)ap.y, (int)ap.z, (int)ap.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int rr = brow[cb];
        const uint4 bp = *reinterpret_cast<const uint4*>(sB + rr * 64 + (((g * 2 + lh) ^ swz(rr)) << 4));
        bv[cb] = v8i{(int)bp.x, (int)bp.y, (int)bp.z, (int)bp.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              av[rb], bv[cb], acc[rb][cb], 4, 4, 0, (int)((ea[rb] >> sh) & 0xFFu), 0,
              (int)((eb[cb] >> sh) & 0xFFu));
    }
  }

  // ---- epilogue: bias and activation, then the tile goes through LDS (the ring
  // is free now) so that Y is written as whole rows with 16-byte stores.
  constexpr int TP = BN + 8;   // padded row (halves) of the staging tile
  static_assert(BM * TP * 2 <= LDS, "staging tile must fit in the ring");
  __syncthreads();
  __half* tile = reinterpret_cast<__half*>(smem);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int nl = brow[cb];
    const float bn = bias ? __half2float(bias[n0 + nl]) : 0.f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float yv = acc[rb][cb][v] + bn;
        if (EPI == 1) yv = gelu_tanh_f32(yv);
        tile[(wm * 128 + rb * 32 + (v >> 2) * 8 + lh * 4 + (v & 3)) * TP + nl] = __float2half_rn(yv);
      }
  }
  __syncthreads();
  for (int c = tid; c < BM * (BN / 8); c += 256) {
    const int row = c / (BN / 8), c8 = c - row * (BN / 8);
    if (m0 + row < M)
      *reinterpret_cast<uint4*>(Y + (size_t)(m0 + row) * N + n0 + c8 * 8) =
          *reinterpret_cast<const uint4*>(tile + row * TP + c8 * 8);
  }
}

// Large-tile FP4 launch; returns hipErrorNotSupported (without launching) when
// the shape does not suit it, so the caller can fall back to the 128 x 128 kernel.
hipError_t launch_gemm_fp4_big(int M, int N, int K, int r, const uint8_t* ac, const void* as,
                               const void* la, const uint8_t* wc, const void* ws, const void* lu,
                               const void* bias, int epi, void* Y, hipStream_t st) {
  using namespace fp4big;
  if (N % BN != 0) return hipErrorNotSupported;
  const int ntiles = ((M + BM - 1) / BM) * (N / BN);
  if (ntiles < 256) return hipErrorNotSupported;   // too few tiles to fill 256 CUs
  auto kern = epi ? gemm_fp4_big_kernel<1> : gemm_fp4_big_kernel<0>;
  static std::atomic<int> raised[2] = {0, 0};
  if (!raised[epi].load(std::memory_order_acquire)) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
    raised[epi].store(1, std::memory_order_release);
  }
  hipLaunchKernelGGL(kern, dim3(ntiles), dim3(256), LDS, st, ac, (const uint8_t*)as, (const __half*)la, wc,
                     (const uint8_t*)ws, (const __half*)lu, (const __half*)bias, (__half*)Y, M, N, K, r);
  return hipGetLastError();
}

}  // namespace svdq
