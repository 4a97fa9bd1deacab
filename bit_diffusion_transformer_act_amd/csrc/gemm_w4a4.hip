// svdq_gemm_w4a4: the 4-bit GEMM with the low-rank up-projection, scale
// dequantization, bias and GELU fused into one kernel (the pages fuse the
// up-projection with the 4-bit compute kernel so the 16-bit branch costs no
// extra memory pass: dothoosh.com "How Nunchaku Lite halves diffusion-model
// VRAM", fused-kernel paragraph; W4A4 with both operands 4-bit: same
// article, SVDQuant paragraph, and nextgz.net "Hugging Face brings Nunchaku
// Lite to Diffusers", section "Why W4A4 differs from weight-only backends").
//
// Tiling: 128 x 128 output tile per workgroup of 4 waves (2 x 2, 64 x 64
// per wave = 2 x 2 blocks of 32 x 32), K step 128 codes (64 packed bytes per
// row) double-buffered in LDS with a 16-byte row pad.
//
// Accumulators start from the low-rank product: lora_act (fp32 -> fp16) times
// lora_up on v_mfma_f32_32x32x16_f16, 16 ranks per instruction.
//
// INT4_G64: each lane reads 16 packed bytes (32 codes) per 32-row block
// and group; nibbles become int8 bytes holding 16 q with two ALU ops per
// word (hi = w & 0xF0F0F0F0, lo = (w << 4) & 0xF0F0F0F0), so an int32 result
// is 256 sum q_x q_w exactly. Two v_mfma_i32_32x32x32_i8 give one group's
// partial; the group's scales s_x 2^-8 and s_w are applied in fp32. A and B
// use the same permutation of k inside the instruction, which a dot product
// does not see.
//
// FP4_E2M1_B32: the packed codes are the operands of
// v_mfma_scale_f32_32x32x64_f8f6f4 as they are (lane l: row l%32, k
// 32 (l/32) .. +32), with the E8M0 byte of (row, 32-block) as the lane's
// scale; the hardware applies both scales and accumulates in fp32.
#include "common.hpp"

namespace svdq {

constexpr int GBM = 128, GBN = 128;
constexpr int GROWB = 80;  // LDS row stride (64 data bytes + 16 pad)

// 16 packed INT4 codes (two words) -> one int8 MFMA operand of 16 bytes:
// [even codes of w0, odd codes of w0, even of w1, odd of w1], each byte 16 q.
__device__ __forceinline__ v4i unpack_i4x16(uint32_t w0, uint32_t w1) {
  return v4i{(int)((w0 << 4) & 0xF0F0F0F0u), (int)(w0 & 0xF0F0F0F0u),
             (int)((w1 << 4) & 0xF0F0F0F0u), (int)(w1 & 0xF0F0F0F0u)};
}

template <int FMT, int EPI>
__global__ __launch_bounds__(256)
void gemm_w4a4_kernel(const uint8_t* __restrict__ act_codes, const void* __restrict__ act_scales,
                      const float* __restrict__ lora_act, const uint8_t* __restrict__ w_codes,
                      const void* __restrict__ w_scales, const __half* __restrict__ lora_up,
                      const __half* __restrict__ bias, __half* __restrict__ Y,
                      int M, int N, int K, int r) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][GBM * GROWB];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][GBN * GROWB];
  // INT4: fp32 scales [buf][group in step][row]; FP4: E8M0 bytes, one dword per row
  __shared__ __attribute__((aligned(16))) float sSA[2][2][GBM];
  __shared__ __attribute__((aligned(16))) float sSB[2][2][GBN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * GBN;
  const int m0 = blockIdx.y * GBM;
  const int nk = K >> 7;
  const int KB = K >> 1;  // bytes per packed row
  const int l32 = lane & 31, lh = lane >> 5;

  // ---- low-rank up-projection initialises the accumulators
  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  for (int j0 = 0; j0 < r; j0 += 16) {
    v8h a[2], b[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int m = m0 + wm * 64 + rb * 32 + l32;
      if (m < M) {
        const float4* p = reinterpret_cast<const float4*>(lora_act + (size_t)m * r + j0 + lh * 8);
        const float4 u = p[0], w = p[1];
        a[rb] = v8h{(_Float16)u.x, (_Float16)u.y, (_Float16)u.z, (_Float16)u.w,
                    (_Float16)w.x, (_Float16)w.y, (_Float16)w.z, (_Float16)w.w};
      } else {
        a[rb] = v8h{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int n = n0 + wn * 64 + cb * 32 + l32;
      b[cb] = __builtin_bit_cast(v8h, *reinterpret_cast<const uint4*>(lora_up + (size_t)n * r + j0 + lh * 8));
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[rb], b[cb], acc[rb][cb], 0, 0, 0);
  }

  // ---- global -> register staging for one K step
  // thread t: rows t/4 and 64 + t/4 of each tile, 16-byte chunk t%4
  const int ld_row = tid >> 2, ld_chk = tid & 3;
  uint4 ra[2], rbv[2];
  uint32_t rsa = 0, rsb = 0;  // scale words (2 fp16 or 4 E8M0 bytes)

  auto gload = [&](int ks) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ar = m0 + ld_row + 64 * h;
      ra[h] = (ar < M) ? *reinterpret_cast<const uint4*>(act_codes + (size_t)ar * KB + ks * 64 + ld_chk * 16)
                       : make_uint4(0, 0, 0, 0);
      const int br = n0 + ld_row + 64 * h;
      rbv[h] = *reinterpret_cast<const uint4*>(w_codes + (size_t)br * KB + ks * 64 + ld_chk * 16);
    }
    if (tid < GBM) {
      const int ar = m0 + tid;
      if (FMT == 0)
        rsa = (ar < M) ? *reinterpret_cast<const uint32_t*>(reinterpret_cast<const __half*>(act_scales) + (size_t)ar * (K >> 6) + 2 * ks) : 0u;
      else
        rsa = (ar < M) ? *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(act_scales) + (size_t)ar * (K >> 5) + 4 * ks) : 0u;
    } else {
      const int br = n0 + tid - GBM;
      if (FMT == 0)
        rsb = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const __half*>(w_scales) + (size_t)br * (K >> 6) + 2 * ks);
      else
        rsb = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(w_scales) + (size_t)br * (K >> 5) + 4 * ks);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<uint4*>(&sA[buf][(ld_row + 64 * h) * GROWB + ld_chk * 16]) = ra[h];
      *reinterpret_cast<uint4*>(&sB[buf][(ld_row + 64 * h) * GROWB + ld_chk * 16]) = rbv[h];
    }
    if (tid < GBM) {
      if (FMT == 0) {
        const __half2 hv = __builtin_bit_cast(__half2, rsa);
        sSA[buf][0][tid] = __low2float(hv) * 0.00390625f;   // fold the 16 x 16 nibble shift
        sSA[buf][1][tid] = __high2float(hv) * 0.00390625f;
      } else {
        reinterpret_cast<uint32_t*>(&sSA[buf][0][0])[tid] = rsa;
      }
    } else {
      const int t = tid - GBM;
      if (FMT == 0) {
        const __half2 hv = __builtin_bit_cast(__half2, rsb);
        sSB[buf][0][t] = __low2float(hv);
        sSB[buf][1][t] = __high2float(hv);
      } else {
        reinterpret_cast<uint32_t*>(&sSB[buf][0][0])[t] = rsb;
      }
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int ks = 0; ks < nk; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < nk) gload(ks + 1);

#pragma unroll
    for (int g = 0; g < 2; ++g) {
      uint4 ap[2], bp[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        ap[rb] = *reinterpret_cast<const uint4*>(&sA[buf][(wm * 64 + rb * 32 + l32) * GROWB + g * 32 + lh * 16]);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
        bp[cb] = *reinterpret_cast<const uint4*>(&sB[buf][(wn * 64 + cb * 32 + l32) * GROWB + g * 32 + lh * 16]);

      if constexpr (FMT == 0) {
        v4i a0[2], a1[2], b0[2], b1[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          a0[rb] = unpack_i4x16(ap[rb].x, ap[rb].y);
          a1[rb] = unpack_i4x16(ap[rb].z, ap[rb].w);
        }
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          b0[cb] = unpack_i4x16(bp[cb].x, bp[cb].y);
          b1[cb] = unpack_i4x16(bp[cb].z, bp[cb].w);
        }
        float sw[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) sw[cb] = sSB[buf][g][wn * 64 + cb * 32 + l32];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          // rows of this lane in block rb: (v/4)*8 + lh*4 + v%4
          float sx[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 t4 = *reinterpret_cast<const float4*>(&sSA[buf][g][wm * 64 + rb * 32 + q * 8 + lh * 4]);
            sx[4 * q + 0] = t4.x; sx[4 * q + 1] = t4.y; sx[4 * q + 2] = t4.z; sx[4 * q + 3] = t4.w;
          }
#pragma unroll
          for (int cb = 0; cb < 2; ++cb) {
            v16i p = {};
            p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0[rb], b0[cb], p, 0, 0, 0);
            p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1[rb], b1[cb], p, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 16; ++v)
              acc[rb][cb][v] = fmaf((float)p[v], sx[v] * sw[cb], acc[rb][cb][v]);
          }
        }
      } else {
        const uint32_t* ea = reinterpret_cast<const uint32_t*>(&sSA[buf][0][0]);
        const uint32_t* eb = reinterpret_cast<const uint32_t*>(&sSB[buf][0][0]);
        const int sh = 8 * (2 * g + lh);
        int sa[2], sb[2];
        v8i av[2], bv[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          sa[rb] = (int)((ea[wm * 64 + rb * 32 + l32] >> sh) & 0xFFu);
          av[rb] = v8i{(int)ap[rb].x, (int)ap[rb].y, (int)ap[rb].z, (int)ap[rb].w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          sb[cb] = (int)((eb[wn * 64 + cb * 32 + l32] >> sh) & 0xFFu);
          bv[cb] = v8i{(int)bp[cb].x, (int)bp[cb].y, (int)bp[cb].z, (int)bp[cb].w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                av[rb], bv[cb], acc[rb][cb], 4, 4, 0, sa[rb], 0, sb[cb]);
      }
    }

    if (ks + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: bias, activation, fp16 store
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int n = n0 + wn * 64 + cb * 32 + l32;
    const float bn = bias ? __half2float(bias[n]) : 0.f;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 64 + rb * 32 + (v >> 2) * 8 + lh * 4 + (v & 3);
        if (m < M) {
          float yv = acc[rb][cb][v] + bn;
          if (EPI == 1) yv = gelu_tanh_f32(yv);
          Y[(size_t)m * N + n] = __float2half_rn(yv);
        }
      }
    }
  }
}

hipError_t launch_gemm_w4a4(int fmt, int M, int N, int K, int r, const uint8_t* ac, const void* as,
                            const float* la, const uint8_t* wc, const void* ws, const void* lu,
                            const void* bias, int epi, void* Y, hipStream_t st) {
  const dim3 grid(N / GBN, (M + GBM - 1) / GBM), block(256);
#define SVDQ_LAUNCH(F, E)                                                                   \
  hipLaunchKernelGGL((gemm_w4a4_kernel<F, E>), grid, block, 0, st, ac, as, la, wc, ws,      \
                     (const __half*)lu, (const __half*)bias, (__half*)Y, M, N, K, r)
  if (fmt == 0) {
    if (epi == 0) SVDQ_LAUNCH(0, 0); else SVDQ_LAUNCH(0, 1);
  } else {
    if (epi == 0) SVDQ_LAUNCH(1, 0); else SVDQ_LAUNCH(1, 1);
  }
#undef SVDQ_LAUNCH
  return hipGetLastError();
}

}  // namespace svdq
