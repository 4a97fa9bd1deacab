// svdq_quantize_act: fused activation smoothing, low-rank down-projection
// and per-group 4-bit activation quantization, one pass over X.
//
// The pages' fused kernels put the low-rank down-projection next to the
// quantization kernel so the 16-bit branch costs no extra memory pass
// (dothoosh.com "How Nunchaku Lite halves diffusion-model VRAM", fused-kernel
// paragraph; nextgz.net "Hugging Face brings Nunchaku Lite to Diffusers",
// section "Why W4A4 differs from weight-only backends").
//
// Work split (gfx950, wave64): a workgroup of 16 waves owns 16 rows of X and
// all of K; wave w handles 64-wide K steps w, w+16, w+32, ... In a step,
// lane l holds row (l % 16) and the 16 contiguous channels
// [64 s + 16 (l / 16), +16): two 16-byte loads. That register tile is at the
// same time
//   - the A operand of two v_mfma_f32_16x16x32_f16 against lora_down (the
//     MFMA k index (l/16)*8 + j is mapped to channel 64 s + 16 (l/16) + 8 h + j
//     for call h = 0, 1; B uses the same map, so the dot product is exact
//     over the permuted k), and
//   - one quarter of an INT4 group (lanes l, l^16, l^32, l^48) or one half
//     of an FP4 block (lanes l, l^16), whose amax is a two-/one-step xor
//     shuffle reduction.
// Partial low-rank sums of the 16 waves meet in LDS and are added in a fixed
// order, so lora_act (stored as fp16) is deterministic.
#include <atomic>

#include "common.hpp"

namespace svdq {

template <int FMT, int NCB>
__global__ __launch_bounds__(1024)
void quantize_act_kernel(const __half* __restrict__ X, const float* __restrict__ smooth_inv,
                         const __half* __restrict__ lora_down, uint8_t* __restrict__ codes,
                         void* __restrict__ scales, __half* __restrict__ lora_act,
                         int M, int K) {
#pragma clang fp contract(off)
  extern __shared__ float red[];  // [16 waves][16 rows][16 * NCB]
  constexpr int kWaves = 16;
  constexpr int R = 16 * NCB;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m0 = blockIdx.x * 16;
  const int row = m0 + (lane & 15);
  const int q4 = lane >> 4;
  const bool row_ok = row < M;
  const int steps = K >> 6;
  const size_t xrow = (size_t)row * (size_t)K;

  v4f lacc[NCB > 0 ? NCB : 1];
#pragma unroll
  for (int c = 0; c < (NCB > 0 ? NCB : 1); ++c) lacc[c] = v4f{0.f, 0.f, 0.f, 0.f};

  // X for the wave's first step; each iteration prefetches the next step's
  // X before working on the current one.
  uint4 xa = make_uint4(0, 0, 0, 0), xb = make_uint4(0, 0, 0, 0);
  if (row_ok && wave < steps) {
    const uint4* p = reinterpret_cast<const uint4*>(X + xrow + wave * 64 + q4 * 16);
    xa = p[0];
    xb = p[1];
  }
  for (int s = wave; s < steps; s += kWaves) {
    const int k0 = s * 64 + q4 * 16;
    const uint4 ca = xa, cb = xb;
    if (row_ok && s + kWaves < steps) {
      const uint4* p = reinterpret_cast<const uint4*>(X + xrow + k0 + kWaves * 64);
      xa = p[0];
      xb = p[1];
    }
    if constexpr (NCB > 0) {
      const v8h a0 = __builtin_bit_cast(v8h, ca);
      const v8h a1 = __builtin_bit_cast(v8h, cb);
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        const uint4* pb = reinterpret_cast<const uint4*>(lora_down + (size_t)(c * 16 + (lane & 15)) * K + k0);
        const v8h b0 = __builtin_bit_cast(v8h, pb[0]);
        const v8h b1 = __builtin_bit_cast(v8h, pb[1]);
        lacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0, lacc[c], 0, 0, 0);
        lacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1, lacc[c], 0, 0, 0);
      }
    }
    // smoothing: x_hat = fl32(fp32(x) * smooth_inv), a plain IEEE multiply
    float xh[16];
    {
      const float4* ps = reinterpret_cast<const float4*>(smooth_inv + k0);
      const __half* ha = reinterpret_cast<const __half*>(&ca);
      const __half* hb = reinterpret_cast<const __half*>(&cb);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 sv = ps[i];
        const __half* hs = (i < 2) ? ha + 4 * i : hb + 4 * (i - 2);
        xh[4 * i + 0] = __half2float(hs[0]) * sv.x;
        xh[4 * i + 1] = __half2float(hs[1]) * sv.y;
        xh[4 * i + 2] = __half2float(hs[2]) * sv.z;
        xh[4 * i + 3] = __half2float(hs[3]) * sv.w;
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(xh[i]));

    uint32_t w0 = 0, w1 = 0;
    if constexpr (FMT == 0) {
      // INT4, group 64 = this step: reduce over the four lanes of the row.
      amax = lane_max_xor(amax, 16);
      amax = lane_max_xor(amax, 32);
      const float s32 = amax / 7.0f;                    // IEEE division
      const __half s16 = __float2half_rn(fminf(s32, 65504.0f));
      const float sf = __half2float(s16);
      if (sf != 0.0f) {
        // q = clamp(rint(fl32(x_hat / s)), -7, 7) without a division per value:
        // y = x_hat * rcp(s) is within 2^-19 |y| of fl32(x_hat / s) (rcp and the
        // multiply are each within an ulp), so the two round to the same integer
        // unless y lies within 2^-16 of a half-integer; only such values are
        // recomputed with the IEEE division. Clamping first is harmless: every
        // value beyond +-7 maps to +-7 either way. Rounding is the add/subtract
        // of 1.5 * 2^23, whose low mantissa bits are then the two's-complement
        // code.
        const float rs = __builtin_amdgcn_rcpf(sf);
        bool near_tie = false;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float c = __builtin_amdgcn_fmed3f(xh[i] * rs, -7.0f, 7.0f);
          const float yv = c + 12582912.0f;
          const float rv = yv - 12582912.0f;
          near_tie |= fabsf(c - rv) > 0.4999847412109375f;   // 0.5 - 2^-16
          const uint32_t nib = __float_as_uint(yv) & 0xFu;
          if (i < 8) w0 |= nib << (4 * i); else w1 |= nib << (4 * (i - 8));
        }
        if (near_tie) {
          w0 = 0;
          w1 = 0;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float q = rintf(xh[i] / sf);                // IEEE division, ties to even
            q = fminf(fmaxf(q, -7.0f), 7.0f);
            const uint32_t nib = (uint32_t)((int)q) & 0xFu;
            if (i < 8) w0 |= nib << (4 * i); else w1 |= nib << (4 * (i - 8));
          }
        }
      }
      if (row_ok) {
        *reinterpret_cast<uint2*>(codes + (size_t)row * (K >> 1) + s * 32 + q4 * 8) = make_uint2(w0, w1);
        if (q4 == 0) reinterpret_cast<__half*>(scales)[(size_t)row * (K >> 6) + s] = s16;
      }
    } else {
      // FP4 E2M1, block 32 = half a step: reduce over the lane pair.
      amax = lane_max_xor(amax, 16);
      uint32_t sc = 0;
      if (amax != 0.0f) {
        int ex;
        const float mant = frexpf(amax, &ex);           // amax = mant * 2^ex, mant in [0.5, 1)
        int e = (mant <= 0.75f) ? ex - 3 : ex - 2;      // smallest e with 6 * 2^e >= amax
        e = min(max(e, -127), 127);
        sc = (uint32_t)(e + 127);
        const float p = ldexpf(1.0f, -e);               // exact power of two
        // u = fl32(x_hat / 2^e) = x_hat * 2^-e; v_cvt_scalef32_pk_fp4_f32 with
        // scale 1 rounds two values to E2M1 (nearest, ties to even mantissa,
        // saturating at 6, sign kept, first value in the low nibble) and writes
        // the byte selected by its last operand.
        w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, xh[0] * p, xh[1] * p, 1.0f, 0);
        w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, xh[2] * p, xh[3] * p, 1.0f, 1);
        w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, xh[4] * p, xh[5] * p, 1.0f, 2);
        w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, xh[6] * p, xh[7] * p, 1.0f, 3);
        w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, xh[8] * p, xh[9] * p, 1.0f, 0);
        w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, xh[10] * p, xh[11] * p, 1.0f, 1);
        w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, xh[12] * p, xh[13] * p, 1.0f, 2);
        w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, xh[14] * p, xh[15] * p, 1.0f, 3);
      }
      if (row_ok) {
        *reinterpret_cast<uint2*>(codes + (size_t)row * (K >> 1) + s * 32 + q4 * 8) = make_uint2(w0, w1);
        if ((q4 & 1) == 0) reinterpret_cast<uint8_t*>(scales)[(size_t)row * (K >> 5) + 2 * s + (q4 >> 1)] = (uint8_t)sc;
      }
    }
  }

  if constexpr (NCB > 0) {
    // lane l holds rows (l/16)*4 + i, column c*16 + l%16 of the wave's partial
#pragma unroll
    for (int c = 0; c < NCB; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[(wave * 16 + (lane >> 4) * 4 + i) * R + c * 16 + (lane & 15)] = lacc[c][i];
    __syncthreads();
    for (int t = threadIdx.x; t < 16 * R; t += blockDim.x) {
      const int rr = t / R, cc = t - rr * R;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) sum += red[(w * 16 + rr) * R + cc];
      if (m0 + rr < M) lora_act[(size_t)(m0 + rr) * R + cc] = __float2half_rn(sum);
    }
  }
}

template <int FMT, int NCB>
static hipError_t launch_q(int M, int K, const void* X, const float* si, const void* ld,
                           uint8_t* codes, void* scales, void* la, hipStream_t st) {
  const dim3 grid((M + 15) / 16), block(1024);
  const size_t lds = NCB > 0 ? (size_t)16 * 16 * 16 * NCB * sizeof(float) : 0;
  if (lds > 65536) {
    static std::atomic<int> raised{0};
    if (!raised.load(std::memory_order_acquire)) {
      const hipError_t e = hipFuncSetAttribute(
          reinterpret_cast<const void*>(&quantize_act_kernel<FMT, NCB>),
          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      raised.store(1, std::memory_order_release);
    }
  }
  hipLaunchKernelGGL((quantize_act_kernel<FMT, NCB>), grid, block, lds, st,
                     (const __half*)X, si, (const __half*)ld, codes, scales, (__half*)la, M, K);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_q_r(int M, int K, int r, const void* X, const float* si, const void* ld,
                             uint8_t* codes, void* scales, void* la, hipStream_t st) {
  switch (r / 16) {
    case 0: return launch_q<FMT, 0>(M, K, X, si, ld, codes, scales, la, st);
    case 1: return launch_q<FMT, 1>(M, K, X, si, ld, codes, scales, la, st);
    case 2: return launch_q<FMT, 2>(M, K, X, si, ld, codes, scales, la, st);
    case 3: return launch_q<FMT, 3>(M, K, X, si, ld, codes, scales, la, st);
    case 4: return launch_q<FMT, 4>(M, K, X, si, ld, codes, scales, la, st);
    case 5: return launch_q<FMT, 5>(M, K, X, si, ld, codes, scales, la, st);
    case 6: return launch_q<FMT, 6>(M, K, X, si, ld, codes, scales, la, st);
    case 7: return launch_q<FMT, 7>(M, K, X, si, ld, codes, scales, la, st);
    default: return launch_q<FMT, 8>(M, K, X, si, ld, codes, scales, la, st);
  }
}

hipError_t launch_quantize_act(int fmt, int M, int K, int r, const void* X, const float* si,
                               const void* ld, uint8_t* codes, void* scales, void* la,
                               hipStream_t st) {
  if (fmt == 0) return launch_q_r<0>(M, K, r, X, si, ld, codes, scales, la, st);
  return launch_q_r<1>(M, K, r, X, si, ld, codes, scales, la, st);
}

}  // namespace svdq
