// svdq_quantize_act: fused activation smoothing, low-rank down-projection
// and per-group 4-bit activation quantization, one pass over X.
//
// The pages' fused kernels put the low-rank down-projection next to the
// quantization kernel so the 16-bit branch costs no extra memory pass
// (dothoosh.com "How Nunchaku Lite halves diffusion-model VRAM", fused-kernel
// paragraph; nextgz.net "Hugging Face brings Nunchaku Lite to Diffusers",
// section "Why W4A4 differs from weight-only backends").
//
// Work split (gfx950, wave64): a workgroup of W waves (4, 8 or 16) owns 16 rows
// of X and all of K (or, with few rows and a long K, one slice of K: see
// launch_q_r); wave w handles 64-wide K steps w, w+W, w+2W, ..., with the
// loads of its next one or two steps in flight. The loads are the kernel's
// bottleneck: the vector memory unit spends about 50 cycles on an instruction
// that touches 16 half lines and about 17 on one that covers 8 whole lines, so
// with a low-rank pass (X plus two 16-rank blocks of lora_down per step at
// rank 32) every load covers 8 whole 128-byte lines and a per-wave LDS
// scratch turns them into the layout below. In a step, lane l holds row
// (l % 16) and two 8-channel chunks: q*8 .. +8 and 32 + q*8 .. +8 of the step
// (q = l / 16). That register tile is at the same time
//   - the A operands of two v_mfma_f32_16x16x32_f16 against lora_down, in the
//     instruction's own layout (lane l: row l % 16, k 8 (l / 16) .. +8), one
//     call per 32-channel half, and
//   - a quarter of an INT4 group (lanes l, l^16, l^32, l^48), or a quarter of
//     each of the two FP4 blocks of the step, whose amax is a two-step xor
//     shuffle reduction.
// smooth_inv is staged in LDS once per workgroup (a global-load variant serves
// K beyond the LDS budget). Partial low-rank sums of the W waves meet in LDS
// and are added in a fixed order (then the slices', in slice order, when K is
// split), so lora_act (stored in fp32) is deterministic.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace svdq {

constexpr int kQuantLdsMax = 144 * 1024;   // LDS budget per workgroup (gfx950 has 160 KB)

// LDS bytes besides smooth_inv: per wave a re-layout scratch of two blocks of
// 16 rows x 128 bytes (X, and the 16-rank blocks of lora_down one after the
// other), which the low-rank partials reuse after the main loop, then two
// round buffers (sized for the 4 scale bytes per step of NVFP4)
template <int WAVES>
constexpr size_t quant_scratch_bytes(int ncb) {
  const size_t scr = ncb > 0 ? (size_t)WAVES * 2 * 2048 : 0;   // none without a low-rank pass
  const size_t part = (size_t)WAVES * 16 * 16 * ncb * sizeof(float);
  return scr > part ? scr : part;
}
template <int WAVES>
constexpr size_t quant_lds_bytes(int ncb) {
  return quant_scratch_bytes<WAVES>(ncb) + 2 * (size_t)(16 * (WAVES * 32 + 16) + 16 * WAVES * 4);
}

// E4M3 (OCP FP8, bias 7) byte of a non-negative fp32 value: round to nearest,
// ties to the even mantissa, saturating at 448 (0x7E). Below 2^-6 the quantum
// is 2^-9 (a * 512 is exact); above, the fp32 mantissa is rounded to 3 bits in
// the integer domain (a carry moves into the exponent, as it should).
__device__ __forceinline__ uint32_t e4m3_rne_byte(float a) {
  if (!(a < 448.0f)) return 0x7Eu;
  if (a < 0.015625f) return (uint32_t)__builtin_rintf(a * 512.0f);
  uint32_t b = __float_as_uint(a);
  b += 0x7FFFFu + ((b >> 20) & 1u);
  return min((b >> 20) - ((127u - 7u) << 3), 0x7Eu);
}

// value of an E4M3 byte below 0x7F (exact in fp32)
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  return c < 8u ? (float)c * 0.001953125f : __uint_as_float((((c >> 3) + 120u) << 23) | ((c & 7u) << 20));
}

// gridDim.y = S > 1 splits K: workgroup (b, y) takes rows 16 b .. +16 over the
// y-th of S slices of whole 64-channel steps. Then
//  - LORA_ONLY: the slice's low-rank partial sums (fp32) go to the tail of each
//    row of `codes` (S r 4 bytes before the row's end, slice y at y r 4), no
//    codes or scales;
//  - NCB = 0: codes and scales of the slice; with rq > 0, the workgroup of the
//    last slice first adds the S partials of its rows in slice order and stores
//    lora_act (rq wide), before it writes the codes that overwrite them (the
//    tail lies inside its own slice, and the partials were written by an
//    earlier launch on the same stream).
// LORA_ONLY with S = 1: lora_act alone, in the fused kernel's summation order.
template <int IO, int FMT, int NCB, int WAVES, bool SLDS, bool LORA_ONLY>
__global__ __launch_bounds__(64 * WAVES)
void quantize_act_kernel(const uint16_t* __restrict__ X, const float* __restrict__ smooth_inv,
                         const uint16_t* __restrict__ lora_down, uint8_t* __restrict__ codes,
                         void* __restrict__ scales, float* __restrict__ lora_act,
                         int M, int K, float gs, float gs6, int rq) {
#pragma clang fp contract(off)
  // LDS: the waves' re-layout scratch (reused after the main loop for the
  // [WAVES][16 rows][16 * NCB] low-rank partials), two round buffers (codes,
  // then scales, of 16 rows x WAVES steps), then smooth_inv[K] if SLDS
  extern __shared__ float lds_f[];
  constexpr int R = 16 * NCB;
  constexpr int NL = NCB > 0 ? NCB : 1;
  constexpr int CROW = WAVES * 32 + 16;         // padded code row of a round (bytes)
  constexpr int SB = FMT == 2 ? 4 : 2;          // scale bytes per row and step
  constexpr int SROW = WAVES * SB;              // scale row of a round (bytes)
  constexpr int RBUF = 16 * CROW + 16 * SROW;   // one round buffer (bytes, multiple of 16)
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float* red = lds_f;
  uint4* scr = reinterpret_cast<uint4*>(lds_f) + (size_t)wave * 2 * 128;   // this wave's scratch (NCB > 0)
  uint8_t* rbuf = reinterpret_cast<uint8_t*>(lds_f) + quant_scratch_bytes<WAVES>(NCB);
  float* s_si = reinterpret_cast<float*>(rbuf + 2 * RBUF);
  const int m0 = blockIdx.x * 16;
  const int row = m0 + (lane & 15);
  const int q4 = lane >> 4;
  const bool row_ok = row < M;
  // this workgroup's slice of the 64-channel steps (all of them when gridDim.y == 1)
  const int steps_all = K >> 6;
  const int sps = (steps_all + (int)gridDim.y - 1) / (int)gridDim.y;
  const int sbeg = (int)blockIdx.y * sps;
  const int steps = max(min(sps, steps_all - sbeg), 0);
  // With a low-rank pass (six or more loads per step) the loads read whole
  // lines: lane l reads 16 bytes (chunk l % 8) of row l / 8 and of row 8 + l / 8
  // of the 16-row block, so one instruction covers 8 128-byte lines (the vector
  // memory unit's time per instruction grows with the number of lines it
  // touches: 16 half lines cost about three times as much), and relayout()
  // moves the values to the MFMA layout. Without one (two loads per step) that
  // detour costs more than it saves, and lane l reads its own chunks of row
  // l % 16 directly. Rows past M read row M - 1 (never stored; rows are
  // independent in the MFMA and in the amax groups). An unconditional load
  // matters: a select on the load's destination would make every prefetch wait
  // for the previous one.
  constexpr bool kLines = NCB > 0;
  const int r8 = lane >> 3, c8 = lane & 7;
  const size_t xrow = (size_t)min(row, M - 1) * (size_t)K;
  const size_t xrow_a = (size_t)min(m0 + r8, M - 1) * (size_t)K;
  const size_t xrow_b = (size_t)min(m0 + 8 + r8, M - 1) * (size_t)K;

  // smooth_inv into LDS; called after the first loads of X are out, so the two
  // latencies overlap
  auto stage_si = [&]() {
    if constexpr (SLDS && !LORA_ONLY) {
      for (int i = threadIdx.x * 4; i < K; i += 64 * WAVES * 4)
        *reinterpret_cast<float4*>(s_si + i) = *reinterpret_cast<const float4*>(smooth_inv + i);
      __syncthreads();
    }
  };

  v4f lacc[NL];
#pragma unroll
  for (int c = 0; c < NL; ++c) lacc[c] = v4f{0.f, 0.f, 0.f, 0.f};

  // NCB = 0, rq > 0, last slice: lora_act from the partials at the rows' tails
  auto lora_from_partials = [&]() {
    if constexpr (NCB == 0 && !LORA_ONLY) {
      if (rq > 0 && blockIdx.y == gridDim.y - 1) {
        const int S = (int)gridDim.y;
        for (int t = threadIdx.x; t < 16 * rq; t += blockDim.x) {
          const int rr = t / rq, cc = t - rr * rq;
          if (m0 + rr < M) {
            const float* pp = reinterpret_cast<const float*>(codes + (size_t)(m0 + rr) * (K >> 1) + (K >> 1) -
                                                             (size_t)S * rq * 4);
            float sum = 0.f;
            for (int y = 0; y < S; ++y) sum += pp[y * rq + cc];
            lora_act[(size_t)(m0 + rr) * rq + cc] = sum;
          }
        }
        __syncthreads();   // every partial is read before this workgroup writes codes
      }
    }
  };

  // One step's loads: X's 16 rows x 64 channels and each 16-rank block of
  // lora_down over the same channels, as whole lines (rows r8 and 8 + r8, chunk
  // c8); relayout() turns them into the MFMA operand layout. Register sets rotate
  // so that the loads of the next one or two steps of the wave are in flight
  // while a step is processed.
  struct Step {
    uint4 xa, xb;
    uint4 lb[NL][2];
  };
  // Loads are unconditional (past the last step they re-read it, and the step
  // is never processed): a branch around them would leave the compiler's
  // vmcnt bookkeeping unsure how many are in flight, and every use would then
  // wait for all of them.
  auto load = [&](Step& d, int s) {
    if constexpr (!kLines) {
      const int k0 = (sbeg + min(s, steps - 1)) * 64 + q4 * 8;
      d.xa = *reinterpret_cast<const uint4*>(X + xrow + k0);
      d.xb = *reinterpret_cast<const uint4*>(X + xrow + k0 + 32);
      return;
    }
    const int k0 = (sbeg + min(s, steps - 1)) * 64 + c8 * 8;
    d.xa = *reinterpret_cast<const uint4*>(X + xrow_a + k0);
    d.xb = *reinterpret_cast<const uint4*>(X + xrow_b + k0);
    if constexpr (NCB > 0) {
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        d.lb[c][0] = *reinterpret_cast<const uint4*>(lora_down + (size_t)(c * 16 + r8) * K + k0);
        d.lb[c][1] = *reinterpret_cast<const uint4*>(lora_down + (size_t)(c * 16 + 8 + r8) * K + k0);
      }
    }
  };

  // Through this wave's scratch, [block][16 rows][8 chunks of 16 bytes] with the
  // chunk slot XOR-ed with the row (conflict-free 16-byte accesses both ways),
  // into the MFMA operand layout: lane l then holds row (rank) l % 16 and chunks
  // q4 and 4 + q4, i.e. channels 8 q4 .. +8 and 32 + 8 q4 .. +8 of the step.
  // Block 0 takes X, block 1 the rank blocks in turn. One wave's LDS accesses
  // complete in order; the fences only keep the compiler from moving them
  // across each other.
  auto wave_fence = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto relayout = [&](Step& d) {
    const int r16 = lane & 15;
    auto put = [&](int blk, int rr, const uint4& v) { scr[blk * 128 + rr * 8 + (c8 ^ (rr & 7))] = v; };
    auto get = [&](int blk, int h) { return scr[blk * 128 + r16 * 8 + ((4 * h + q4) ^ (r16 & 7))]; };
    wave_fence();   // the previous step's reads are done
    put(0, r8, d.xa);
    put(0, 8 + r8, d.xb);
    put(1, r8, d.lb[0][0]);
    put(1, 8 + r8, d.lb[0][1]);
    wave_fence();
    d.xa = get(0, 0);
    d.xb = get(0, 1);
    d.lb[0][0] = get(1, 0);
    d.lb[0][1] = get(1, 1);
#pragma unroll
    for (int c = 1; c < NCB; ++c) {   // the next rank block through the same slot
      wave_fence();
      put(1, r8, d.lb[c][0]);
      put(1, 8 + r8, d.lb[c][1]);
      wave_fence();
      d.lb[c][0] = get(1, 0);
      d.lb[c][1] = get(1, 1);
    }
  };

  // INT4 codes of 8 values against scale sf (nonzero), rs = rcp(sf); raises
  // tmax to the largest |v * rs - q|, which tells whether a value may round
  // differently from the IEEE quotient (tmax > 0.5 - 2^-16, tested once per
  // group: cheaper than a flag per value).
  // y = v * rs is formed exactly inside fma(v, rs, 1.5 * 2^23), which rounds it
  // to an integer (ties to even) in the low mantissa bits; the clamp to +-7 is
  // a med3 in that domain, and fma(v, rs, -q) is y - q with one rounding. The
  // low byte of the clamped value is q as a two's-complement int8, and byte
  // permutes gather the eight low nibbles (even k in the low nibble).
  auto int4_codes = [&](const float* v, float rs, float& tmax) {
    constexpr float kM = 12582912.0f;   // 1.5 * 2^23
    uint32_t b[8];
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float yv = __builtin_amdgcn_fmed3f(fmaf(v[i], rs, kM), kM - 7.0f, kM + 7.0f);
      t[i] = fmaf(v[i], rs, -(yv - kM));
      b[i] = __float_as_uint(yv);
    }
#pragma unroll
    for (int i = 0; i < 8; i += 2)
      tmax = __builtin_fmaxf(tmax, __builtin_fmaxf(fabsf(t[i]), fabsf(t[i + 1])));
    const uint32_t e = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[6], b[4], 0x0c0c0400u),
                                             __builtin_amdgcn_perm(b[2], b[0], 0x0c0c0400u), 0x05040100u);
    const uint32_t o = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[7], b[5], 0x0c0c0400u),
                                             __builtin_amdgcn_perm(b[3], b[1], 0x0c0c0400u), 0x05040100u);
    return (e & 0x0F0F0F0Fu) | ((o << 4) & 0xF0F0F0F0u);
  };
  auto int4_codes_exact = [&](const float* v, float sf) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float q = rintf(v[i] / sf);                           // IEEE division, ties to even
      q = fminf(fmaxf(q, -7.0f), 7.0f);
      w |= ((uint32_t)((int)q) & 0xFu) << (4 * i);
    }
    return w;
  };
  // FP4 E2M1 block: scale byte and the codes of this lane's 8 values
  auto fp4_block = [&](const float* v, float amax, uint32_t& w) {
    uint32_t sc = 0;
    w = 0;
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
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0] * p, v[1] * p, 1.0f, 0);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2] * p, v[3] * p, 1.0f, 1);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4] * p, v[5] * p, 1.0f, 2);
      w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6] * p, v[7] * p, 1.0f, 3);
    }
    return sc;
  };

  // process step s into round buffer rb (its column is this wave's index)
  auto process = [&](const Step& dl, int s, uint8_t* rb) {
    Step d = dl;
    if constexpr (kLines) relayout(d);
    const int k0 = (sbeg + s) * 64 + q4 * 8;
    if constexpr (NCB > 0) {
#pragma unroll
      for (int c = 0; c < NCB; ++c) {
        lacc[c] = Io<IO>::mma16x16x32(d.xa, d.lb[c][0], lacc[c]);
        lacc[c] = Io<IO>::mma16x16x32(d.xb, d.lb[c][1], lacc[c]);
      }
    }
    if constexpr (LORA_ONLY) return;
    // smoothing: x_hat = fl32(fp32(x) * smooth_inv), a plain IEEE multiply.
    // xh[0..7]: channels k0 .. k0+7, xh[8..15]: channels k0+32 .. k0+39.
    float xh[16];
    {
      float sv[16];
      const float* ps = SLDS ? s_si : smooth_inv;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4 u0 = *reinterpret_cast<const float4*>(ps + k0 + 32 * h);
        const float4 u1 = *reinterpret_cast<const float4*>(ps + k0 + 32 * h + 4);
        sv[8 * h + 0] = u0.x; sv[8 * h + 1] = u0.y; sv[8 * h + 2] = u0.z; sv[8 * h + 3] = u0.w;
        sv[8 * h + 4] = u1.x; sv[8 * h + 5] = u1.y; sv[8 * h + 6] = u1.z; sv[8 * h + 7] = u1.w;
      }
      // one fma with a -0 addend: the product rounded once, sign of zero kept.
      // The -0 sits in a register, so that with fp16 input each product is one
      // v_fma_mix_f32 reading the 16-bit half in place (no separate convert;
      // an fp32 literal cannot be an operand of that instruction).
      const uint16_t* ha = reinterpret_cast<const uint16_t*>(&d.xa);
      const uint16_t* hb = reinterpret_cast<const uint16_t*>(&d.xb);
      float nz = -0.0f;
      asm volatile("" : "+s"(nz));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xh[i] = fmaf(Io<IO>::to_f(ha[i]), sv[i], nz);
        xh[8 + i] = fmaf(Io<IO>::to_f(hb[i]), sv[8 + i], nz);
      }
    }
    uint8_t* crow = rb + (lane & 15) * CROW + wave * 32 + q4 * 4;
    uint8_t* srow = rb + 16 * CROW + (lane & 15) * SROW + wave * SB;
    if constexpr (FMT == 0) {
      // INT4, group 64 = this step: reduce over the four lanes of the row.
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(xh[i]));
      amax = lane_max_xor16(amax);
      amax = lane_max_xor32(amax);
      const float s32 = div7_rn(amax);                  // = fl32(amax / 7)
      const __half s16 = __float2half_rn(fminf(s32, 65504.0f));
      const float sf = __half2float(s16);
      uint32_t w0 = 0, w1 = 0;
      if (sf != 0.0f) {
        // q = clamp(rint(fl32(x_hat / s)), -7, 7) without a division per value:
        // y = x_hat * rcp(s) is within 2^-19 |y| of fl32(x_hat / s) (rcp is within
        // an ulp), so the two round to the same integer unless y lies within
        // 2^-16 of a half-integer; only such groups are recomputed with the IEEE
        // division. Clamping the rounded value equals rounding the clamped one,
        // and a value beyond +-7.5 (possible only with a saturated scale) is
        // flagged and recomputed.
        const float rs = __builtin_amdgcn_rcpf(sf);
        float tmax = 0.0f;
        w0 = int4_codes(xh, rs, tmax);
        w1 = int4_codes(xh + 8, rs, tmax);
        if (tmax > 0.4999847412109375f) {   // 0.5 - 2^-16
          w0 = int4_codes_exact(xh, sf);
          w1 = int4_codes_exact(xh + 8, sf);
        }
      }
      *reinterpret_cast<uint32_t*>(crow) = w0;
      *reinterpret_cast<uint32_t*>(crow + 16) = w1;
      if (q4 == 0) *reinterpret_cast<__half*>(srow) = s16;
    } else if constexpr (FMT == 2) {
      // NVFP4, block 16 = a quarter step: xh[0..7] and lane l ^ 16's xh[0..7]
      // form block 4s + q4 / 2, xh[8..15] likewise block 4s + 2 + q4 / 2.
      // s = E4M3(fl32(amax / fl32(6 g))), divisor d = fl32(E4M3(s) g), codes
      // E2M1(fl32(x_hat / d)) with the IEEE division; the convert (scale 1)
      // rounds to nearest, ties to even, saturates at 6 and keeps the sign.
      float am0 = 0.f, am1 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        am0 = fmaxf(am0, fabsf(xh[i]));
        am1 = fmaxf(am1, fabsf(xh[8 + i]));
      }
      am0 = lane_max_xor16(am0);
      am1 = lane_max_xor16(am1);
      uint32_t w[2], sc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float* v = xh + 8 * h;
        sc[h] = e4m3_rne_byte((h ? am1 : am0) / gs6);
        const float d = e4m3_to_f32(sc[h]) * gs;
        w[h] = 0;
        if (d != 0.0f) {
          // u = fl32(x_hat / d) without a division per value: y = x_hat * rcp(d)
          // (rcp within 1 ulp, one rounding of the product) is within 3.5 ulp of
          // u, so the two convert to the same E2M1 code unless a rounding
          // boundary of E2M1 (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; ties to even)
          // lies between them or on one. Every boundary has its low 21 mantissa
          // bits zero, so y is then within 8 units of 0 mod 2^21 in its low bits
          // (below a power-of-two boundary the mantissa is near all ones): such
          // blocks, and divisors near either end of the fp32 range (whose
          // reciprocal would leave the normal range), take the IEEE division.
          float u[8];
          bool exact = !(d >= 0x1p-125f && d <= 0x1p125f);
          if (!exact) {
            const float rd = __builtin_amdgcn_rcpf(d);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              u[i] = v[i] * rd;
              exact |= ((__float_as_uint(u[i]) + 8u) & 0x1FFFFFu) <= 16u;
            }
          }
          if (exact) {
#pragma unroll
            for (int i = 0; i < 8; ++i) u[i] = v[i] / d;
          }
          w[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[h], u[0], u[1], 1.0f, 0);
          w[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[h], u[2], u[3], 1.0f, 1);
          w[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[h], u[4], u[5], 1.0f, 2);
          w[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[h], u[6], u[7], 1.0f, 3);
        }
      }
      *reinterpret_cast<uint32_t*>(crow) = w[0];
      *reinterpret_cast<uint32_t*>(crow + 16) = w[1];
      // scale bytes of the step: [block 0, 1, 2, 3] = lanes q4 0 / 2 (xh[0..7]) and (xh[8..15])
      if ((q4 & 1) == 0) {
        srow[q4 >> 1] = (uint8_t)sc[0];
        srow[2 + (q4 >> 1)] = (uint8_t)sc[1];
      }
    } else {
      // FP4 E2M1, block 32 = half a step: xh[0..7] belong to block 2s, xh[8..15]
      // to block 2s + 1; each block is reduced over the four lanes of the row.
      float am0 = 0.f, am1 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        am0 = fmaxf(am0, fabsf(xh[i]));
        am1 = fmaxf(am1, fabsf(xh[8 + i]));
      }
      am0 = lane_max_xor32(lane_max_xor16(am0));
      am1 = lane_max_xor32(lane_max_xor16(am1));
      uint32_t w0, w1;
      const uint32_t sc0 = fp4_block(xh, am0, w0);
      const uint32_t sc1 = fp4_block(xh + 8, am1, w1);
      *reinterpret_cast<uint32_t*>(crow) = w0;
      *reinterpret_cast<uint32_t*>(crow + 16) = w1;
      if (q4 == 0) *reinterpret_cast<uint16_t*>(srow) = (uint16_t)(sc0 | (sc1 << 8));
    }
  };

  // The waves advance in rounds: in round p wave w processes step p W + w and
  // leaves its codes and scales in the round buffer; after a barrier the
  // workgroup writes the round out as whole 16-byte pieces of each row (codes:
  // 32 W contiguous bytes per row, scales: 2 W), so each store instruction
  // covers full lines instead of one 16-byte piece per row and step. The
  // barriers wait for LDS only, so the loads of later rounds stay in flight.
  const int nrounds = (steps + WAVES - 1) / WAVES;
  auto round = [&](const Step& d, int p) {
    uint8_t* rb = rbuf + (p & 1) * RBUF;
    const int s = p * WAVES + wave;
    if (s < steps) process(d, s, rb);
    if constexpr (LORA_ONLY) return;   // nothing to write out, no round barrier
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_s_barrier();
    const int vs = min(WAVES, steps - p * WAVES);   // steps in this round
    for (int c = threadIdx.x; c < 16 * 2 * WAVES; c += 64 * WAVES) {
      const int rl = c / (2 * WAVES), ch = c - rl * (2 * WAVES);
      if (ch < 2 * vs && m0 + rl < M)
        *reinterpret_cast<uint4*>(codes + (size_t)(m0 + rl) * (K >> 1) + (size_t)(sbeg + p * WAVES) * 32 + ch * 16) =
            *reinterpret_cast<const uint4*>(rb + rl * CROW + ch * 16);
    }
    for (int c = threadIdx.x; c < 16 * WAVES; c += 64 * WAVES) {
      const int rl = c / WAVES, j = c - rl * WAVES;
      if (j < vs && m0 + rl < M) {
        // a row holds SB scale bytes per 64-channel step
        uint8_t* dst = reinterpret_cast<uint8_t*>(scales) + (size_t)(m0 + rl) * (size_t)((K >> 6) * SB) +
                       (size_t)(sbeg + p * WAVES + j) * SB;
        if constexpr (SB == 4)
          *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(rb + 16 * CROW + rl * SROW + j * 4);
        else
          *reinterpret_cast<uint16_t*>(dst) = *reinterpret_cast<const uint16_t*>(rb + 16 * CROW + rl * SROW + j * 2);
      }
    }
    // the buffer is rewritten two rounds later, after the next round's barrier,
    // by which time every wave has finished reading it here
  };

  // D register sets in flight: three where the register budget allows
  // (64 * WAVES threads leave 512 / (WAVES / 4) VGPRs per lane), else two.
  constexpr int D = (WAVES == 4) ? 3 : (WAVES == 8) ? (NCB <= 3 ? 3 : 2) : (NCB == 0 ? 3 : 2);
  if constexpr (D == 3) {
    Step d0, d1, d2;
    load(d0, wave);
    load(d1, wave + WAVES);
    stage_si();
    lora_from_partials();
    for (int p = 0; p < nrounds; p += 3) {
      load(d2, (p + 2) * WAVES + wave);
      round(d0, p);
      if (p + 1 >= nrounds) break;
      load(d0, (p + 3) * WAVES + wave);
      round(d1, p + 1);
      if (p + 2 >= nrounds) break;
      load(d1, (p + 4) * WAVES + wave);
      round(d2, p + 2);
    }
  } else {
    Step d0, d1;
    load(d0, wave);
    stage_si();
    lora_from_partials();
    for (int p = 0; p < nrounds; p += 2) {
      load(d1, (p + 1) * WAVES + wave);
      round(d0, p);
      if (p + 1 >= nrounds) break;
      load(d0, (p + 2) * WAVES + wave);
      round(d1, p + 1);
    }
  }

  if constexpr (NCB > 0) {
    __syncthreads();   // every wave is done with its scratch, which the partials reuse
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
      for (int w = 0; w < WAVES; ++w) sum += red[(w * 16 + rr) * R + cc];
      if (m0 + rr < M) {
        if (gridDim.y > 1)   // the slice's partial, at the row's tail in codes
          reinterpret_cast<float*>(codes + (size_t)(m0 + rr) * (K >> 1) + (K >> 1) -
                                   (size_t)gridDim.y * R * 4)[blockIdx.y * R + cc] = sum;
        else
          lora_act[(size_t)(m0 + rr) * R + cc] = sum;
      }
    }
  }
}

template <int IO, int FMT, int NCB, int WAVES, bool SLDS, bool LO>
static hipError_t launch_qws(int M, int K, int slices, const void* X, const float* si, const void* ld,
                             uint8_t* codes, void* scales, void* la, float gs, hipStream_t st, int rq) {
  const dim3 grid((M + 15) / 16, slices), block(64 * WAVES);
  const size_t lds = quant_lds_bytes<WAVES>(NCB) + (SLDS ? (size_t)K * sizeof(float) : 0);
  if (lds > 65536) {
    // raised once per instantiation and device to the largest size it may need
    static std::atomic<uint64_t> raised{0};
    const hipError_t e = raise_lds_limit(
        raised, reinterpret_cast<const void*>(&quantize_act_kernel<IO, FMT, NCB, WAVES, SLDS, LO>), kQuantLdsMax);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((quantize_act_kernel<IO, FMT, NCB, WAVES, SLDS, LO>), grid, block, lds, st,
                     (const uint16_t*)X, si, (const uint16_t*)ld, codes, scales, (float*)la, M, K, gs,
                     6.0f * gs, rq);
  return hipGetLastError();
}

// smooth_inv goes to LDS when it fits beside the low-rank partials (the
// low-rank-only pass does not read it)
template <int IO, int FMT, int NCB, int WAVES, bool LO>
static hipError_t launch_qw(int M, int K, int slices, const void* X, const float* si, const void* ld,
                            uint8_t* codes, void* scales, void* la, float gs, hipStream_t st, int rq) {
  if constexpr (!LO) {
    if (quant_lds_bytes<WAVES>(NCB) + (size_t)K * sizeof(float) <= (size_t)kQuantLdsMax)
      return launch_qws<IO, FMT, NCB, WAVES, true, LO>(M, K, slices, X, si, ld, codes, scales, la, gs, st, rq);
  }
  return launch_qws<IO, FMT, NCB, WAVES, false, LO>(M, K, slices, X, si, ld, codes, scales, la, gs, st, rq);
}

// 16 rows per workgroup. For ranks up to 32, 16 waves (4 per SIMD): more waves
// keep more loads in flight per CU and measured faster than 8 at every M (e.g.
// 17.2 -> 15.3 us at M4096 K3072, 51.2 -> 46.6 us at M4096 K12288); for ranks
// 48 to 96, 8 waves (the ring's lora_down operands need the registers); for
// ranks of 112 and more, 4 waves (the lora_down operands of a step take
// 8 * r / 16 VGPRs per set).
template <int IO, int FMT, int NCB, bool LO>
static hipError_t launch_q(int M, int K, int slices, const void* X, const float* si, const void* ld,
                           uint8_t* codes, void* scales, void* la, float gs, hipStream_t st, int rq = 0) {
  if constexpr (NCB >= 7) {
    return launch_qw<IO, FMT, NCB, 4, LO>(M, K, slices, X, si, ld, codes, scales, la, gs, st, rq);
  } else if constexpr (NCB > 2) {
    return launch_qw<IO, FMT, NCB, 8, LO>(M, K, slices, X, si, ld, codes, scales, la, gs, st, rq);
  } else {
    return launch_qw<IO, FMT, NCB, 16, LO>(M, K, slices, X, si, ld, codes, scales, la, gs, st, rq);
  }
}

// the low-rank down-projection alone: over all of K into lora_act (S = 1, the
// fused kernel's summation order), or per K slice into the tails of the code
// rows (S > 1)
template <int IO>
static hipError_t launch_lora_only(int M, int K, int r, int S, const void* X, const void* ld, uint8_t* codes,
                                   void* la, hipStream_t st) {
  switch (r / 16) {
    case 1: return launch_q<IO, 0, 1, true>(M, K, S, X, nullptr, ld, codes, nullptr, la, 1.0f, st);
    case 2: return launch_q<IO, 0, 2, true>(M, K, S, X, nullptr, ld, codes, nullptr, la, 1.0f, st);
    case 3: return launch_q<IO, 0, 3, true>(M, K, S, X, nullptr, ld, codes, nullptr, la, 1.0f, st);
    case 4: return launch_q<IO, 0, 4, true>(M, K, S, X, nullptr, ld, codes, nullptr, la, 1.0f, st);
    case 5: return launch_q<IO, 0, 5, true>(M, K, S, X, nullptr, ld, codes, nullptr, la, 1.0f, st);
    case 6: return launch_q<IO, 0, 6, true>(M, K, S, X, nullptr, ld, codes, nullptr, la, 1.0f, st);
    case 7: return launch_q<IO, 0, 7, true>(M, K, S, X, nullptr, ld, codes, nullptr, la, 1.0f, st);
    default: return launch_q<IO, 0, 8, true>(M, K, S, X, nullptr, ld, codes, nullptr, la, 1.0f, st);
  }
}

template <int IO, int FMT>
static hipError_t launch_q_r(int M, int K, int r, const void* X, const float* si, const void* ld,
                             uint8_t* codes, void* scales, void* la, float gs, hipStream_t st) {
  // A workgroup walks all of K for its 16 rows, so with few row blocks most CUs
  // would idle. Then K is cut into S slices of whole steps, S doubling while the
  // row blocks fill fewer than 256 workgroups and each slice keeps at least 8
  // steps (32 with a low-rank pass): a first launch leaves each slice's low-rank partial sums in the
  // tails of the code rows, a second quantizes the slices (codes and scales are
  // independent per group), its last-slice workgroups summing the partials into
  // lora_act before their codes overwrite them. S stays below the point where
  // the partials (S r 4 bytes per row) would not fit in the last slice's codes.
  const int nb = (M + 15) / 16, steps = K >> 6;
  int S = 1;
  while (nb * S < 256 && S < 8 && steps >= 16 * S) {
    const int S2 = 2 * S, last = steps - (S2 - 1) * ((steps + S2 - 1) / S2);
    // with a low-rank pass, slices of fewer than 32 steps lose to the fused
    // kernel (two short launches: M1024 K3072 r32 13 -> 18 us, K12288 43 -> 26 us)
    if (r > 0 && (steps < 32 * S2 || S2 * r * 4 > last * 32)) break;
    S = S2;
  }
  if (S > 1) {
    if (r > 0) {
      const hipError_t e = launch_lora_only<IO>(M, K, r, S, X, ld, codes, nullptr, st);
      if (e != hipSuccess) return e;
    }
    return launch_q<IO, FMT, 0, false>(M, K, S, X, si, ld, codes, scales, la, gs, st, r);
  }
  switch (r / 16) {
    case 0: return launch_q<IO, FMT, 0, false>(M, K, 1, X, si, ld, codes, scales, la, gs, st);
    case 1: return launch_q<IO, FMT, 1, false>(M, K, 1, X, si, ld, codes, scales, la, gs, st);
    case 2: return launch_q<IO, FMT, 2, false>(M, K, 1, X, si, ld, codes, scales, la, gs, st);
    case 3: return launch_q<IO, FMT, 3, false>(M, K, 1, X, si, ld, codes, scales, la, gs, st);
    case 4: return launch_q<IO, FMT, 4, false>(M, K, 1, X, si, ld, codes, scales, la, gs, st);
    case 5: return launch_q<IO, FMT, 5, false>(M, K, 1, X, si, ld, codes, scales, la, gs, st);
    case 6: return launch_q<IO, FMT, 6, false>(M, K, 1, X, si, ld, codes, scales, la, gs, st);
    case 7: return launch_q<IO, FMT, 7, false>(M, K, 1, X, si, ld, codes, scales, la, gs, st);
    default: return launch_q<IO, FMT, 8, false>(M, K, 1, X, si, ld, codes, scales, la, gs, st);
  }
}

template <int IO>
static hipError_t launch_q_io(int fmt, int M, int K, int r, const void* X, const float* si,
                              const void* ld, uint8_t* codes, void* scales, void* la,
                              hipStream_t st, float gscale) {
  if (fmt == 0) return launch_q_r<IO, 0>(M, K, r, X, si, ld, codes, scales, la, 1.0f, st);
  if (fmt == 2) return launch_q_r<IO, 2>(M, K, r, X, si, ld, codes, scales, la, gscale, st);
  return launch_q_r<IO, 1>(M, K, r, X, si, ld, codes, scales, la, 1.0f, st);
}

hipError_t launch_quantize_act(int fmt, int io, int M, int K, int r, const void* X, const float* si,
                               const void* ld, uint8_t* codes, void* scales, void* la,
                               hipStream_t st, float gscale) {
  if (io == 1) return launch_q_io<1>(fmt, M, K, r, X, si, ld, codes, scales, la, st, gscale);
  return launch_q_io<0>(fmt, M, K, r, X, si, ld, codes, scales, la, st, gscale);
}

}  // namespace svdq
