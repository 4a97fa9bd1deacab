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
// operand reuse: 256 x 256 per workgroup, one workgroup per CU, 8 waves of
// 128 x 64 (4 x 2 blocks of 32 x 32, 128 fp32 accumulators per lane held in
// AGPRs), two per SIMD, so that one wave's LDS reads, DMA issue and barrier
// waits overlap the other's MFMAs. Operands reach LDS by LDS-DMA in units that
// keep the memory pipeline's request count low (each request costs about as
// much as the bytes it moves):
//  - codes in stage pairs of 256 codes: whole 128-byte row lines, 8 rows per
//    instruction, two 64 KB pair slots (the pair in use and the next one);
//  - scales in groups of 4 steps: 16 bytes per row, two 8 KB group slots.
// The 8 MFMAs of each half-step (64 codes) run while the next half-step's
// operands are read from LDS; the DMA of the pair after next is threaded
// between the MFMAs of the last half-step of a pair, after the one barrier per
// pair. The low-rank up-projection is added after the main loop, so its global
// loads never wait behind the DMA. Built with MFMA results in AGPRs (no
// VGPR-form flag): the accumulators are only touched by MFMAs until the epilogue.
#include <atomic>
#include <type_traits>

#include "chain.hpp"
#include "common.hpp"
#include "launch.hpp"
#include "pipeline.hpp"

namespace svdq {

namespace fp4big {
constexpr int BM = 256, BN = 256;
constexpr int RB = 4;                         // 32-row blocks per wave
constexpr int ROW = 128;                      // bytes of a code row per stage pair
constexpr int PAIR = (BM + BN) * ROW;         // 64 KB: one pair of A rows and B rows
// The ring holds A slot 0, A slot 1, B slot 0, B slot 1 (32 KB each), so that
// the slot and the 32-row block of an operand read are immediate offsets
// (under 64 KB) from one lane address per half-step.
constexpr int SLOT = BM * ROW;                // 32 KB
constexpr int BOFF = 2 * SLOT;                // B slots after both A slots
constexpr int SROW = 16;                      // bytes of a scale row per group of 4 steps
constexpr int SGRP = (BM + BN) * SROW;        // 8 KB group slot
constexpr int LDS = 2 * PAIR + 2 * SGRP;      // 144 KB
// 8 waves in a 2 x 4 grid, each 128 rows x 64 columns (two per SIMD)
constexpr int NW = 8, NT = 64 * NW;
constexpr int CB = 2;                         // 32-column blocks per wave
constexpr int WNC = 32 * CB;                  // columns per wave
constexpr int CI = PAIR / (1024 * NW);        // code DMA instructions per wave and pair
constexpr int SI = SGRP / (1024 * NW);        // scale DMA instructions per wave and group
static_assert((NW / 2) * WNC == BN && 2 * 128 == BM, "the wave grid covers the tile");
static_assert(CI == RB * CB, "one code DMA per MFMA of the last half-step");
static_assert(SI == 1, "one scale DMA per wave and group");
static_assert(BM == BN && SLOT == BN * ROW, "A and B slots of one size");
}  // namespace fp4big

// The eight 16-byte chunks of a 128-byte code row are XOR-swizzled with
// (row >> 1) & 7, so the 16 rows that one ds_read_b128 serves per pass (same
// logical chunk) land in 16 distinct 16-byte bank slots.
__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }

template <int IO, int EPI>
__global__ __launch_bounds__(fp4big::NT, 1)
void gemm_fp4_big_kernel(const uint8_t* __restrict__ act_codes, const uint8_t* __restrict__ act_scales,
                         const float* __restrict__ lora_act, const uint8_t* __restrict__ w_codes,
                         const uint8_t* __restrict__ w_scales, const uint16_t* __restrict__ lora_up,
                         const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y,
                         int M, int N, int K, int r, ChainEpilogue ce) {
  using namespace fp4big;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / (NW / 2), wn = wave % (NW / 2);
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
  const int nk = K >> 7;          // steps of 128 codes, a multiple of 4
  const int np = nk >> 1;         // stage pairs
  const int ng = nk >> 2;         // scale groups
  const int KB = K >> 1;
  const int SK = K >> 5;          // scale bytes per row

  // ---- DMA plan. Code instruction j (0..CI-1) of wave w fills slot rows
  // 8 NW j + 8 w .. +8 (the first CI/2: A, the rest: B); lane L takes row + L/8
  // and chunk L%8. Scale instruction j of wave w fills slot rows 64 (NW j + w)
  // + L (A rows below 256, then B).
  const uint8_t* tA = act_codes + (size_t)m0 * KB;
  const uint8_t* tB = w_codes + (size_t)n0 * KB;
  const uint8_t* tsA = act_scales + (size_t)m0 * SK;
  const uint8_t* tsB = w_scales + (size_t)n0 * SK;
  const int alast = M - 1 - m0;                 // rows past M re-read the last row
  const int rl = 8 * wave + (lane >> 3);
  const int coff = ((lane & 7) ^ swz8(rl)) * 16;  // swz8(8 NW j + rl) == swz8(rl)
  constexpr int CH = CI / 2;
  uint32_t aoff[CH], boff[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    aoff[j] = (uint32_t)min(8 * NW * j + rl, alast) * (uint32_t)KB + (uint32_t)coff;
    boff[j] = (uint32_t)(8 * NW * j + rl) * (uint32_t)KB + (uint32_t)coff;
  }
  uint32_t soff[SI];
#pragma unroll
  for (int j = 0; j < SI; ++j) {
    const int sr = 64 * (NW * j + wave) + lane;   // slot row
    soff[j] = (uint32_t)(sr < BM ? min(sr, alast) : sr - BM) * (uint32_t)SK;
  }
  const uint8_t* tsW = 64 * wave < BM ? tsA : tsB;   // the half this wave's scale rows lie in
  const uint32_t lds0 = lds_addr(smem);

  auto code_dma = [&](int pp, int j) {   // pair pp, instruction j (constant)
    const uint32_t lds = lds0 + (uint32_t)((j < CH ? 0 : BOFF) + (pp & 1) * SLOT +
                                           (8 * NW * (j % CH) + 8 * wave) * ROW);
    if (j < CH) dma16_so(tA, aoff[j] + (uint32_t)(pp * ROW), lds);
    else dma16_so(tB, boff[j - CH] + (uint32_t)(pp * ROW), lds);
  };
  auto scale_dma = [&](int q, int j) {   // scale group q, instruction j (constant)
    const uint32_t lds = lds0 + (uint32_t)(2 * PAIR + (q & 1) * SGRP + 64 * (NW * j + wave) * SROW);
    dma16_so(tsW, soff[j] + (uint32_t)(q * SROW), lds);
  };

  // With two waves per SIMD a lane may use at most 256 registers, and the
  // compiler then selects MFMAs with VGPR results unless the function is seen
  // to use AGPRs; an empty asm statement with an AGPR operand keeps the 128
  // accumulators in AGPRs (VGPR results spill).
  asm volatile("" ::"a"(0));
  v16f acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  int arow[RB], brow[CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) arow[rb] = wm * 128 + rb * 32 + l32;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) brow[cb] = wn * WNC + cb * 32 + l32;
  const int s8 = swz8(l32);   // == swz8(arow[rb]) == swz8(brow[cb])

  // operands of half-step hs (0..3) of pair pp: step 2 pp + hs / 2, K half hs % 2
  struct Ops { uint4 a[RB], b[CB]; };
  // lane addresses of half-step hs: row block 0 of A and of B in slot 0
  uint32_t la[4], lb[4];
#pragma unroll
  for (int hs = 0; hs < 4; ++hs) {
    const int ch = ((2 * hs + lh) ^ s8) << 4;
    la[hs] = (uint32_t)(arow[0] * ROW + ch);
    lb[hs] = (uint32_t)(BOFF + brow[0] * ROW + ch);
  }
  auto load_ops = [&](Ops& o, int pp, int hs) {
    const uint8_t* pa = smem + la[hs] + (pp & 1) * SLOT;
    const uint8_t* pb = smem + lb[hs] + (pp & 1) * SLOT;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) o.a[rb] = *reinterpret_cast<const uint4*>(pa + rb * 32 * ROW);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) o.b[cb] = *reinterpret_cast<const uint4*>(pb + cb * 32 * ROW);
  };
  struct Sc { uint32_t a[RB], b[CB]; };
  auto load_sc = [&](Sc& e, int ks) {   // the 4 E8M0 bytes of step ks for this lane's rows
    const uint8_t* sS = smem + 2 * PAIR + ((ks >> 2) & 1) * SGRP + (ks & 3) * 4;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) e.a[rb] = *reinterpret_cast<const uint32_t*>(sS + arow[rb] * SROW);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      e.b[cb] = *reinterpret_cast<const uint32_t*>(sS + (BM + brow[cb]) * SROW);
  };
  // lane l < 32 holds K block 0 of the half-step, lane l + 32 block 1
  auto mfma = [&](const Ops& o, const Sc& e, int g, int rb, int cb) {
    const int sh = 8 * (2 * g + lh);
    const v8i av = v8i{(int)o.a[rb].x, (int)o.a[rb].y, (int)o.a[rb].z, (int)o.a[rb].w, 0, 0, 0, 0};
    const v8i bv = v8i{(int)o.b[cb].x, (int)o.b[cb].y, (int)o.b[cb].z, (int)o.b[cb].w, 0, 0, 0, 0};
    acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        av, bv, acc[rb][cb], 4, 4, 0, (int)((e.a[rb] >> sh) & 0xFFu), 0, (int)((e.b[cb] >> sh) & 0xFFu));
  };
  auto mma = [&](const Ops& o, const Sc& e, int g) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) mfma(o, e, g, rb, cb);
  };
  // the same 8 MFMAs with the DMA of pair dp (and scale group dq) threaded
  // between them, one DMA instruction after each MFMA (issuing all DMA first,
  // or raising the wave priority around the MFMAs, measured no faster)
  auto mma_dma = [&](const Ops& o, const Sc& e, int g, int dp, int dq, auto with_scales) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        mfma(o, e, g, rb, cb);
        const int i = rb * CB + cb;
        code_dma(dp, i);
        if constexpr (decltype(with_scales)::value) {
          if (i < SI) scale_dma(dq, i);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  };

  Ops P0, P1;
  Sc E0, E1;
  using T_ = std::true_type;
  using F_ = std::false_type;
  // one stage pair. On entry P0 holds its half-step 0 and E0 the scales of its
  // first step. MORE: a pair follows (published at the end of this one); DMA:
  // the pair after that (and, for SDMA, the next scale group) is loaded now.
  // All three are compile-time, so the body is straight-line code.
  // Scheduling fences keep the reads of a half-step from being hoisted above
  // the MFMAs before it (which needs more than the 256 registers of a lane).
  auto fence = [&]() { __builtin_amdgcn_sched_barrier(0); };
  auto pair = [&](int pp, auto more, auto dma, auto sdma) {
    load_ops(P1, pp, 1);
    fence();
    mma(P0, E0, 0);
    fence();
    load_ops(P0, pp, 2);
    load_sc(E1, 2 * pp + 1);
    fence();
    mma(P1, E0, 1);
    fence();
    load_ops(P1, pp, 3);
    fence();
    mma(P0, E1, 0);
    fence();
    if constexpr (decltype(more)::value) {
      // every LDS read of this pair has completed, and so has the DMA of the next
      // pair and scale group; past the barrier no wave reads this pair's slot (nor
      // the previous scale group's), which the DMA reuses
      waitvm_lgkm0<0>();
      __syncthreads();
      load_ops(P0, pp + 1, 0);
      load_sc(E0, 2 * pp + 2);
    }
    fence();
    if constexpr (decltype(dma)::value) mma_dma(P1, E1, 1, pp + 2, (pp >> 1) + 1, sdma);
    else mma(P1, E1, 1);
    fence();
  };

  // prologue: pair 0, scale group 0, pair 1 (nk >= 4, so np >= 2)
#pragma unroll
  for (int j = 0; j < CI; ++j) code_dma(0, j);
#pragma unroll
  for (int j = 0; j < SI; ++j) scale_dma(0, j);
#pragma unroll
  for (int j = 0; j < CI; ++j) code_dma(1, j);
  waitvm<CI>();   // pair 0 and scale group 0 have landed
  __syncthreads();
  load_ops(P0, 0, 0);
  load_sc(E0, 0);
  int q = 0;
  for (; q + 1 < ng; ++q) {
    pair(2 * q, T_{}, T_{}, T_{});       // loads pair 2q + 2 and scale group q + 1
    pair(2 * q + 1, T_{}, T_{}, F_{});   // loads pair 2q + 3
  }
  pair(2 * q, T_{}, F_{}, F_{});

  // ---- low-rank up-projection: lora_act (fp32, as a hi + lo pair of 16-bit
  // operands) times lora_up into the same accumulators, v_mfma_f32_32x32x16_f16
  // (lane l: row l%32, ranks j0 + 8 (l/32) .. +8). The loads go out before the
  // last pair's MFMAs.
  constexpr int LR = 1;   // 16-rank blocks per round trip
  auto lora_load = [&](float4 (&fa)[RB][LR][2], uint4 (&ub)[CB][LR], int j0) {
    const int nj = min(r - j0, 16 * LR) >> 4;
#pragma unroll
    for (int h = 0; h < LR; ++h) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int m = m0 + arow[rb];
        const bool ok = m < M && h < nj;
        const float* src = lora_act + (size_t)min(m, M - 1) * r + j0 + 16 * h + lh * 8;
        fa[rb][h][0] = ok ? *reinterpret_cast<const float4*>(src) : make_float4(0.f, 0.f, 0.f, 0.f);
        fa[rb][h][1] = ok ? *reinterpret_cast<const float4*>(src + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const int n = n0 + brow[cb];
        ub[cb][h] = (h < nj) ? *reinterpret_cast<const uint4*>(lora_up + (size_t)n * r + j0 + 16 * h + lh * 8)
                             : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lora_mma = [&](const float4 (&fa)[RB][LR][2], const uint4 (&ub)[CB][LR]) {
#pragma unroll
    for (int h = 0; h < LR; ++h)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        uint4 hi, lo;
        split8_h16<IO>(fa[rb][h][0], fa[rb][h][1], hi, lo);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          acc[rb][cb] = Io<IO>::mma32x32x16(hi, ub[cb][h], acc[rb][cb]);
          acc[rb][cb] = Io<IO>::mma32x32x16(lo, ub[cb][h], acc[rb][cb]);
        }
      }
  };
  float4 ua[RB][LR][2];
  uint4 ub[CB][LR];
  if (r > 0) lora_load(ua, ub, 0);
  pair(2 * q + 1, F_{}, F_{}, F_{});
  if (r > 0) {
    lora_mma(ua, ub);
    for (int j0 = 16 * LR; j0 < r; j0 += 16 * LR) {
      lora_load(ua, ub, j0);
      lora_mma(ua, ub);
    }
  }

  // ---- epilogue: bias and activation, then the tile goes through LDS (the ring
  // is free now) so that Y is written as whole rows with 16-byte stores; in the
  // fused MLP chain (EPI 3: GELU, then the down-projection's quantizer) the
  // staged tile is quantized and multiplied by lora_down2 there instead.
  constexpr int TP = BN + 8;   // padded row (halves) of the staging tile
  static_assert(BM * TP * 2 + BN * 4 <= LDS, "staging tile (and the chain's smooth_inv) must fit in the ring");
  waitvm<0>();   // no DMA outstanding
  __syncthreads();
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);
  float* si_lds = reinterpret_cast<float*>(smem + BM * TP * 2);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int nl = brow[cb];
    const float bn = bias ? Io<IO>::to_f(bias[n0 + nl]) : 0.f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float yv = acc[rb][cb][v] + bn;
        if (EPI == 1 || EPI == 3) yv = gelu_tanh_f32(yv);
        tile[(wm * 128 + rb * 32 + (v >> 2) * 8 + lh * 4 + (v & 3)) * TP + nl] = Io<IO>::from_f(yv);
      }
  }
  if constexpr (EPI == 3) {
    if (tid < BN / 4)
      *reinterpret_cast<float4*>(si_lds + 4 * tid) = *reinterpret_cast<const float4*>(ce.smooth_inv + n0 + 4 * tid);
  }
  __syncthreads();
  if constexpr (EPI != 3) {
    for (int c = tid; c < BM * (BN / 8); c += NT) {
      const int row = c / (BN / 8), c8 = c - row * (BN / 8);
      if (m0 + row < M)
        *reinterpret_cast<uint4*>(Y + (size_t)(m0 + row) * N + n0 + c8 * 8) =
            *reinterpret_cast<const uint4*>(tile + row * TP + c8 * 8);
    }
  } else {
    chain_quantize_tile<IO, BM, BN, TP, NT>(tile, si_lds, m0, n0, M, N, ce, tid);
    if (ce.r > 0)
      chain_lowrank_partial<IO, BM, BN, TP, NT>(tile, m0, n0, M, N, ce, ce.partial + (size_t)(n0 / BN) * M * ce.r,
                                            wave, lane);
  }
}

bool fp4_big_fits(int M, int N, int K) {
  using namespace fp4big;
  if (N % BN != 0 || K % 512 != 0) return false;                      // whole scale groups
  return ((M + BM - 1) / BM) * (N / BN) >= 256;                       // enough tiles to fill 256 CUs
}

// Large-tile FP4 launch; returns hipErrorNotSupported (without launching) when
// the shape does not suit it, so the caller can fall back to the 128 x 128 kernel.
hipError_t launch_gemm_fp4_big(int io, int M, int N, int K, int r, const uint8_t* ac, const void* as,
                               const void* la, const uint8_t* wc, const void* ws, const void* lu,
                               const void* bias, int epi, void* Y, hipStream_t st, const ChainEpilogue* chain) {
  using namespace fp4big;
  if (!fp4_big_fits(M, N, K)) return hipErrorNotSupported;
  if (epi == 3 && !chain) return hipErrorInvalidValue;
  const int ntiles = ((M + BM - 1) / BM) * (N / BN);
  const int e3 = epi == 3 ? 2 : epi != 0 ? 1 : 0;
  const int v = 3 * (io == 1) + e3;
  using K_t = void (*)(const uint8_t*, const uint8_t*, const float*, const uint8_t*, const uint8_t*,
                       const uint16_t*, const uint16_t*, uint16_t*, int, int, int, int, ChainEpilogue);
  static const K_t kerns[6] = {gemm_fp4_big_kernel<0, 0>, gemm_fp4_big_kernel<0, 1>, gemm_fp4_big_kernel<0, 3>,
                               gemm_fp4_big_kernel<1, 0>, gemm_fp4_big_kernel<1, 1>, gemm_fp4_big_kernel<1, 3>};
  const K_t kern = kerns[v];
  static std::atomic<uint64_t> raised[6] = {};
  const hipError_t e = raise_lds_limit(raised[v], reinterpret_cast<const void*>(kern), LDS);
  if (e != hipSuccess) return e;
  const ChainEpilogue ce = chain ? *chain : ChainEpilogue{nullptr, nullptr, 0, nullptr, nullptr, nullptr};
  hipLaunchKernelGGL(kern, dim3(ntiles), dim3(NT), LDS, st, ac, (const uint8_t*)as, (const float*)la, wc,
                     (const uint8_t*)ws, (const uint16_t*)lu, (const uint16_t*)bias, (uint16_t*)Y, M, N, K, r, ce);
  return hipGetLastError();
}

}  // namespace svdq
