// svdq_gemm_nvfp4: the 4-bit GEMM with the low-rank up-projection, bias and
// GELU fused, for NVFP4 operands: FP4 E2M1 codes with one FP8 E4M3 scale per
// block of 16 along K and one fp32 scale per tensor (the pages' svdq_w4a4
// precision "nvfp4", group size 16: dothoosh.com "How Nunchaku Lite halves
// diffusion-model VRAM", quantization_config block and kernel-family list).
//
// CDNA4's block-scaled matrix instruction takes one power-of-two (E8M0) scale
// per 32 values, so a group-16 E4M3 scale cannot ride on it. Instead both
// operands are dequantized in registers to fp16, where E2M1 x E4M3 is exact
// (at most 6 significant bits, range 2^-10 .. 2688), and multiplied on
// v_mfma_f32_32x32x16_f16, whose K of 16 is one NVFP4 block: each product is
// exact and the sums are fp32, as in the block-scaled path. Dequantization is
// two instructions per two codes: v_cvt_scalef32_pk_f16_fp4 with the exact
// scale 2^8 (E2M1 pair -> fp16 pair x 256; the instruction applies a
// power-of-two scale), then v_pk_mul_f16 by the E4M3 scale read as fp16 bits
// (byte << 7 is the fp16 pattern of the E4M3 value x 2^-8, subnormals
// included; op_sel broadcasts one half of a row's two-block scale word, so
// the pair needs no shuffle of its own). The per-tensor scales are applied
// once, as alpha, to the fp32 sum.
//
// Tiling as in the large FP4 kernel: 256 x BN per workgroup, 4 waves of
// 128 x BN/2 (32 x 32 blocks, fp32 accumulators in AGPRs), one workgroup per
// CU, operands in LDS by LDS-DMA in stage pairs of 256 codes (128-byte rows,
// XOR-swizzled 16-byte chunks) with 16 scale bytes per row and pair. Each
// half-step (64 codes) is 4 K-blocks x RB x CB MFMAs; its LDS reads are issued
// one half-step ahead, and the DMA of pair p + 2 goes out after the barrier
// that ends pair p.
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "pipeline.hpp"

namespace svdq {

namespace nvfp4 {
constexpr int BM = 256;
constexpr int RB = 4;                  // 32-row blocks per wave
constexpr int ROW = 128;               // code bytes of a row per stage pair (256 codes)
constexpr int SROW = 16;               // E4M3 bytes of a row per stage pair
constexpr int SLOT_ROWS = 512;         // rows of a slot (A rows, then B rows, then padding)
constexpr int CODES = SLOT_ROWS * ROW;          // 64 KB
constexpr int SCALES = SLOT_ROWS * SROW;        // 8 KB
constexpr int SLOT = CODES + SCALES;
constexpr int LDS = 2 * SLOT;                   // 144 KB
}  // namespace nvfp4

__device__ __forceinline__ int nv_swz8(int row) { return (row >> 1) & 7; }

// fp16 pair (s_lo, s_lo) and (s_hi, s_hi) from two E4M3 scale bytes (each
// value x 2^-8; the sign bit of a scale byte is ignored: scales are magnitudes)
__device__ __forceinline__ uint32_t nv_scale_pair(uint32_t two) {
  const uint32_t w = __builtin_amdgcn_perm(two, two, 0x0c010c00u);   // [b0, 0, b1, 0]
  return (w << 7) & 0x3F803F80u;                                      // [fp16(b0), fp16(b1)]
}

// 8 E2M1 codes (one dword, even code in the low nibble) times the scale pair
// -> the 8 fp16 values of an MFMA operand, in k order
template <int HI>
__device__ __forceinline__ v8h nv_dequant8(uint32_t w, uint32_t spair) {
  // both halves of the multiplier from one half of the pair (op_sel of v_pk_mul_f16)
  const v2h f = __builtin_bit_cast(v2h, spair);
  const v2h s = __builtin_shufflevector(f, f, HI, HI);
  const v2h h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * s;
  const v2h h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * s;
  const v2h h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * s;
  const v2h h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * s;
  return v8h{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

template <int IO, int EPI, int BN>
__global__ __launch_bounds__(256, 1)
void gemm_nvfp4_kernel(const uint8_t* __restrict__ act_codes, const uint8_t* __restrict__ act_scales,
                       const float* __restrict__ lora_act, const uint8_t* __restrict__ w_codes,
                       const uint8_t* __restrict__ w_scales, const uint16_t* __restrict__ lora_up,
                       const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, float alpha,
                       int M, int N, int K, int r) {
  using namespace nvfp4;
  constexpr int CB = BN / 64;                    // 32-column blocks per wave
  constexpr int NCODE = (BM + BN) / 32;          // code DMA instructions per thread and pair
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;

  // XCD-aware grouped tile order (each XCD a contiguous range, 4 M-tiles per group)
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
  const int np = K >> 8;           // stage pairs of 256 codes
  const int KB = K >> 1;
  const int SK = K >> 4;           // scale bytes per row

  // ---- DMA plan. Code instruction j of wave w fills slot rows 32 j + 8 w .. +8
  // (rows < BM: A, then B); lane L takes row + L / 8 and chunk L % 8. Scale
  // instruction j fills rows 256 j + 64 w + L (16 bytes each); B rows past BN
  // re-read the last B row into the slot's padding. A rows past M re-read the
  // last row (never stored).
  const uint8_t* tA = act_codes + (size_t)m0 * KB;
  const uint8_t* tB = w_codes + (size_t)n0 * KB;
  const uint8_t* tsA = act_scales + (size_t)m0 * SK;
  const uint8_t* tsB = w_scales + (size_t)n0 * SK;
  const int alast = M - 1 - m0;
  const int rl = 8 * wave + (lane >> 3);
  const int coff = ((lane & 7) ^ nv_swz8(rl)) * 16;
  const uint32_t saoff = (uint32_t)min(64 * wave + lane, alast) * (uint32_t)SK;
  const uint32_t sboff = (uint32_t)min(64 * wave + lane, BN - 1) * (uint32_t)SK;
  const uint32_t lds0 = lds_addr(smem);

  auto dma_pair = [&](int pp) {
    const uint32_t slot = lds0 + (uint32_t)((pp & 1) * SLOT);
#pragma unroll
    for (int j = 0; j < NCODE; ++j) {
      // offsets are formed here rather than kept: registers are the scarce resource
      const uint32_t lds = slot + (uint32_t)((32 * j + 8 * wave) * ROW);
      const uint32_t col = (uint32_t)(coff + pp * ROW);
      if (32 * j < BM) dma16_so(tA, (uint32_t)min(32 * j + rl, alast) * (uint32_t)KB + col, lds);
      else dma16_so(tB, (uint32_t)(32 * j - BM + rl) * (uint32_t)KB + col, lds);
    }
    dma16_so(tsA, saoff + (uint32_t)(pp * SROW), slot + CODES + (uint32_t)(64 * wave * SROW));
    dma16_so(tsB, sboff + (uint32_t)(pp * SROW), slot + CODES + (uint32_t)((256 + 64 * wave) * SROW));
  };

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
  for (int cb = 0; cb < CB; ++cb) brow[cb] = wn * (BN / 2) + cb * 32 + l32;
  const int s8 = nv_swz8(l32);   // == nv_swz8 of every arow / brow

  // operands of half-step hs (0..3) of pair pp: this lane's 32 codes
  // (64 hs + 32 lh .. +32) of each row block, and their two scale bytes
  struct Ops {
    uint4 a[RB], b[CB];
    uint32_t sa[RB], sb[CB];
  };
  // one lane base per operand and half-step; the 32-row blocks are immediate
  // offsets of the LDS reads
  const int a_lane = (wm * 128 + l32) * ROW, b_lane = (BM + wn * (BN / 2) + l32) * ROW;
  const int sa_lane = CODES + (wm * 128 + l32) * SROW + 2 * lh;
  const int sb_lane = CODES + (256 + wn * (BN / 2) + l32) * SROW + 2 * lh;
  auto load_ops = [&](Ops& o, int pp, int hs) {
    const uint8_t* st = smem + (pp & 1) * SLOT;
    const int ch = ((2 * hs + lh) ^ s8) << 4;
    const uint8_t* pa = st + (a_lane + ch);
    const uint8_t* pb = st + (b_lane + ch);
    const uint8_t* psa = st + sa_lane + 4 * hs;
    const uint8_t* psb = st + sb_lane + 4 * hs;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      o.a[rb] = *reinterpret_cast<const uint4*>(pa + rb * 32 * ROW);
      o.sa[rb] = *reinterpret_cast<const uint16_t*>(psa + rb * 32 * SROW);
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      o.b[cb] = *reinterpret_cast<const uint4*>(pb + cb * 32 * ROW);
      o.sb[cb] = *reinterpret_cast<const uint16_t*>(psb + cb * 32 * SROW);
    }
  };
  // Dequantization runs one K block ahead of the MFMAs: while the 16 MFMAs of
  // block j execute, the VALU turns block j + 1 (or the next half-step's block
  // 0) into fp16 operands, 1 MFMA : 4 VALU in the issue order. K block j of a
  // half-step uses dword j of each fragment and scale byte j / 2.
  v8h A0[RB], B0[CB], A1[RB], B1[CB];
  uint32_t pa[RB], pb[CB];
  auto pairs = [&](const Ops& o) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) pa[rb] = nv_scale_pair(o.sa[rb]);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) pb[cb] = nv_scale_pair(o.sb[cb]);
  };
  auto deq = [&](v8h (&A)[RB], v8h (&B)[CB], const Ops& o, int j) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const uint32_t w = j == 0 ? o.a[rb].x : j == 1 ? o.a[rb].y : j == 2 ? o.a[rb].z : o.a[rb].w;
      A[rb] = (j >> 1) ? nv_dequant8<1>(w, pa[rb]) : nv_dequant8<0>(w, pa[rb]);
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const uint32_t w = j == 0 ? o.b[cb].x : j == 1 ? o.b[cb].y : j == 2 ? o.b[cb].z : o.b[cb].w;
      B[cb] = (j >> 1) ? nv_dequant8<1>(w, pb[cb]) : nv_dequant8<0>(w, pb[cb]);
    }
  };
  auto mm = [&](const v8h (&A)[RB], const v8h (&B)[CB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[rb], B[cb], acc[rb][cb], 0, 0, 0);
  };
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < RB * CB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // four VALU
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // one half-step: on entry A0 / B0 hold K block 0 of cur and pa / pb its scale
  // pairs; on exit they hold block 0 of nxt (whose LDS reads were issued earlier)
  auto half = [&](const Ops& cur, const Ops& nxt) {
    deq(A1, B1, cur, 1);
    mm(A0, B0);
    interleave();
    deq(A0, B0, cur, 2);
    mm(A1, B1);
    interleave();
    deq(A1, B1, cur, 3);
    mm(A0, B0);
    interleave();
    pairs(nxt);
    deq(A0, B0, nxt, 0);
    mm(A1, B1);
    interleave();
  };

  Ops P0, P1;
  // prologue: pairs 0 and 1 in flight, wait for pair 0
  dma_pair(0);
  if (np > 1) {
    dma_pair(1);
    waitvm<NCODE + 2>();
  } else {
    waitvm<0>();
  }
  __syncthreads();
  load_ops(P0, 0, 0);
  pairs(P0);
  deq(A0, B0, P0, 0);
  for (int pp = 0; pp < np; ++pp) {
    load_ops(P1, pp, 1);
    half(P0, P1);
    load_ops(P0, pp, 2);
    half(P1, P0);
    load_ops(P1, pp, 3);
    half(P0, P1);
    if (pp + 1 < np) {
      // pair pp + 1 has landed (the only DMA in flight), and every read of pair
      // pp is done; after the barrier pair pp's slot is free for pair pp + 2
      waitvm_lgkm0<0>();
      __syncthreads();
      load_ops(P0, pp + 1, 0);
      if (pp + 2 < np) dma_pair(pp + 2);
    }
    half(P1, P0);   // on the last pair, the look-ahead block is never used
  }

  // ---- per-tensor scales, then the low-rank up-projection into the same
  // accumulators (v_mfma_f32_32x32x16_f16, lane l: row l%32, ranks 8 (l/32) .. +8;
  // lora_act is fp32 and enters as a hi + lo pair of 16-bit operands)
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] *= alpha;
  for (int j0 = 0; j0 < r; j0 += 16) {
    float4 fa[RB][2];
    uint4 ub[CB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int m = min(m0 + arow[rb], M - 1);
      const float* src = lora_act + (size_t)m * r + j0 + lh * 8;
      fa[rb][0] = *reinterpret_cast<const float4*>(src);
      fa[rb][1] = *reinterpret_cast<const float4*>(src + 4);
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      ub[cb] = *reinterpret_cast<const uint4*>(lora_up + (size_t)(n0 + brow[cb]) * r + j0 + lh * 8);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      uint4 hi, lo;
      split8_h16<IO>(fa[rb][0], fa[rb][1], hi, lo);
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        acc[rb][cb] = Io<IO>::mma32x32x16(hi, ub[cb], acc[rb][cb]);
        acc[rb][cb] = Io<IO>::mma32x32x16(lo, ub[cb], acc[rb][cb]);
      }
    }
  }

  // ---- epilogue: bias and activation, staged through LDS so that Y is written
  // as whole rows with 16-byte stores
  constexpr int TP = BN + 8;
  static_assert(BM * TP * 2 <= LDS, "staging tile must fit in the ring");
  waitvm<0>();
  __syncthreads();
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int nl = brow[cb];
    const float bn = bias ? Io<IO>::to_f(bias[n0 + nl]) : 0.f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float yv = acc[rb][cb][v] + bn;
        if (EPI == 1) yv = gelu_tanh_f32(yv);
        tile[(wm * 128 + rb * 32 + (v >> 2) * 8 + lh * 4 + (v & 3)) * TP + nl] = Io<IO>::from_f(yv);
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

template <int IO, int EPI, int BN>
static hipError_t launch_nv(int M, int N, int K, int r, const uint8_t* ac, const uint8_t* as,
                            const void* la, const uint8_t* wc, const uint8_t* ws, const void* lu,
                            const void* bias, float alpha, void* Y, hipStream_t st) {
  using namespace nvfp4;
  auto kern = gemm_nvfp4_kernel<IO, EPI, BN>;
  static std::atomic<uint64_t> raised{0};
  const hipError_t e = raise_lds_limit(raised, reinterpret_cast<const void*>(kern), LDS);
  if (e != hipSuccess) return e;
  const int ntiles = ((M + BM - 1) / BM) * (N / BN);
  hipLaunchKernelGGL(kern, dim3(ntiles), dim3(256), LDS, st, ac, as, (const float*)la, wc, ws,
                     (const uint16_t*)lu, (const uint16_t*)bias, (uint16_t*)Y, alpha, M, N, K, r);
  return hipGetLastError();
}

template <int IO>
static hipError_t launch_nv_io(int M, int N, int K, int r, const uint8_t* ac, const uint8_t* as,
                               const void* la, const uint8_t* wc, const uint8_t* ws, const void* lu,
                               const void* bias, float alpha, int epi, void* Y, hipStream_t st) {
  // 256 x 256 tiles unless that grid would fill at most half the CUs: then
  // 256 x 128 tiles, twice as many in one round (M1024 K12288 N3072: 48 tiles,
  // 243 -> 159 us; with 144 or 192 tiles the second round costs more, 77 -> 97 us)
  if (N % 256 == 0 && ((M + 255) / 256) * (N / 256) > 128) {
    return epi ? launch_nv<IO, 1, 256>(M, N, K, r, ac, as, la, wc, ws, lu, bias, alpha, Y, st)
               : launch_nv<IO, 0, 256>(M, N, K, r, ac, as, la, wc, ws, lu, bias, alpha, Y, st);
  }
  return epi ? launch_nv<IO, 1, 128>(M, N, K, r, ac, as, la, wc, ws, lu, bias, alpha, Y, st)
             : launch_nv<IO, 0, 128>(M, N, K, r, ac, as, la, wc, ws, lu, bias, alpha, Y, st);
}

hipError_t launch_gemm_nvfp4(int io, int M, int N, int K, int r, const uint8_t* ac, const uint8_t* as,
                             const void* la, const uint8_t* wc, const uint8_t* ws, const void* lu,
                             const void* bias, float alpha, int epi, void* Y, hipStream_t st) {
  if (io == 1) return launch_nv_io<1>(M, N, K, r, ac, as, la, wc, ws, lu, bias, alpha, epi, Y, st);
  return launch_nv_io<0>(M, N, K, r, ac, as, la, wc, ws, lu, bias, alpha, epi, Y, st);
}

}  // namespace svdq
