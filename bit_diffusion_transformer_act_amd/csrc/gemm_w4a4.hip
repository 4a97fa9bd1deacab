// svdq_gemm_w4a4: the 4-bit GEMM with the low-rank up-projection, scale
// dequantization, bias and GELU fused into one kernel (the pages fuse the
// up-projection with the 4-bit compute kernel so the 16-bit branch costs no
// extra memory pass: dothoosh.com "How Nunchaku Lite halves diffusion-model
// VRAM", fused-kernel paragraph; W4A4 with both operands 4-bit: same
// article, SVDQuant paragraph, and nextgz.net "Hugging Face brings Nunchaku
// Lite to Diffusers", section "Why W4A4 differs from weight-only backends").
//
// Tiling: a workgroup of 4 waves (2 x 2) owns a BM x BN output tile, each wave
// (32 WM) x (32 WN): 16 x 16 MFMA blocks for INT4, 32 x 32 for FP4. The K loop walks steps of
// 128 codes (64 packed bytes per row). Each step (A codes, B codes and both
// operands' scale words) is brought into an LDS ring of STAGES buffers by
// LDS-DMA loads (global_load_lds_dwordx4 / _dword): no register staging, and
// the loads for step ks + STAGES - 1 are in flight while step ks computes.
// One barrier per step. Code rows are 64 bytes with the four 16-byte chunks
// XOR-swizzled by (row >> 2) & 3, so 16 consecutive rows read at one chunk
// index touch 16 distinct 16-byte bank slots.
//
// Blocks are remapped so that each of the 8 XCDs (round-robin dispatch)
// works on a contiguous range of tiles in 8-M-tile groups, which keeps the A
// and B rows of concurrently running tiles in that XCD's L2.
//
// Accumulators start from the low-rank product: lora_act (fp32, entering as a
// hi + lo pair of 16-bit operands) times lora_up on 16-bit MFMAs.
//
// INT4_G64: each lane reads 8 packed bytes (16 codes) per 16-row block and
// group; nibbles become int8 bytes holding 16 q (hi = w & 0xF0F0F0F0,
// lo = (w << 4) & 0xF0F0F0F0), so the int32 result is 256 sum q_x q_w exactly.
// One v_mfma_i32_16x16x64_i8 gives a 16 x 16 block's partial P of one group.
// The int32 accumulation starts from the bit pattern of 1.5 * 2^23, so the
// result read as fp32 is exactly 1.5*2^23 + 256 P; one fma with s_w and the
// exact constant -1.5*2^23 s_w yields fl(256 P s_w) = 256 fl(P s_w) with no
// int-to-float convert, and a second fma adds s_x times that to the fp32
// accumulator: two VALU ops per output and group, plain fp32 fmas on scales
// converted once per step (gfx950 issues v_fma_mix with a 16-bit operand
// slower than v_fma_f32). The accumulators therefore hold 256 times the sum (the
// low-rank start is scaled to match); the epilogue's multiply by 2^-8 is exact.
// A and B use the same permutation of k inside the instruction, which a dot
// product does not see.
//
// FP4_E2M1_B32: the packed codes are the operands of
// v_mfma_scale_f32_32x32x64_f8f6f4 as they are (lane l: row l%32, k
// 32 (l/32) .. +32), with the E8M0 byte of (row, 32-block) as the lane's
// scale; the hardware applies both scales and accumulates in fp32.
#include <algorithm>
#include <atomic>

#include "chain.hpp"
#include "common.hpp"
#include "launch.hpp"
#include "pipeline.hpp"

namespace svdq {

// 16 packed INT4 codes (two words) -> one int8 MFMA operand of 16 bytes:
// [even codes of w0, odd codes of w0, even of w1, odd of w1], each byte 16 q.
__device__ __forceinline__ v4i unpack_i4x16(uint32_t w0, uint32_t w1) {
  return v4i{(int)((w0 << 4) & 0xF0F0F0F0u), (int)(w0 & 0xF0F0F0F0u),
             (int)((w1 << 4) & 0xF0F0F0F0u), (int)(w1 & 0xF0F0F0F0u)};
}


// 0x4B400000 is 1.5 * 2^23 as fp32: integers added to it stay exact in the
// mantissa while |x| < 2^22.
constexpr int kMagicBits = 0x4B400000;
#define SVDQ_M16 kMagicBits, kMagicBits, kMagicBits, kMagicBits
__device__ constexpr v4i kMagic4 = {SVDQ_M16};
#undef SVDQ_M16

template <int WM, int WN, int STAGES>
struct GemmShape {
  static constexpr int BM = 64 * WM, BN = 64 * WN;
  static constexpr int A_BYTES = BM * 64, B_BYTES = BN * 64;
  static constexpr int SC_ROWS = (BM + BN + 255) / 256 * 256;   // scale rows (A, B, padding)
  static constexpr int STAGE = A_BYTES + B_BYTES;                 // one step's codes
  // Scales go in groups of two steps, [SC_ROWS][2] 4-byte words (a row's words of
  // steps 2g and 2g + 1 are adjacent in memory, so two lanes per row read one
  // line where one lane per row and step would read two). A group is loaded with
  // the codes of its first step; STAGES / 2 + 1 slots keep a slot from being
  // refilled while its steps are still read.
  static constexpr int SC_SLOTS = STAGES / 2 + 1;
  static constexpr int SC_GROUP = SC_ROWS * 8;
  static constexpr int SC_GINSTR = SC_GROUP / 1024;               // dword DMAs per wave per group
  static constexpr int LDS = STAGES * STAGE + SC_SLOTS * SC_GROUP;
  static constexpr int NC = BM / 64 + BN / 64;                    // code DMAs per thread per step
};

// 3 waves per SIMD (at most 168 VGPRs): the INT4 inner loop is VALU-bound and
// needs the extra wave to cover LDS and MFMA latencies.
template <int IO, int FMT, int EPI, int WM, int WN, int STAGES>
__global__ __launch_bounds__(256, 3)
void gemm_w4a4_kernel(const uint8_t* __restrict__ act_codes, const void* __restrict__ act_scales,
                      const float* __restrict__ lora_act, const uint8_t* __restrict__ w_codes,
                      const void* __restrict__ w_scales, const uint16_t* __restrict__ lora_up,
                      const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y,
                      int M, int N, int K, int r, QkvEpilogue qe, ChainEpilogue ce, SplitK sk) {
  using S = GemmShape<WM, WN, STAGES>;
  constexpr int BM = S::BM, BN = S::BN;
  // the 3-stage tiles rely on three workgroups per CU (the launch bound): their
  // LDS must fit three times in the CU's 160 KB, or occupancy drops silently
  static_assert(STAGES != 3 || 3 * S::LDS <= 160 * 1024, "three 3-stage workgroups must fit in a CU's LDS");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;

  // ---- tile index, XCD-aware: XCD x (blocks x, x+8, ...) takes the x-th
  // contiguous eighth of the logical tiles, which run in groups of 8 M-tiles
  // with N outer, so the ~64 tiles resident on one XCD form an 8 x 8 patch and
  // share A and B rows through that XCD's L2.
  const int ntm = (M + BM - 1) / BM;
  const int ntn = N / BN;
  const int ntiles = ntm * ntn;
  // EPI 4 (split K): workgroup ids run over (split, tile); the XCD remap over all
  // of them keeps the tiles of one split, which share A and B rows, on one XCD
  const int nsplit = EPI == 4 ? sk.splits : 1;
  const int total = ntiles * nsplit;
  int pid = blockIdx.x;
  if ((total & 7) == 0) pid = (pid & 7) * (total >> 3) + (pid >> 3);
  const int split = EPI == 4 ? pid / ntiles : 0;
  pid -= split * ntiles;
  constexpr int GROUP_M = 8;
  const int gsz = GROUP_M * ntn;
  const int first_m = (pid / gsz) * GROUP_M;
  const int gm = min(ntm - first_m, GROUP_M);
  const int m0 = (first_m + (pid % gsz) % gm) * BM;
  const int n0 = ((pid % gsz) / gm) * BN;
  // this workgroup's K steps: all of them, or split `split` of nsplit near-equal runs
  const int nk_all = K >> 7;
  const int ks0 = (int)((long long)split * nk_all / nsplit);
  const int nk = (int)((long long)(split + 1) * nk_all / nsplit) - ks0;
  const int KB = K >> 1;  // bytes per packed row
  const int sstride = (FMT == 0) ? (K >> 6) * 2 : (K >> 5);  // scale bytes per row

  // ---- DMA source pointers (per lane) for step 0; advance by 64 B (codes) / 4 B (scales)
  const uint8_t* ga[BM / 64];
  const uint8_t* gb[BN / 64];
  const uint8_t* gs[S::SC_GINSTR];
  uint32_t la_off[BM / 64], lb_off[BN / 64], ls_off[S::SC_GINSTR];
  const uint32_t lds0 = lds_addr(smem);
#pragma unroll
  for (int i = 0; i < BM / 64; ++i) {
    // wave w, instruction i: 16 rows starting at w*(BM/4) + 16 i; lane -> (row, slot)
    const int rloc = wave * (BM / 4) + 16 * i;
    const int row = rloc + (lane >> 2);
    const int chunk = (lane & 3) ^ swz(row);
    const int grow = min(m0 + row, M - 1);
    ga[i] = act_codes + (size_t)grow * KB + chunk * 16 + (size_t)ks0 * 64;
    la_off[i] = rloc * 64;
  }
#pragma unroll
  for (int i = 0; i < BN / 64; ++i) {
    const int rloc = wave * (BN / 4) + 16 * i;
    const int row = rloc + (lane >> 2);
    const int chunk = (lane & 3) ^ swz(row);
    gb[i] = w_codes + (size_t)(n0 + row) * KB + chunk * 16 + (size_t)ks0 * 64;
    lb_off[i] = S::A_BYTES + rloc * 64;
  }
#pragma unroll
  for (int i = 0; i < S::SC_GINSTR; ++i) {
    // 32 rows per instruction, lanes 2 j and 2 j + 1 on row rloc + j (its words of the group's two steps)
    const int rloc = (wave * S::SC_GINSTR + i) * 32;
    const int row = rloc + (lane >> 1);   // rows [0, BM) are A, [BM, BM + BN) are B, beyond: padding
    const uint8_t* p;
    if (row < BM) p = reinterpret_cast<const uint8_t*>(act_scales) + (size_t)min(m0 + row, M - 1) * sstride;
    else if (row < BM + BN) p = reinterpret_cast<const uint8_t*>(w_scales) + (size_t)(n0 + row - BM) * sstride;
    else p = reinterpret_cast<const uint8_t*>(w_scales) + (size_t)n0 * sstride;
    gs[i] = p + (size_t)ks0 * 4;   // 4 scale bytes per row and step in both formats
    ls_off[i] = rloc * 8;
  }

  auto issue = [&](int ks) {
    const uint32_t base = lds0 + (uint32_t)((ks % STAGES) * S::STAGE);
#pragma unroll
    for (int i = 0; i < BM / 64; ++i) dma16(ga[i] + ks * 64, base + la_off[i]);
#pragma unroll
    for (int i = 0; i < BN / 64; ++i) dma16(gb[i] + ks * 64, base + lb_off[i]);
    if ((ks & 1) == 0) {   // the scale group of steps ks and ks + 1 (the last step again past nk)
      const uint32_t sb = lds0 + (uint32_t)(STAGES * S::STAGE + ((ks >> 1) % S::SC_SLOTS) * S::SC_GROUP);
      const int sst = min(ks + (lane & 1), nk - 1);
#pragma unroll
      for (int i = 0; i < S::SC_GINSTR; ++i) dma4(gs[i] + sst * 4, sb + ls_off[i]);
    }
  };

  // prologue loads go out before the low-rank product so they overlap it
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) issue(s);

  // ---- low-rank up-projection initialises the accumulators. INT4 keeps 16 x 16
  // blocks (acc4), FP4 32 x 32 blocks (acc); only one of the two is live.
  constexpr int RB4 = (FMT == 0) ? 2 * WM : 1, CB4 = (FMT == 0) ? 2 * WN : 1;
  constexpr int RB32 = (FMT == 0) ? 1 : WM, CB32 = (FMT == 0) ? 1 : WN;
  v4f acc4[RB4][CB4];
  v16f acc[RB32][CB32];
#pragma unroll
  for (int i = 0; i < RB4; ++i)
#pragma unroll
    for (int j = 0; j < CB4; ++j) acc4[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RB32; ++i)
#pragma unroll
    for (int j = 0; j < CB32; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int rl = split == 0 ? r : 0;   // split K: the low-rank product joins split 0 only
  if constexpr (FMT == 0) {
    // v_mfma_f32_16x16x16_f16: lane l supplies row l%16, ranks j0 + 4 (l/16) .. +4,
    // as the hi and the lo halves of lora_act (two MFMAs per block and 16 ranks).
    // Loads for 16 ranks go out together (more would raise the register peak).
    const int l16 = lane & 15, lq = lane >> 4;
    for (int j0 = 0; j0 < rl; j0 += 16) {
      float4 fa[RB4];
      uint2 ub[CB4];
#pragma unroll
      for (int rb = 0; rb < RB4; ++rb) {
        const int m = m0 + wm * 32 * WM + rb * 16 + l16;
        fa[rb] = (m < M) ? *reinterpret_cast<const float4*>(lora_act + (size_t)m * r + j0 + lq * 4)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int cb = 0; cb < CB4; ++cb) {
        const int n = n0 + wn * 32 * WN + cb * 16 + l16;
        ub[cb] = *reinterpret_cast<const uint2*>(lora_up + (size_t)n * r + j0 + lq * 4);
      }
#pragma unroll
      for (int rb = 0; rb < RB4; ++rb) {
        uint2 hi, lo;
        split4_h16<IO>(fa[rb], hi, lo);
#pragma unroll
        for (int cb = 0; cb < CB4; ++cb) {
          acc4[rb][cb] = Io<IO>::mma16x16x16(hi, ub[cb], acc4[rb][cb]);
          acc4[rb][cb] = Io<IO>::mma16x16x16(lo, ub[cb], acc4[rb][cb]);
        }
      }
    }
  } else {
    // v_mfma_f32_32x32x16_f16: lane l supplies row l%32, ranks j0 + 8 (l/32) .. +8,
    // as the hi and the lo halves of lora_act.
    for (int j0 = 0; j0 < rl; j0 += 16) {
      float4 fa[RB32][2];
      uint4 ub[CB32];
#pragma unroll
      for (int rb = 0; rb < RB32; ++rb) {
        const int m = m0 + wm * 32 * WM + rb * 32 + l32;
        const float* src = lora_act + (size_t)m * r + j0 + lh * 8;
        fa[rb][0] = (m < M) ? *reinterpret_cast<const float4*>(src) : make_float4(0.f, 0.f, 0.f, 0.f);
        fa[rb][1] = (m < M) ? *reinterpret_cast<const float4*>(src + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int cb = 0; cb < CB32; ++cb) {
        const int n = n0 + wn * 32 * WN + cb * 32 + l32;
        ub[cb] = *reinterpret_cast<const uint4*>(lora_up + (size_t)n * r + j0 + lh * 8);
      }
#pragma unroll
      for (int rb = 0; rb < RB32; ++rb) {
        uint4 hi, lo;
        split8_h16<IO>(fa[rb][0], fa[rb][1], hi, lo);
#pragma unroll
        for (int cb = 0; cb < CB32; ++cb) {
          acc[rb][cb] = Io<IO>::mma32x32x16(hi, ub[cb], acc[rb][cb]);
          acc[rb][cb] = Io<IO>::mma32x32x16(lo, ub[cb], acc[rb][cb]);
        }
      }
    }
  }

  if constexpr (FMT == 0) {
    // the INT4 main loop accumulates 256 times the sum (exact power of two)
#pragma unroll
    for (int i = 0; i < RB4; ++i)
#pragma unroll
      for (int j = 0; j < CB4; ++j) acc4[i][j] *= 256.0f;
  }

  // LDS read offsets (within a stage) of this lane's operand rows
  int arow[WM], brow[WN];
#pragma unroll
  for (int rb = 0; rb < WM; ++rb) arow[rb] = wm * 32 * WM + rb * 32 + l32;
#pragma unroll
  for (int cb = 0; cb < WN; ++cb) brow[cb] = wn * 32 * WN + cb * 32 + l32;

  for (int ks = 0; ks < nk; ++ks) {
    // issue(j) puts NC code DMAs in flight, and SC_GINSTR scale DMAs more when j is
    // even; the batches of the STAGES - 2 steps after ks may stay outstanding
    constexpr int NC = S::NC, NG = S::SC_GINSTR;
    static_assert(STAGES == 3 || STAGES == 4, "wait counts are written out for 3 and 4 stages");
    if constexpr (STAGES == 3) {
      if (ks + 1 < nk) {
        if (ks & 1) waitvm<NC + NG>();
        else waitvm<NC>();
      } else {
        waitvm<0>();
      }
    } else {
      if (ks + 2 < nk) {
        waitvm<2 * NC + NG>();
      } else if (ks + 1 < nk) {
        if (ks & 1) waitvm<NC + NG>();
        else waitvm<NC>();
      } else {
        waitvm<0>();
      }
    }
    __syncthreads();
    if (ks + STAGES - 1 < nk) issue(ks + STAGES - 1);

    const uint8_t* st = smem + (ks % STAGES) * S::STAGE;
    const uint8_t* sA = st;
    const uint8_t* sB = st + S::A_BYTES;
    // this step's scale words: word ks & 1 of each row in the slot of group ks / 2
    const uint32_t* sS = reinterpret_cast<const uint32_t*>(smem + STAGES * S::STAGE +
                                                           ((ks >> 1) % S::SC_SLOTS) * S::SC_GROUP) + (ks & 1);

    if constexpr (FMT == 0) {
      // INT4 on v_mfma_i32_16x16x64_i8: the wave tile is (2 WM) x (2 WN) blocks
      // of 16 x 16, one MFMA per block and 64-group. Lane l supplies row l%16
      // and 16 codes (8 packed bytes at 8 (l/16) within the group's 32 bytes);
      // its results are rows 4 (l/16) + i, column l%16 of the block.
      constexpr int RB = 2 * WM, CB = 2 * WN;
      const int l16 = lane & 15, lq = lane >> 4;
      // scale words: 2 fp16 per row (groups 2 ks, 2 ks + 1); 4 rows per 16-byte read
      uint4 sxw[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
      {
        const uint32_t* q = sS + 2 * (wm * 32 * WM + rb * 16 + lq * 4);
        sxw[rb] = make_uint4(q[0], q[2], q[4], q[6]);
      }
      uint32_t sww[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) sww[cb] = sS[2 * (BM + wn * 32 * WN + cb * 16 + l16)];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        v4i av[RB], bv[CB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int rr = wm * 32 * WM + rb * 16 + l16;
          const uint2 ap = *reinterpret_cast<const uint2*>(
              sA + rr * 64 + (((g * 2 + (lq >> 1)) ^ swz(rr)) << 4) + (lq & 1) * 8);
          av[rb] = unpack_i4x16(ap.x, ap.y);
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          const int rr = wn * 32 * WN + cb * 16 + l16;
          const uint2 bp = *reinterpret_cast<const uint2*>(
              sB + rr * 64 + (((g * 2 + (lq >> 1)) ^ swz(rr)) << 4) + (lq & 1) * 8);
          bv[cb] = unpack_i4x16(bp.x, bp.y);
        }
        // the group's scales in fp32, converted once: fp32 fma issues faster
        // than v_fma_mix with a 16-bit operand (the empty asm keeps the
        // compiler from folding the conversions back into the fmas)
        float sxf[RB][4];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const uint32_t wx[4] = {sxw[rb].x, sxw[rb].y, sxw[rb].z, sxw[rb].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float f = (float)__builtin_bit_cast(v2h, wx[i])[g];
            asm volatile("" : "+v"(f));
            sxf[rb][i] = f;
          }
        }
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
          float swf = (float)__builtin_bit_cast(v2h, sww[cb])[g];
          asm volatile("" : "+v"(swf));
          // -1.5*2^23 s_w is exact: s_w has 11 significant bits, 3 s_w at most 13
          const float swm = swf * -12582912.0f;
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            // int32 accumulation starts at the bit pattern of 1.5 * 2^23, so the
            // result read as fp32 is exactly 1.5 * 2^23 + 256 P (|256 P| < 2^22)
            const v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[rb], bv[cb], kMagic4, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              // t = fl(256 P s_w): one rounding of (1.5*2^23 + 256 P) s_w - 1.5*2^23 s_w
              const float t = fmaf(__int_as_float(p[i]), swf, swm);
              acc4[rb][cb][i] = fmaf(t, sxf[rb][i], acc4[rb][cb][i]);
            }
          }
        }
      }
    } else {
      uint32_t ea[WM], eb[WN];
#pragma unroll
      for (int rb = 0; rb < WM; ++rb) ea[rb] = sS[2 * arow[rb]];
#pragma unroll
      for (int cb = 0; cb < WN; ++cb) eb[cb] = sS[2 * (BM + brow[cb])];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int sh = 8 * (2 * g + lh);
        v8i av[WM], bv[WN];
#pragma unroll
        for (int rb = 0; rb < WM; ++rb) {
          const int rr = arow[rb];
          const uint4 ap = *reinterpret_cast<const uint4*>(sA + rr * 64 + (((g * 2 + lh) ^ swz(rr)) << 4));
          av[rb] = v8i{(int)ap.x, (int)ap.y, (int)ap.z, (int)ap.w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int cb = 0; cb < WN; ++cb) {
          const int rr = brow[cb];
          const uint4 bp = *reinterpret_cast<const uint4*>(sB + rr * 64 + (((g * 2 + lh) ^ swz(rr)) << 4));
          bv[cb] = v8i{(int)bp.x, (int)bp.y, (int)bp.z, (int)bp.w, 0, 0, 0, 0};
        }
#pragma unroll
        for (int rb = 0; rb < WM; ++rb)
#pragma unroll
          for (int cb = 0; cb < WN; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                av[rb], bv[cb], acc[rb][cb], 4, 4, 0, (int)((ea[rb] >> sh) & 0xFFu), 0,
                (int)((eb[cb] >> sh) & 0xFFu));
      }
    }
  }

  if constexpr (EPI == 4) {
    // split K: this split's fp32 partial of the tile (256 times the sum, as the
    // accumulators hold it) goes to its slice [split][M][N]; the reduce kernel
    // adds the slices in split order and applies the epilogue
    static_assert(FMT == 0, "split K runs the INT4 kernel");
    const int l16 = lane & 15, lq = lane >> 4;
    float* part = sk.part + (size_t)split * M * N;
#pragma unroll
    for (int rb = 0; rb < RB4; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + wm * 32 * WM + rb * 16 + lq * 4 + i;
        if (m < M) {
#pragma unroll
          for (int cb = 0; cb < CB4; ++cb) part[(size_t)m * N + n0 + wn * 32 * WN + cb * 16 + l16] = acc4[rb][cb][i];
        }
      }
    return;
  }
  // ---- epilogue: bias and activation, then the tile goes through LDS (the ring
  // is free now) so that Y is written as whole rows with 16-byte stores.
  constexpr int TP = BN + 8;   // padded row (halves) of the staging tile
  static_assert(BM * TP * 2 <= S::LDS, "staging tile must fit in the ring");
  __syncthreads();
  uint16_t* tile = reinterpret_cast<uint16_t*>(smem);
  uint2 ce_pre[EPI == 3 ? 2 : 1][EPI == 3 ? BN / 16 : 1];   // lora_down operands of the chain's partial
  if constexpr (FMT == 0) {
    const int l16 = lane & 15, lq = lane >> 4;
    // the fused QKV epilogue applies to the Q and K thirds (a tile is one head:
    // BN == 128); the block-uniform test keeps every barrier below uniform
    bool normrope = false;
    if constexpr (EPI == 2) {
      static_assert(BN == 128, "the QKV epilogue needs one 128-channel head per tile");
      normrope = (n0 / BN) < 2 * qe.heads;
    }
    float yv[RB4][CB4][4];
#pragma unroll
    for (int cb = 0; cb < CB4; ++cb) {
      const int nl = wn * 32 * WN + cb * 16 + l16;
      const float bn = bias ? Io<IO>::to_f(bias[n0 + nl]) : 0.f;
#pragma unroll
      for (int rb = 0; rb < RB4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = fmaf(acc4[rb][cb][i], 0.00390625f, bn);   // exact 2^-8, then + bias
          if (EPI == 1 || EPI == 3) v = gelu_tanh_f32(v);
          yv[rb][cb][i] = v;
        }
    }
    if constexpr (EPI == 2) {
      if (normrope) {
        // RMSNorm over the head's 128 channels: this lane's 4 columns, then the
        // 16 lanes of its 16-lane row (DPP), then the two waves of the row pair
        // through LDS (summed in a fixed order, so both see the same total)
        float* red = reinterpret_cast<float*>(smem + BM * TP * 2);   // [WM][2 waves][64 rows]
#pragma unroll
        for (int rb = 0; rb < RB4; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float ss = 0.f;
#pragma unroll
            for (int cb = 0; cb < CB4; ++cb) ss = fmaf(yv[rb][cb][i], yv[rb][cb][i], ss);
            ss = row16_sum(ss);
            if (l16 == 0) red[(wm * 2 + wn) * 64 + rb * 16 + lq * 4 + i] = ss;
          }
        __syncthreads();
        const int part = (n0 / BN) / qe.heads;   // 0: Q, 1: K
        const uint16_t* nw = reinterpret_cast<const uint16_t*>(qe.qk_norm_w) + part * BN;
#pragma unroll
        for (int rb = 0; rb < RB4; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rl = rb * 16 + lq * 4 + i;
            const float tot = red[(wm * 2 + 0) * 64 + rl] + red[(wm * 2 + 1) * 64 + rl];
            const float inv = __builtin_amdgcn_rsqf(fmaf(tot, 1.0f / 128.0f, qe.eps));
            const int m = min(m0 + wm * 32 * WM + rl, M - 1);
#pragma unroll
            for (int cb = 0; cb < CB4; ++cb) {
              const int d = wn * 32 * WN + cb * 16 + l16;   // channel within the head
              const float v = yv[rb][cb][i] * inv * Io<IO>::to_f(nw[d]);
              // partner channel d ^ 1 sits in lane ^ 1 (columns are lanes)
              const float pv = __int_as_float(
                  __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
              const float2 cs = *reinterpret_cast<const float2*>(qe.rope + ((size_t)m * 64 + (d >> 1)) * 2);
              // (a, b) -> (a cos - b sin, a sin + b cos)
              yv[rb][cb][i] = (d & 1) ? fmaf(pv, cs.y, v * cs.x) : fmaf(-pv, cs.y, v * cs.x);
            }
          }
      }
    }
#pragma unroll
    for (int cb = 0; cb < CB4; ++cb) {
      const int nl = wn * 32 * WN + cb * 16 + l16;
#pragma unroll
      for (int rb = 0; rb < RB4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          tile[(wm * 32 * WM + rb * 16 + lq * 4 + i) * TP + nl] = Io<IO>::from_f(yv[rb][cb][i]);
    }
    if constexpr (EPI == 3) {
      // The fused MLP chain: U (the 16-bit values just staged) is the input of the
      // down-projection's quantizer, exactly as if it had gone through memory.
      // This wave's 64 columns are one INT4 group of the down-projection's K, so
      // a row's group max is a max over this lane's 4 columns and the 16 lanes of
      // its DPP row. Codes and scales are staged in LDS, then stored as lines.
      static_assert(WN == 2 && 32 * WN == 64, "one INT4 group per wave");
      static_assert(BM * TP * 2 + BM * (BN / 2) + BM * 4 <= S::LDS, "chain staging must fit in the ring");
      uint8_t* cst = smem + BM * TP * 2;                                // [BM][BN / 2] code bytes
      __half* sst = reinterpret_cast<__half*>(cst + BM * (BN / 2));     // [BM][2] scales
      // the low-rank partial's first 32 ranks of lora_down go out now, so their
      // latency hides behind the quantization below
      if (ce.r > 0) {
        const uint16_t* ldn = reinterpret_cast<const uint16_t*>(ce.lora_down);
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
          for (int k = 0; k < BN / 16; ++k)
            ce_pre[jb][k] = *reinterpret_cast<const uint2*>(
                ldn + (size_t)(min(jb * 16, ce.r - 16) + l16) * N + n0 + k * 16 + lq * 4);
      }
      float sv[CB4];
#pragma unroll
      for (int cb = 0; cb < CB4; ++cb) sv[cb] = ce.smooth_inv[n0 + wn * 64 + cb * 16 + l16];
#pragma unroll
      for (int rb = 0; rb < RB4; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = wm * 32 * WM + rb * 16 + lq * 4 + i;
          float x[CB4];
          float amax = 0.f;
#pragma unroll
          for (int cb = 0; cb < CB4; ++cb) {
            // x_hat = fl32(u * smooth_inv): one multiply, -0 addend keeps the sign of zero
            x[cb] = fmaf(Io<IO>::to_f(Io<IO>::from_f(yv[rb][cb][i])), sv[cb], -0.0f);
            amax = fmaxf(amax, fabsf(x[cb]));
          }
          amax = row16_max(amax);
          const __half s16 = __float2half_rn(fminf(div7_rn(amax), 65504.0f));   // fl32(amax / 7)
          const float sf = __half2float(s16);
          // q = clamp(rint(fl32(x / s)), -7, 7): x * rcp(s) rounded inside
          // fma(x, rcp(s), 1.5 * 2^23) gives the same integer unless the product
          // lies within 2^-16 of a half-integer (rcp is within an ulp, so it is
          // within 2^-19 |y| of the quotient); such lanes redo the IEEE division
          constexpr float kM = 12582912.0f;   // 1.5 * 2^23
          const float rs = sf != 0.0f ? __builtin_amdgcn_rcpf(sf) : 0.0f;
          int qn[CB4];
          float tmax = 0.0f;
#pragma unroll
          for (int cb = 0; cb < CB4; ++cb) {
            const float y = __builtin_amdgcn_fmed3f(fmaf(x[cb], rs, kM), kM - 7.0f, kM + 7.0f);
            tmax = __builtin_fmaxf(tmax, fabsf(fmaf(x[cb], rs, -(y - kM))));
            qn[cb] = (int)(__float_as_uint(y) & 0xFu);
          }
          const bool near_tie = tmax > 0.4999847412109375f;   // 0.5 - 2^-16
          if (near_tie && sf != 0.0f) {
#pragma unroll
            for (int cb = 0; cb < CB4; ++cb)
              qn[cb] = (int)fminf(fmaxf(rintf(x[cb] / sf), -7.0f), 7.0f) & 0xF;   // IEEE division
          }
#pragma unroll
          for (int cb = 0; cb < CB4; ++cb) {
            const int qo = __builtin_amdgcn_update_dpp(0, qn[cb], 0xB1, 0xF, 0xF, false);   // column + 1
            if ((l16 & 1) == 0) cst[row * (BN / 2) + wn * 32 + cb * 8 + (l16 >> 1)] = (uint8_t)(qn[cb] | (qo << 4));
          }
          if (l16 == 0) sst[row * 2 + wn] = s16;
        }
    }
  } else {
#pragma unroll
    for (int cb = 0; cb < CB32; ++cb) {
      const int nl = brow[cb];
      const float bn = bias ? Io<IO>::to_f(bias[n0 + nl]) : 0.f;
#pragma unroll
      for (int rb = 0; rb < RB32; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float yv = acc[rb][cb][v] + bn;
          if (EPI == 1 || EPI == 3) yv = gelu_tanh_f32(yv);
          tile[(wm * 32 * WM + rb * 32 + (v >> 2) * 8 + lh * 4 + (v & 3)) * TP + nl] = Io<IO>::from_f(yv);
        }
    }
    if constexpr (EPI == 3) {
      // the fused MLP chain on a 4-bit float up-projection: the down-projection's
      // smoothing vector for the tile's columns, next to the staged tile
      static_assert(BM * TP * 2 + BN * 4 <= S::LDS, "chain staging must fit in the ring");
      float* si_lds = reinterpret_cast<float*>(smem + BM * TP * 2);
      if (tid < BN / 4)
        *reinterpret_cast<float4*>(si_lds + 4 * tid) = *reinterpret_cast<const float4*>(ce.smooth_inv + n0 + 4 * tid);
    }
  }
  __syncthreads();
  if constexpr (EPI == 3 && FMT != 0) {
    // the staged U tile through the down-projection's quantizer, and its low-rank partial
    const float* si_lds = reinterpret_cast<const float*>(smem + BM * TP * 2);
    chain_quantize_tile<IO, BM, BN, TP>(tile, si_lds, m0, n0, M, N, ce, tid);
    if (ce.r > 0)
      chain_lowrank_partial<IO, BM, BN, TP>(tile, m0, n0, M, N, ce, ce.partial + (size_t)(n0 / BN) * M * ce.r,
                                            wave, lane);
  } else if constexpr (EPI != 3) {
    for (int c = tid; c < BM * (BN / 8); c += 256) {
      const int row = c / (BN / 8), c8 = c - row * (BN / 8);
      if (m0 + row < M)
        *reinterpret_cast<uint4*>(Y + (size_t)(m0 + row) * N + n0 + c8 * 8) =
            *reinterpret_cast<const uint4*>(tile + row * TP + c8 * 8);
    }
  } else {
    const uint8_t* cst = smem + BM * TP * 2;
    const uint32_t* sst = reinterpret_cast<const uint32_t*>(cst + BM * (BN / 2));
    for (int c = tid; c < BM * (BN / 32); c += 256) {          // codes: 64 bytes per row
      const int row = c / (BN / 32), c16 = c - row * (BN / 32);
      if (m0 + row < M)
        *reinterpret_cast<uint4*>(ce.codes + (size_t)(m0 + row) * (N >> 1) + (n0 >> 1) + c16 * 16) =
            *reinterpret_cast<const uint4*>(cst + row * (BN / 2) + c16 * 16);
    }
    for (int row = tid; row < BM; row += 256)                  // scales: the tile's 2 groups per row
      if (m0 + row < M)
        *reinterpret_cast<uint32_t*>(reinterpret_cast<__half*>(ce.scales) + (size_t)(m0 + row) * (N >> 6) +
                                     (n0 >> 6)) = sst[row];
    // low-rank partial of the down-projection over this tile's 128 columns:
    // P[m][j] = sum_n U[m][n] lora_down[j][n0 + n], v_mfma 16x16x16 (lane l: row or
    // rank l % 16, k 4 (l / 16) .. +4; result: rank l % 16, rows 4 (l / 16) + i).
    // Wave w takes rows 32 w .. +32; written in full to the tile's slice.
    const int l16 = lane & 15, lq = lane >> 4;
    const uint16_t* ldn = reinterpret_cast<const uint16_t*>(ce.lora_down);
    float* part = ce.partial + ((size_t)(n0 / BN) * M) * ce.r;
    for (int jb = 0; jb < ce.r; jb += 16) {
      v4f pacc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int k0 = 0; k0 < BN; k0 += 16) {
        const uint2 bw = jb < 32 ? ce_pre[jb >> 4][k0 >> 4]
                                 : *reinterpret_cast<const uint2*>(ldn + (size_t)(jb + l16) * N + n0 + k0 + lq * 4);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint2 aw = *reinterpret_cast<const uint2*>(tile + (wave * 32 + h * 16 + l16) * TP + k0 + lq * 4);
          pacc[h] = Io<IO>::mma16x16x16(aw, bw, pacc[h]);
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + wave * 32 + h * 16 + lq * 4 + i;
          if (m < M) part[(size_t)m * ce.r + jb + l16] = pacc[h][i];
        }
    }
  }
}

// lora_act[m][j] = sum_t partial[t][m][j] (fp32), summed in the order t = 0, 1, ...
// Each thread takes 4 consecutive elements (16-byte loads) and keeps the loads
// of 8 tiles in flight ahead of the adds (the order of the adds is unchanged).
__global__ __launch_bounds__(256)
void chain_reduce_kernel(const float* __restrict__ partial, float* __restrict__ lora_act, int M, int r,
                         int tiles) {
  const size_t n = (size_t)M * r;   // a multiple of 16 (r % 16 == 0)
  for (size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4; e < n; e += (size_t)gridDim.x * 256 * 4) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    int t = 0;
    for (; t + 8 <= tiles; t += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4*>(partial + (size_t)(t + u) * n + e);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        s.x += v[u].x;
        s.y += v[u].y;
        s.z += v[u].z;
        s.w += v[u].w;
      }
    }
    for (; t < tiles; ++t) {
      const float4 v = *reinterpret_cast<const float4*>(partial + (size_t)t * n + e);
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    *reinterpret_cast<float4*>(lora_act + e) = s;
  }
}

hipError_t launch_chain_reduce(int M, int r, int tiles, const float* partial, float* lora_act,
                               hipStream_t st) {
  const size_t n4 = (size_t)M * r / 4;
  const int grid = (int)std::min<size_t>((n4 + 255) / 256, 2048);
  hipLaunchKernelGGL(chain_reduce_kernel, dim3(grid), dim3(256), 0, st, partial, lora_act, M, r, tiles);
  return hipGetLastError();
}

template <int IO, int FMT, int EPI, int WM, int WN, int STAGES>
static hipError_t launch_cfg(int M, int N, int K, int r, const uint8_t* ac, const void* as,
                             const void* la, const uint8_t* wc, const void* ws, const void* lu,
                             const void* bias, void* Y, hipStream_t st, const QkvEpilogue& qe,
                             const ChainEpilogue& ce, const SplitK& sk = SplitK{nullptr, 1}) {
  using S = GemmShape<WM, WN, STAGES>;
  auto kern = gemm_w4a4_kernel<IO, FMT, EPI, WM, WN, STAGES>;
  if (S::LDS > 65536) {
    static std::atomic<uint64_t> raised{0};
    const hipError_t e = raise_lds_limit(raised, reinterpret_cast<const void*>(kern), S::LDS);
    if (e != hipSuccess) return e;
  }
  const int ntiles = ((M + S::BM - 1) / S::BM) * (N / S::BN);
  hipLaunchKernelGGL(kern, dim3(ntiles * (EPI == 4 ? sk.splits : 1)), dim3(256), S::LDS, st, ac, as,
                     (const float*)la, wc, ws, (const uint16_t*)lu, (const uint16_t*)bias, (uint16_t*)Y, M, N,
                     K, r, qe, ce, sk);
  return hipGetLastError();
}

template <int IO>
static hipError_t launch_gemm_io(int fmt, int M, int N, int K, int r, const uint8_t* ac, const void* as,
                                 const void* la, const uint8_t* wc, const void* ws, const void* lu,
                                 const void* bias, int epi, void* Y, hipStream_t st,
                                 const QkvEpilogue* qkv, const ChainEpilogue* chain) {
  const QkvEpilogue qe = qkv ? *qkv : QkvEpilogue{nullptr, nullptr, 0.f, 1};
  const ChainEpilogue ce = chain ? *chain : ChainEpilogue{nullptr, nullptr, 0, nullptr, nullptr, nullptr};
#define SVDQ_GO(F, E, WM_, WN_, ST_) \
  return launch_cfg<IO, F, E, WM_, WN_, ST_>(M, N, K, r, ac, as, la, wc, ws, lu, bias, Y, st, qe, ce)
  // INT4 tile size by how many 128 x 128 tiles the problem has: with fewer than
  // one per CU, 64 x 64 tiles; with fewer than two, 64 x 128; else 128 x 128 (up
  // to three workgroups per CU run at once). The arithmetic of an output is the
  // same in every shape. (The 4-bit float path keeps 128 x 128: its smaller
  // tiles measured slower.)
  const int t128 = ((M + 127) / 128) * (N / 128);
  const int small = t128 < 256 ? 2 : t128 < 512 ? 1 : 0;
  if (epi == 2) {   // fused QKV epilogue: INT4 only, one 128-channel head per tile
    if (fmt != 0 || !qkv) return hipErrorInvalidValue;
    if (small) SVDQ_GO(0, 2, 1, 2, 3);
    SVDQ_GO(0, 2, 2, 2, 3);
  }
  if (epi == 3) {   // fused MLP chain
    if (!chain) return hipErrorInvalidValue;
    if (fmt == 0) SVDQ_GO(0, 3, 2, 2, 3);
    const hipError_t e = launch_gemm_fp4_big(IO, M, N, K, r, ac, as, la, wc, ws, lu, bias, 3, Y, st, chain);
    if (e != hipErrorNotSupported) return e;
    SVDQ_GO(1, 3, 2, 2, 4);
  }
  if (fmt == 0) {
    if (small == 2) {
      if (epi == 0) SVDQ_GO(0, 0, 1, 1, 3); else SVDQ_GO(0, 1, 1, 1, 3);
    }
    if (small == 1) {
      if (epi == 0) SVDQ_GO(0, 0, 1, 2, 3); else SVDQ_GO(0, 1, 1, 2, 3);
    }
    if (epi == 0) SVDQ_GO(0, 0, 2, 2, 3); else SVDQ_GO(0, 1, 2, 2, 3);
  } else {
    const hipError_t e = launch_gemm_fp4_big(IO, M, N, K, r, ac, as, la, wc, ws, lu, bias, epi, Y, st);
    if (e != hipErrorNotSupported) return e;
    if (epi == 0) SVDQ_GO(1, 0, 2, 2, 4); else SVDQ_GO(1, 1, 2, 2, 4);
  }
#undef SVDQ_GO
}

// Y[m][n] = act(sum_s part[s][m][n] * 2^-8 + bias[n]), the slices added in
// split order (deterministic); the same epilogue arithmetic as the unsplit
// kernel. 8 consecutive outputs per thread (16-byte loads and stores).
template <int IO, int ACT>
__global__ __launch_bounds__(256)
void splitk_reduce_kernel(const float* __restrict__ part, int S, const uint16_t* __restrict__ bias,
                          uint16_t* __restrict__ Y, int M, int N) {
  const size_t mn = (size_t)M * N;
  for (size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8; e < mn; e += (size_t)gridDim.x * 256 * 8) {
    float4 a = *reinterpret_cast<const float4*>(part + e);
    float4 b = *reinterpret_cast<const float4*>(part + e + 4);
    for (int t = 1; t < S; ++t) {
      const float4 c = *reinterpret_cast<const float4*>(part + (size_t)t * mn + e);
      const float4 d = *reinterpret_cast<const float4*>(part + (size_t)t * mn + e + 4);
      a.x += c.x; a.y += c.y; a.z += c.z; a.w += c.w;
      b.x += d.x; b.y += d.y; b.z += d.z; b.w += d.w;
    }
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    const int n = (int)(e % (size_t)N);
    uint16_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float y = fmaf(v[j], 0.00390625f, bias ? Io<IO>::to_f(bias[n + j]) : 0.f);   // exact 2^-8, then + bias
      if (ACT) y = gelu_tanh_f32(y);
      o[j] = Io<IO>::from_f(y);
    }
    *reinterpret_cast<uint4*>(Y + e) = make_uint4(o[0] | ((uint32_t)o[1] << 16), o[2] | ((uint32_t)o[3] << 16),
                                                  o[4] | ((uint32_t)o[5] << 16), o[6] | ((uint32_t)o[7] << 16));
  }
}

int splitk_splits(int fmt, int M, int N, int K) {
  // INT4 only, and only where 128 x 128 tiles fill fewer than 256 workgroups:
  // K is cut into S (a power of two) runs while S tiles' worth of workgroups
  // fit in the 768 slots (three per CU) and each run keeps at least 8 steps
  if (fmt != 0 || N % 128 != 0) return 1;
  const long long t128 = (long long)((M + 127) / 128) * (N / 128);
  if (t128 >= 256) return 1;
  const int nk = K >> 7;
  int S = 1;
  while (t128 * S * 2 <= 768 && nk / (S * 2) >= 8) S *= 2;
  return S;
}

size_t splitk_bytes(int fmt, int M, int N, int K) {
  const int S = splitk_splits(fmt, M, N, K);
  return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

template <int IO>
static hipError_t launch_split_io(int M, int N, int K, int r, int S, const uint8_t* ac, const void* as,
                                  const void* la, const uint8_t* wc, const void* ws, const void* lu,
                                  const void* bias, int epi, void* Y, float* part, hipStream_t st) {
  const QkvEpilogue qe{nullptr, nullptr, 0.f, 1};
  const ChainEpilogue ce{nullptr, nullptr, 0, nullptr, nullptr, nullptr};
  hipError_t e = launch_cfg<IO, 0, 4, 2, 2, 3>(M, N, K, r, ac, as, la, wc, ws, lu, bias, Y, st, qe, ce,
                                              SplitK{part, S});
  if (e != hipSuccess) return e;
  const size_t n8 = (size_t)M * N / 8;
  const int grid = (int)std::min<size_t>((n8 + 255) / 256, 4096);
  if (epi == 1)
    hipLaunchKernelGGL((splitk_reduce_kernel<IO, 1>), dim3(grid), dim3(256), 0, st, part, S,
                       (const uint16_t*)bias, (uint16_t*)Y, M, N);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<IO, 0>), dim3(grid), dim3(256), 0, st, part, S,
                       (const uint16_t*)bias, (uint16_t*)Y, M, N);
  return hipGetLastError();
}

hipError_t launch_gemm_w4a4_split(int fmt, int io, int M, int N, int K, int r, const uint8_t* ac, const void* as,
                                  const void* la, const uint8_t* wc, const void* ws, const void* lu,
                                  const void* bias, int epi, void* Y, void* workspace, size_t workspace_bytes,
                                  hipStream_t st) {
  const int S = splitk_splits(fmt, M, N, K);
  if (S <= 1 || workspace == nullptr || workspace_bytes < splitk_bytes(fmt, M, N, K))
    return launch_gemm_w4a4(fmt, io, M, N, K, r, ac, as, la, wc, ws, lu, bias, epi, Y, st);
  float* part = static_cast<float*>(workspace);
  if (io == 1) return launch_split_io<1>(M, N, K, r, S, ac, as, la, wc, ws, lu, bias, epi, Y, part, st);
  return launch_split_io<0>(M, N, K, r, S, ac, as, la, wc, ws, lu, bias, epi, Y, part, st);
}

int chain_tile_n(int fmt, int M, int N, int K) { return (fmt != 0 && fp4_big_fits(M, N, K)) ? 256 : 128; }

hipError_t launch_gemm_w4a4(int fmt, int io, int M, int N, int K, int r, const uint8_t* ac, const void* as,
                            const void* la, const uint8_t* wc, const void* ws, const void* lu,
                            const void* bias, int epi, void* Y, hipStream_t st, const QkvEpilogue* qkv,
                            const ChainEpilogue* chain) {
  if (io == 1) return launch_gemm_io<1>(fmt, M, N, K, r, ac, as, la, wc, ws, lu, bias, epi, Y, st, qkv, chain);
  return launch_gemm_io<0>(fmt, M, N, K, r, ac, as, la, wc, ws, lu, bias, epi, Y, st, qkv, chain);
}

}  // namespace svdq
