// awq_gemv_w4a16: 4-bit weights, 16-bit activations, for the memory-bound
// modulation / adaptive-norm projections (dothoosh.com "How Nunchaku Lite
// halves diffusion-model VRAM", kernel-family list, the awq_w4a16 entry;
// int4 with group size 64 in the quantization_config block).
//
//   y[m,n] = sum_k x[m,k] (q[n,k] - z[n,g]) s[n,g],  g = k / 64
//
// HBM-bound: every weight byte is read once. Dequantization uses a bit trick
// in the activations' 16-bit type: (word >> 4j) & 0x000F000F | 0x64006400 is
// the packed fp16 pair (1024 + q_j, 1024 + q_{j+4}) and | 0x43004300 the bf16
// pair (128 + q_j, 128 + q_{j+4}), both exact, and v_dot2_f32_f16 / _bf16
// accumulates x (B + q) in fp32 against x stored as pairs (x_j, x_{j+4}). In
// fp16 the odd pairs skip the shift: word & 0x00F000F0 | 0x64006400 is
// (1024 + 16 q_j, 1024 + 16 q_{j+4}), exact, and their products go to a second
// accumulator that enters at 1/16 (exact). Per 32-code chunk,
// sum x (q - z) = P - D - z S, with P the accumulators' total, D the chunk's
// share of the offsets (1024 x for the even pairs and 64 x for the odd ones in
// fp16; 128 x in bf16) and S = sum x, both precomputed once per chunk; so any
// fp16 zero point works. Scales and zero points are fp16 in both cases (the
// stored format).
//
// Work split: one 8-wave workgroup per CU; wave w of the grid (W waves in all)
// owns rows w, w + W, w + 2W, ... (in pairs: see below), so at any moment the
// grid reads one contiguous window of the matrix, and every CU streams the
// same number of bytes. A row is read as a stream of units of 64 chunks of 16
// bytes (lane l takes chunk l of the unit): each load instruction covers 1 KB
// of whole cache lines, and a ring of three units keeps two in flight. Where a
// row is an odd number of 32-chunk halves (K = 3072, for one), rows go in
// pairs, one per half-wave, so that no unit is half empty. x and its chunk sums
// sit in LDS. A row's lane partials are summed with lane swaps and DPP at its
// last unit.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace svdq {

constexpr int kGemvWaves = 8;   // waves per workgroup
// units in the register ring of a wave (two in flight while one is processed):
// the fastest of the depths 2 to 10 measured (K3072 N18432: 3 -> 11.9 us,
// 4 -> 12.3, 6 -> 13.3, 8 -> 14.3; at M4 18.8 against 23.1 with 6)
constexpr int kGemvRing = 3;

// Sum over the 64 lanes; every lane gets the same total (a fixed order: the
// xor-32 and xor-16 partners via v_permlane32/16_swap, then within each 16-lane
// row the mirror, half-mirror and two quad permutations of DPP).
__device__ __forceinline__ float wave_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  return v;
}

// Sum over each 32-lane half; every lane gets its half's total (the xor-16
// partner, then the DPP steps of wave_sum).
__device__ __forceinline__ float half_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  return v;
}

// dot2 of packed 16-bit pairs in the activations' type, fp32 accumulation
template <int IO>
__device__ __forceinline__ float dot2_io(uint32_t a, uint32_t b, float c) {
  if constexpr (IO == 1)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a), __builtin_bit_cast(v2bf, b), c, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(v2h, a), __builtin_bit_cast(v2h, b), c, false);
}

// PAIRS: a row is an odd number of 32-chunk halves (K = 1024 x odd), so
// 64-chunk units would leave every other load half empty. The wave's rows then
// go in pairs, the even row of a pair in lanes 0-31 and the odd one in lanes
// 32-63, in units of 32 chunks per half: every load is a whole 1 KB.
// XR (M 1, K 3072: rows in pairs, three units per pair, as many as the ring
// holds): ring slot i always carries unit i of a pair, so each lane keeps the x
// pairs and (D, S) of its three chunks in registers instead of reading them
// from LDS per unit.
template <int IO, int MR, bool PAIRS, bool XR>
__global__ __launch_bounds__(64 * kGemvWaves)
void awq_gemv_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes,
                     const __half* __restrict__ scales, const __half* __restrict__ zeros,
                     const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int N, int K) {
  // 1.0 as a pair, and the pair (B, B) of the dequantization trick's exact offset
  constexpr uint32_t kOne = IO == 1 ? 0x3F803F80u : 0x3C003C00u;
  constexpr uint32_t kMagic = IO == 1 ? 0x43004300u : 0x64006400u;
  // LDS: x pairs as [m][chunk group of 16][4 segments of a chunk][16 chunks][4
  // pairs] (for a fixed segment, the 16 chunks of a group are 16 bytes apart:
  // conflict-free 16-byte reads; a lane's four segments are 256 bytes apart, one
  // address and three immediate offsets), then each chunk's (D, S) [m][chunk][2].
  // Both are padded to whole units of the row (npad chunks; the padding holds
  // zeros and only feeds results that are discarded).
  extern __shared__ uint32_t lds[];
  const int nch = K >> 5;                 // 32-code chunks per row (16 bytes each)
  const int G = K >> 6;
  const int KB = K >> 1;                  // code bytes per row
  constexpr int UL = PAIRS ? 32 : 64;     // chunks of a row per unit
  const int nseg = (nch + UL - 1) / UL;   // units per row (per pair of rows)
  const int npad = nseg * UL;             // chunks per row in LDS
  const bool full = npad == nch;          // no unit reaches past the row's end
  uint32_t* xs = lds;
  float* xc = reinterpret_cast<float*>(lds + (size_t)MR * npad * 16);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long W = (long long)gridDim.x * kGemvWaves;
  const long long wg = (long long)blockIdx.x * kGemvWaves + wave;
  const int ul = PAIRS ? (lane & 31) : lane;
  const bool hl = PAIRS && lane >= 32;    // PAIRS: the odd row of the pair
  // the wave's row groups (PAIRS: pairs of rows) are wg, wg + W, wg + 2W, ...
  constexpr int RG = PAIRS ? 2 : 1;
  const long long ngrp = ((long long)N + RG - 1) / RG;
  const int ng = wg < ngrp ? (int)((ngrp - wg + W - 1) / W) : 0;
  const int nunits = ng * nseg;

  struct Unit {
    uint4 w;
    __half s, z;
  };
  // Loads are unconditional: past the wave's last unit they re-read it (never
  // processed), so the compiler's count of loads in flight stays exact; the odd
  // half of a last pair with one row re-reads that row (its total is never
  // stored). The row and unit offsets are wave-uniform (scalar base address);
  // a lane adds its chunk and, for the odd half of a pair, one row.
  int lrow = 0, lseg = 0;   // row group of the wave and unit within it
  auto load_next = [&](Unit& d) {
    // a wave with no rows re-reads row 0
    const int gi = max(min(lrow, ng - 1), 0);
    const int ra = ng > 0 ? (int)(((long long)gi * W + wg) * RG) : 0;
    const int rb = PAIRS ? min(ra + 1, N - 1) : ra;
    const int c0 = lseg * UL;
    const int cl = full ? ul : min(ul, nch - 1 - c0);   // the lane's chunk within the unit
    const bool odd = hl && rb != ra;
    const uint8_t* cb = codes + (size_t)ra * KB + (size_t)c0 * 16;
    const __half* sb = scales + (size_t)ra * G + (c0 >> 1);
    const __half* zb = zeros + (size_t)ra * G + (c0 >> 1);
    d.w = *reinterpret_cast<const uint4*>(cb + (uint32_t)((odd ? KB : 0) + cl * 16));
    const uint32_t so = (uint32_t)((odd ? G : 0) + (cl >> 1)) * 2u;   // byte offset
    d.s = *reinterpret_cast<const __half*>(reinterpret_cast<const uint8_t*>(sb) + so);
    d.z = *reinterpret_cast<const __half*>(reinterpret_cast<const uint8_t*>(zb) + so);
    if (++lseg == nseg) {
      lseg = 0;
      ++lrow;
    }
  };

  // the weight stream starts before x is staged, so its first latency overlaps the staging
  Unit d[kGemvRing];
#pragma unroll
  for (int i = 0; i < kGemvRing - 1; ++i) load_next(d[i]);

  for (int idx = tid; idx < MR * npad * 4; idx += 64 * kGemvWaves) {
    // idx = (m npad + c) 4 + e: segment e of chunk c = channels 32 c + 8 e .. +8
    const int e = idx & 3, mc = idx >> 2;
    const int m = mc / npad, c = mc - m * npad;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (c < nch) v = *reinterpret_cast<const uint4*>(x + (size_t)m * K + (size_t)c * 32 + e * 8);
    uint32_t* o = xs + (((size_t)m * npad + (c & ~15)) * 4 + e * 16 + (c & 15)) * 4;
    o[0] = (v.x & 0xFFFFu) | (v.z << 16);          // (x_0, x_4)
    o[1] = (v.x >> 16) | (v.z & 0xFFFF0000u);      // (x_1, x_5)
    o[2] = (v.y & 0xFFFFu) | (v.w << 16);          // (x_2, x_6)
    o[3] = (v.y >> 16) | (v.w & 0xFFFF0000u);      // (x_3, x_7)
  }
  __syncthreads();
  for (int mc = tid; mc < MR * npad; mc += 64 * kGemvWaves) {
    // the chunk's D (the offsets' share: B x, or (B / 16) x for fp16's odd
    // pairs, which enter at 1/16) and S = sum x
    const int m = mc / npad, c = mc - m * npad;
    constexpr uint32_t k64 = 0x54005400u;   // (64, 64) in fp16
    float dsum = 0.f, ssum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t pr = xs[(((size_t)m * npad + (c & ~15)) * 4 + e * 16 + (c & 15)) * 4 + j];
        dsum = dot2_io<IO>(pr, (IO == 0 && (j & 1)) ? k64 : kMagic, dsum);
        ssum = dot2_io<IO>(pr, kOne, ssum);
      }
    xc[2 * mc] = dsum;
    xc[2 * mc + 1] = ssum;
  }
  __syncthreads();

  if (ng == 0) return;

  // Row totals are collected in registers (the wave's i-th row in lane i; the
  // grid gives no wave more than 64 rows) and written after the loop: a store
  // on one path only would leave the compiler unsure how many loads are in
  // flight and drain the ring at every row.
  float acc[MR], out[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = out[m] = 0.f;
  // the dequantization constants live in registers, so that (w & mask) | magic
  // is one v_and_or_b32
  uint32_t kmask = 0x000F000Fu, kmask1 = 0x00F000F0u, kmag = kMagic;
  asm volatile("" : "+v"(kmask), "+v"(kmask1), "+v"(kmag));
  // this lane's LDS words: x pairs of chunk ul (segment e at +64 e words), its (D, S)
  const uint32_t* xl = xs + ((size_t)(ul & ~15) * 4 + (ul & 15)) * 4;
  const float2* xcl = reinterpret_cast<const float2*>(xc) + ul;
  int prow = 0, pseg = 0;   // row group of the wave and unit within it
  static_assert(!XR || (MR == 1 && PAIRS && kGemvRing == 3), "XR: one row of x, pairs, three ring slots");
  uint4 xr[XR ? 3 : 1][4];
  float2 dsr[XR ? 3 : 1];
  if constexpr (XR) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) xr[u][e] = *reinterpret_cast<const uint4*>(xl + (size_t)u * UL * 16 + e * 64);
      dsr[u] = xcl[u * UL];
    }
  }
  // slot: the ring slot of the unit (XR: its unit within the pair)
  auto process = [&](const Unit& d, int slot) {
    const int c0 = pseg * UL;
    const bool valid = full || c0 + ul < nch;
    const uint32_t w[4] = {d.w.x, d.w.y, d.w.z, d.w.w};
    const float s = __half2float(d.s);
    const float z = __half2float(d.z);
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const uint32_t* xm = xl + ((size_t)m * npad + c0) * 16;
      float part = 0.f, part16 = 0.f;   // part16: fp16's odd pairs, at 16 times their weight
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint4 xp = XR ? xr[slot][e] : *reinterpret_cast<const uint4*>(xm + e * 64);
        const uint32_t xv[4] = {xp.x, xp.y, xp.z, xp.w};
        if constexpr (IO == 0) {
          // pairs 1 and 3 keep their codes at bits 4-7 of each half: 1024 + 16 q
          const uint32_t w8 = w[e] >> 8;
          part = dot2_io<IO>((w[e] & kmask) | kmag, xv[0], part);
          part16 = dot2_io<IO>((w[e] & kmask1) | kmag, xv[1], part16);
          part = dot2_io<IO>((w8 & kmask) | kmag, xv[2], part);
          part16 = dot2_io<IO>((w8 & kmask1) | kmag, xv[3], part16);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) part = dot2_io<IO>(((w[e] >> (4 * j)) & kmask) | kmag, xv[j], part);
        }
      }
      const float2 ds = XR ? dsr[slot] : xcl[(size_t)m * npad + c0];
      const float tot = IO == 0 ? fmaf(part16, 0.0625f, part) : part;
      const float t = fmaf(s, fmaf(-z, ds.y, tot - ds.x), acc[m]);
      acc[m] = valid ? t : acc[m];
    }
    if (++pseg == nseg) {   // the row (PAIRS: the pair) is complete
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        if constexpr (PAIRS) {
          // each half's total, then both in every lane: the even row's from the
          // low half, the odd row's from the high half
          const float t = half_sum(acc[m]);
          const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
          const int slot = 2 * prow;
          out[m] = (lane == slot) ? __uint_as_float(h[0]) : (lane == slot + 1) ? __uint_as_float(h[1]) : out[m];
        } else {
          const float t = wave_sum(acc[m]);
          out[m] = (lane == prow) ? t : out[m];
        }
        acc[m] = 0.f;
      }
      pseg = 0;
      ++prow;
    }
  };

  for (int u0 = 0; u0 < nunits; u0 += kGemvRing) {
#pragma unroll
    for (int i = 0; i < kGemvRing; ++i) {
      load_next(d[(i + kGemvRing - 1) % kGemvRing]);
      if (u0 + i < nunits) process(d[i], i);
    }
  }
  {
    // lane i holds the total of the wave's i-th row (PAIRS: lanes 2i, 2i + 1 the rows of its i-th pair)
    const int gi = PAIRS ? (lane >> 1) : lane;
    const long long row = ((long long)gi * W + wg) * RG + (PAIRS ? (lane & 1) : 0);
    if (gi < ng && row < N) {
      const float b = bias ? Io<IO>::to_f(bias[row]) : 0.f;
#pragma unroll
      for (int m = 0; m < MR; ++m) y[(size_t)m * N + row] = Io<IO>::from_f(out[m] + b);
    }
  }
}

template <int IO, int MR, bool PAIRS, bool XR = false>
static hipError_t launch_k(int N, int K, const void* x, const uint8_t* q, const void* s,
                           const void* z, const void* b, void* y, hipStream_t st) {
  // about one workgroup per CU for large N, at least ~4 rows per wave for small
  // N, and never more than 64 rows per wave (the kernel keeps one row per lane)
  const int rows_cap = kGemvWaves * 64;
  const int grid = max(max(1, min(256, (N + 8 * 4 - 1) / (8 * 4))), (N + rows_cap - 1) / rows_cap);
  constexpr int UL = PAIRS ? 32 : 64;
  const size_t npad = (size_t)((K >> 5) + UL - 1) / UL * UL;   // chunks per row in LDS, whole units
  const size_t lds = (size_t)MR * npad * 16 * sizeof(uint32_t) + (size_t)MR * npad * 2 * sizeof(float);
  if (lds > 65536) {   // at most 96768 bytes (M 7, K 4160: 130 chunks padded to 192)
    static std::atomic<uint64_t> raised{0};
    const hipError_t e =
        raise_lds_limit(raised, reinterpret_cast<const void*>(&awq_gemv_kernel<IO, MR, PAIRS, XR>), 96 * 1024);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((awq_gemv_kernel<IO, MR, PAIRS, XR>), dim3(grid), dim3(64 * kGemvWaves), lds, st,
                     (const uint16_t*)x, q, (const __half*)s, (const __half*)z, (const uint16_t*)b, (uint16_t*)y,
                     N, K);
  return hipGetLastError();
}

template <int IO, int MR>
static hipError_t launch_mr(int N, int K, const void* x, const uint8_t* q, const void* s,
                            const void* z, const void* b, void* y, hipStream_t st) {
  // rows of an odd number of 32-chunk halves go in pairs (whole 1 KB loads);
  // one row of x at K 3072 keeps x in registers
  if constexpr (MR == 1)
    if (K == 3072) return launch_k<IO, 1, true, true>(N, K, x, q, s, z, b, y, st);
  if (((K >> 5) & 63) == 32) return launch_k<IO, MR, true>(N, K, x, q, s, z, b, y, st);
  return launch_k<IO, MR, false>(N, K, x, q, s, z, b, y, st);
}

template <int IO>
static hipError_t launch_gemv_io(int M, int N, int K, const void* x, const uint8_t* q, const void* s,
                                 const void* z, const void* b, void* y, hipStream_t st) {
  switch (M) {
    case 1: return launch_mr<IO, 1>(N, K, x, q, s, z, b, y, st);
    case 2: return launch_mr<IO, 2>(N, K, x, q, s, z, b, y, st);
    case 3: return launch_mr<IO, 3>(N, K, x, q, s, z, b, y, st);
    case 4: return launch_mr<IO, 4>(N, K, x, q, s, z, b, y, st);
    case 5: return launch_mr<IO, 5>(N, K, x, q, s, z, b, y, st);
    case 6: return launch_mr<IO, 6>(N, K, x, q, s, z, b, y, st);
    case 7: return launch_mr<IO, 7>(N, K, x, q, s, z, b, y, st);
    default: return launch_mr<IO, 8>(N, K, x, q, s, z, b, y, st);
  }
}

hipError_t launch_awq_gemv(int io, int M, int N, int K, const void* x, const uint8_t* q, const void* s,
                           const void* z, const void* b, void* y, hipStream_t st) {
  if (io == 1) return launch_gemv_io<1>(M, N, K, x, q, s, z, b, y, st);
  return launch_gemv_io<0>(M, N, K, x, q, s, z, b, y, st);
}

}  // namespace svdq
