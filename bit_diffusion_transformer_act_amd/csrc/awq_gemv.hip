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
// accumulates x (B + q) in fp32 against x stored as pairs (x_j, x_{j+4}). Per
// 32-code chunk, sum x (q - z) = sum x (B + q) - (B + z) sum x, with the second
// term one fma from the precomputed chunk sum of x, so any fp16 zero point
// works. Scales and zero points are fp16 in both cases (the stored format).
//
// Work split: one 8-wave workgroup per CU; wave w of the grid owns the
// contiguous rows [w N / W, (w + 1) N / W) (W waves in all), so every CU streams
// the same number of bytes. The rows of a wave are contiguous in memory and
// are read as a stream of units of 64 chunks of 16 bytes (lane l takes chunk
// l of the unit): each load instruction covers 1 KB of whole cache lines, and
// a ring of units keeps several in flight. Where a row is an odd number of
// 32-chunk halves (K = 3072, for one), rows go in pairs, one per half-wave, so
// that no unit is half empty. x and its chunk sums sit in LDS. A
// row's lane partials are summed with lane swaps and DPP at its last unit.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace svdq {

constexpr int kGemvWaves = 8;   // waves per workgroup
constexpr int kGemvRing = 6;    // units in flight per wave

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
template <int IO, int MR, bool PAIRS>
__global__ __launch_bounds__(64 * kGemvWaves)
void awq_gemv_kernel(const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes,
                     const __half* __restrict__ scales, const __half* __restrict__ zeros,
                     const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int N, int K) {
  // 1.0 as a pair, and the exact offset B of the dequantization trick with its bit pattern
  constexpr uint32_t kOne = IO == 1 ? 0x3F803F80u : 0x3C003C00u;
  constexpr uint32_t kMagic = IO == 1 ? 0x43004300u : 0x64006400u;
  constexpr float kB = IO == 1 ? 128.0f : 1024.0f;
  // LDS: x pairs as [m][4 segments of a chunk][chunk][4 pairs] (for a fixed
  // segment, consecutive chunks are 16 bytes apart: conflict-free reads), then
  // the chunk sums of x [m][chunk]
  extern __shared__ uint32_t lds[];
  const int nch = K >> 5;                 // 32-code chunks per row (16 bytes each)
  const int G = K >> 6;
  uint32_t* xs = lds;
  float* xc = reinterpret_cast<float*>(lds + (size_t)MR * nch * 16);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const long long W = (long long)gridDim.x * kGemvWaves;
  const long long wg = (long long)blockIdx.x * kGemvWaves + wave;
  const int r0 = (int)(wg * N / W), r1 = (int)((wg + 1) * N / W);
  constexpr int UL = PAIRS ? 32 : 64;      // chunks of a row per unit
  const int ul = PAIRS ? (lane & 31) : lane;
  const int hl = PAIRS ? (lane >> 5) : 0;   // PAIRS: the half's row within its pair
  const int nseg = (nch + UL - 1) / UL;     // units per row (per pair of rows)
  const int nrow = max(r1 - r0, 0);
  const int nunits = (PAIRS ? (nrow + 1) >> 1 : nrow) * nseg;

  struct Unit {
    uint4 w;
    __half s, z;
  };
  // Loads are unconditional: past the wave's last unit they re-read it (never
  // processed), so the compiler's count of loads in flight stays exact; the odd
  // half of a last pair with one row re-reads that row (its total is never stored).
  int lrow = 0, lseg = 0;   // row (PAIRS: pair) of the wave and unit within it
  auto load_next = [&](Unit& d) {
    // a wave with no rows re-reads row 0
    const int row = max(min(r0 + (PAIRS ? 2 * lrow + hl : lrow), r1 - 1), 0);
    const int c = min(lseg * UL + ul, nch - 1);
    d.w = *reinterpret_cast<const uint4*>(codes + (size_t)row * (K >> 1) + (size_t)c * 16);
    d.s = scales[(size_t)row * G + (c >> 1)];
    d.z = zeros[(size_t)row * G + (c >> 1)];
    if (++lseg == nseg) {
      lseg = 0;
      ++lrow;
    }
  };

  // the weight stream starts before x is staged, so its first latency overlaps the staging
  Unit d[kGemvRing];
#pragma unroll
  for (int i = 0; i < kGemvRing - 1; ++i) load_next(d[i]);

  for (int idx = tid; idx < MR * nch * 4; idx += 64 * kGemvWaves) {
    // idx = (m nch + c) 4 + e: segment e of chunk c = channels 32 c + 8 e .. +8
    const int e = idx & 3, mc = idx >> 2;
    const int m = mc / nch, c = mc - m * nch;
    const uint4 v = *reinterpret_cast<const uint4*>(x + (size_t)m * K + (size_t)c * 32 + e * 8);
    uint32_t* o = xs + (((size_t)m * 4 + e) * nch + c) * 4;
    o[0] = (v.x & 0xFFFFu) | (v.z << 16);          // (x_0, x_4)
    o[1] = (v.x >> 16) | (v.z & 0xFFFF0000u);      // (x_1, x_5)
    o[2] = (v.y & 0xFFFFu) | (v.w << 16);          // (x_2, x_6)
    o[3] = (v.y >> 16) | (v.w & 0xFFFF0000u);      // (x_3, x_7)
  }
  __syncthreads();
  for (int mc = tid; mc < MR * nch; mc += 64 * kGemvWaves) {
    const int m = mc / nch, c = mc - m * nch;
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sum = dot2_io<IO>(xs[(((size_t)m * 4 + e) * nch + c) * 4 + j], kOne, sum);
    xc[mc] = sum;
  }
  __syncthreads();

  if (r1 <= r0) return;

  // Row totals are collected in registers (row i of the wave in lane i; the
  // grid gives no wave more than 64 rows) and written after the loop: a store
  // on one path only would leave the compiler unsure how many loads are in
  // flight and drain the ring at every row.
  float acc[MR], out[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) acc[m] = out[m] = 0.f;
  int prow = 0, pseg = 0;   // row (PAIRS: pair) of the wave and unit within it
  auto process = [&](const Unit& d) {
    const int c = pseg * UL + ul;
    if (c < nch) {
      const uint32_t w[4] = {d.w.x, d.w.y, d.w.z, d.w.w};
      const float s = __half2float(d.s);
      const float zb = kB + __half2float(d.z);
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint4 xp = *reinterpret_cast<const uint4*>(xs + (((size_t)m * 4 + e) * nch + c) * 4);
          const uint32_t xv[4] = {xp.x, xp.y, xp.z, xp.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t hb = ((w[e] >> (4 * j)) & 0x000F000Fu) | kMagic;
            part = dot2_io<IO>(hb, xv[j], part);
          }
        }
        acc[m] = fmaf(s, fmaf(-zb, xc[m * nch + c], part), acc[m]);
      }
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
      if (u0 + i < nunits) process(d[i]);
    }
  }
  if (lane < r1 - r0) {
    const float b = bias ? Io<IO>::to_f(bias[r0 + lane]) : 0.f;
#pragma unroll
    for (int m = 0; m < MR; ++m) y[(size_t)m * N + r0 + lane] = Io<IO>::from_f(out[m] + b);
  }
}

template <int IO, int MR, bool PAIRS>
static hipError_t launch_k(int N, int K, const void* x, const uint8_t* q, const void* s,
                           const void* z, const void* b, void* y, hipStream_t st) {
  // about one workgroup per CU for large N, at least ~4 rows per wave for small
  // N, and never more than 64 rows per wave (the kernel keeps one row per lane)
  const int rows_cap = kGemvWaves * 64;
  const int grid = max(max(1, min(256, (N + 8 * 4 - 1) / (8 * 4))), (N + rows_cap - 1) / rows_cap);
  const size_t lds = (size_t)MR * (K >> 5) * 16 * sizeof(uint32_t) + (size_t)MR * (K >> 5) * sizeof(float);
  if (lds > 65536) {   // M K = 32768 needs 68 KB
    static std::atomic<uint64_t> raised{0};
    const hipError_t e =
        raise_lds_limit(raised, reinterpret_cast<const void*>(&awq_gemv_kernel<IO, MR, PAIRS>), 72 * 1024);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((awq_gemv_kernel<IO, MR, PAIRS>), dim3(grid), dim3(64 * kGemvWaves), lds, st,
                     (const uint16_t*)x, q, (const __half*)s, (const __half*)z, (const uint16_t*)b, (uint16_t*)y,
                     N, K);
  return hipGetLastError();
}

template <int IO, int MR>
static hipError_t launch_mr(int N, int K, const void* x, const uint8_t* q, const void* s,
                            const void* z, const void* b, void* y, hipStream_t st) {
  // rows of an odd number of 32-chunk halves go in pairs (whole 1 KB loads)
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
