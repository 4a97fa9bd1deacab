// Kernel launchers behind the C ABI (arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace svdq {

// Raises a kernel's dynamic LDS limit to `bytes` on the current device, once
// per device and call site: the attribute belongs to the device that is
// current when it is set, so `done` keeps one bit per device id (ids past 63
// set it on every call).
inline hipError_t raise_lds_limit(std::atomic<uint64_t>& done, const void* kern, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// io: 16-bit type of activations, low-rank branch, biases and outputs (0 fp16, 1 bf16)
// fmt 0 INT4 g64, 1 FP4 E2M1 b32, 2 NVFP4 (gscale: the per-tensor scale)
hipError_t launch_quantize_act(int fmt, int io, int M, int K, int r, const void* X, const float* smooth_inv,
                               const void* lora_down, uint8_t* codes, void* scales, void* lora_act,
                               hipStream_t stream, float gscale = 1.0f);

// Parameters of the fused QKV epilogue (epi == 2): per-head RMSNorm of the Q
// and K thirds of the output (heads of 128 channels, `heads` per third) with
// weights qk_norm_w fp16 [2][128] and epsilon eps, then the rotation of channel
// pairs (2i, 2i+1) by rope fp32 [M][64][2] (cos, sin per token and pair).
struct QkvEpilogue {
  const void* qk_norm_w;
  const float* rope;
  float eps;
  int heads;
};

// Parameters of the fused MLP chain (epi == 3, INT4 or FP4 up-projection):
// GELU, then the down-projection's INT4 quantizer on the 16-bit result U:
// smoothing by smooth_inv [N], INT4 g64 codes [M][N/2] and fp16 scales
// [M][N/64], and the per-tile fp32 partials of U lora_down^T ([N/BN][M][r]
// with BN = chain_tile_n(...), summed by launch_chain_reduce into the fp32
// lora_act).
struct ChainEpilogue {
  const float* smooth_inv;
  const void* lora_down;
  int r;
  uint8_t* codes;
  void* scales;
  float* partial;
};

hipError_t launch_chain_reduce(int M, int r, int tiles, const float* partial, float* lora_act,
                               hipStream_t stream);

// Split K (epi == 4 of the INT4 kernel): `splits` workgroups per output tile,
// each over a contiguous run of K steps, write fp32 partials [splits][M][N]
// (256 times the sum, the low-rank start in split 0) to `part`.
struct SplitK {
  float* part;
  int splits;
};

// splits the split-K path uses for this shape (1: it does not split), and the
// bytes of fp32 partials it needs
int splitk_splits(int fmt, int M, int N, int K);
size_t splitk_bytes(int fmt, int M, int N, int K);

// launch_gemm_w4a4 (epi 0 or 1) with K split across workgroups where the shape
// has too few output tiles for the GPU; falls back to the unsplit kernel when
// the shape does not split or the workspace is smaller than splitk_bytes()
hipError_t launch_gemm_w4a4_split(int fmt, int io, int M, int N, int K, int r, const uint8_t* act_codes,
                                  const void* act_scales, const void* lora_act, const uint8_t* w_codes,
                                  const void* w_scales, const void* lora_up, const void* bias, int epi,
                                  void* Y, void* workspace, size_t workspace_bytes, hipStream_t stream);

hipError_t launch_gemm_w4a4(int fmt, int io, int M, int N, int K, int r, const uint8_t* act_codes,
                            const void* act_scales, const void* lora_act, const uint8_t* w_codes,
                            const void* w_scales, const void* lora_up, const void* bias, int epi,
                            void* Y, hipStream_t stream, const QkvEpilogue* qkv = nullptr,
                            const ChainEpilogue* chain = nullptr);

// whether the 256 x 256 FP4 kernel takes the shape (else the 128 x 128 one does)
bool fp4_big_fits(int M, int N, int K);

hipError_t launch_gemm_fp4_big(int io, int M, int N, int K, int r, const uint8_t* act_codes,
                               const void* act_scales, const void* lora_act, const uint8_t* w_codes,
                               const void* w_scales, const void* lora_up, const void* bias, int epi,
                               void* Y, hipStream_t stream, const ChainEpilogue* chain = nullptr);

// columns per slice of the fused chain's low-rank partials: the up-projection
// GEMM's tile width for this format and shape
int chain_tile_n(int fmt, int M, int N, int K);

// NVFP4 GEMM: Y = act(alpha * sum (q_x s_x)(q_w s_w) + lora_act lora_up^T + bias)
hipError_t launch_gemm_nvfp4(int io, int M, int N, int K, int r, const uint8_t* act_codes,
                             const uint8_t* act_scales, const void* lora_act, const uint8_t* w_codes,
                             const uint8_t* w_scales, const void* lora_up, const void* bias, float alpha,
                             int epi, void* Y, hipStream_t stream);

hipError_t launch_awq_gemv(int io, int M, int N, int K, const void* x, const uint8_t* codes,
                           const void* scales, const void* zeros, const void* bias, void* y,
                           hipStream_t stream);

}  // namespace svdq
