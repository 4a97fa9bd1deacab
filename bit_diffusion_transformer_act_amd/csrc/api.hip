// Host side of the C ABI: argument validation, the gfx950 capability check
// and dispatch. Nothing here allocates or synchronizes.
//
// The capability check mirrors the pages' loader, which validates the GPU
// at load time and raises a clear error instead of producing wrong output
// (dothoosh.com "How Nunchaku Lite halves diffusion-model VRAM",
// hardware-support paragraph).
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "launch.hpp"
#include "svdq.h"

namespace svdq {
// 64 MiB: the chain's partials at M 4096, N 12288, rank 32 take 50 MB
constexpr size_t kChainScratchBytes = size_t{64} << 20;
__device__ __align__(256) uint8_t scratch[kChainScratchBytes];
}  // namespace svdq

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool arch_is_gfx950(const char* name) { return name && std::strncmp(name, "gfx950", 6) == 0; }

int check_device(int dev) {
  const char* force = std::getenv("SVDQ_FORCE_ARCH");
  if (force && *force) return arch_is_gfx950(force) ? SVDQ_OK : SVDQ_ERR_UNSUPPORTED_DEVICE;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || dev < 0 || dev >= count) {
    (void)hipGetLastError();
    return SVDQ_ERR_UNSUPPORTED_DEVICE;
  }
  if (dev < kMaxDevices) {
    const int c = g_arch_ok[dev].load(std::memory_order_acquire);
    if (c == 1) return SVDQ_OK;
    if (c == 2) return SVDQ_ERR_UNSUPPORTED_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return SVDQ_ERR_UNSUPPORTED_DEVICE;
  }
  const bool ok = arch_is_gfx950(prop.gcnArchName);
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_release);
  return ok ? SVDQ_OK : SVDQ_ERR_UNSUPPORTED_DEVICE;
}

int check_current_device() {
  const char* force = std::getenv("SVDQ_FORCE_ARCH");
  if (force && *force) return arch_is_gfx950(force) ? SVDQ_OK : SVDQ_ERR_UNSUPPORTED_DEVICE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return SVDQ_ERR_UNSUPPORTED_DEVICE;
  }
  return check_device(dev);
}

int finish(hipError_t e) { return e == hipSuccess ? SVDQ_OK : SVDQ_ERR_HIP; }

bool rank_ok(int r) { return r >= 0 && r <= 128 && (r % 16) == 0; }
bool k_ok(int K) { return K >= 128 && K <= 65536 && (K % 128) == 0; }
bool k_nv_ok(int K) { return K >= 256 && K <= 65536 && (K % 256) == 0; }
bool positive_finite(float v) { return std::isfinite(v) && v > 0.0f; }
bool dtype_ok(int d) { return d == SVDQ_F16 || d == SVDQ_BF16; }

// Device scratch of svdq_gemm_w4a4_mlp_noalloc: the fused MLP chain's fp32
// low-rank partials live here instead of in a caller workspace. One copy per
// GPU, held until the process ends; every call on a GPU shares it. Host code
// never names `scratch` as a device address: scratch_address() takes the
// device's own address from hipGetSymbolAddress, once per device, with that
// device current.
constexpr size_t kScratchBytes = svdq::kChainScratchBytes;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return SVDQ_ERR_UNSUPPORTED_DEVICE;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(svdq::scratch));
      if (e != hipSuccess || p == nullptr) {
        (void)hipGetLastError();
        return SVDQ_ERR_HIP;
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SVDQ_OK;
}

size_t mlp_partial_bytes(int M, int N, int r2) {
  if (M < 0 || N < 0 || r2 < 0) return 0;
  return (size_t)(N / 128) * (size_t)M * (size_t)r2 * sizeof(float);
}

// The fused MLP chain behind both entry points. workspace: NULL means the
// device scratch above (then the partials must fit in it).
int mlp_chain(int fmt, int dtype, int M, int N, int K, int r, const uint8_t* act_codes, const void* act_scales,
              const float* lora_act, const uint8_t* w_codes, const void* w_scales, const void* lora_up,
              const void* bias, const float* smooth_inv2, const void* lora_down2, int r2,
              uint8_t* act_codes2, void* act_scales2, float* lora_act2, void* workspace,
              size_t workspace_bytes, bool use_scratch, void* stream) {
  if (fmt != SVDQ_INT4_G64 && fmt != SVDQ_FP4_E2M1_B32) return SVDQ_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return SVDQ_ERR_INVALID_ARG;
  if (M < 0 || M > (1 << 23) || N < 128 || N > 65536 || (N % 128) != 0 || !k_ok(K) || !rank_ok(r) ||
      !rank_ok(r2))
    return SVDQ_ERR_SHAPE;
  if (use_scratch && r2 > 0 && mlp_partial_bytes(M, N, r2) > kScratchBytes) return SVDQ_ERR_SHAPE;
  if (M == 0) return SVDQ_OK;
  if (!act_codes || !act_scales || !w_codes || !w_scales || !smooth_inv2 || !act_codes2 || !act_scales2)
    return SVDQ_ERR_INVALID_ARG;
  if (r > 0 && (!lora_act || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (r2 > 0 && (!lora_down2 || !lora_act2 || (!use_scratch && !workspace))) return SVDQ_ERR_INVALID_ARG;
  if (!use_scratch && r2 > 0 && workspace_bytes < mlp_partial_bytes(M, N, r2)) return SVDQ_ERR_SHAPE;
  if (!aligned16(act_codes) || !aligned16(act_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      (bias && !aligned16(bias)) || !aligned16(smooth_inv2) || !aligned16(act_codes2) ||
      !aligned16(act_scales2))
    return SVDQ_ERR_ALIGN;
  if (r > 0 && (!aligned16(lora_act) || !aligned16(lora_up))) return SVDQ_ERR_ALIGN;
  if (r2 > 0 && (!aligned16(lora_down2) || !aligned16(lora_act2) || (!use_scratch && !aligned16(workspace))))
    return SVDQ_ERR_ALIGN;
  const int dc = check_current_device();
  if (dc != SVDQ_OK) return dc;
  (void)hipGetLastError();
  if (use_scratch && r2 > 0) {
    const int sc = scratch_address(&workspace);
    if (sc != SVDQ_OK) return sc;
  }
  const svdq::ChainEpilogue ce{smooth_inv2, lora_down2, r2, act_codes2, act_scales2,
                               static_cast<float*>(workspace)};
  hipError_t e = svdq::launch_gemm_w4a4(fmt, dtype, M, N, K, r, act_codes, act_scales, lora_act, w_codes,
                                        w_scales, lora_up, bias, 3, nullptr, (hipStream_t)stream, nullptr, &ce);
  if (e == hipSuccess && r2 > 0)
    e = svdq::launch_chain_reduce(M, r2, N / svdq::chain_tile_n(fmt, M, N, K),
                                  static_cast<const float*>(workspace), lora_act2, (hipStream_t)stream);
  return finish(e);
}

}  // namespace


// Shader-clock probe. Each one-wave workgroup reads the constant-rate
// real-time counter (s_memrealtime) and the shader-clock cycle counter
// (s_memtime), polls the real-time counter until `ticks` of it have passed
// (at most 2^24 polls, so the loop always ends), then reads both again; lane 0
// stores (cycles, real-time ticks). The cycle interval lies inside the
// real-time one.
__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long* out, unsigned long long ticks) {
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  unsigned long long r1 = r0;
  for (int i = 0; i < (1 << 24) && r1 - r0 < ticks; ++i) r1 = __builtin_amdgcn_s_memrealtime();
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = c1 - c0;
    out[2 * blockIdx.x + 1] = r1 - r0;
  }
}

extern "C" {

int svdq_version(void) { return 10000 * 0 + 100 * 2 + 0; }

const char* svdq_status_str(int status) {
  switch (status) {
    case SVDQ_OK: return "ok";
    case SVDQ_ERR_INVALID_ARG: return "invalid argument (null pointer or bad enum value)";
    case SVDQ_ERR_SHAPE: return "unsupported shape";
    case SVDQ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SVDQ_ERR_UNSUPPORTED_DEVICE: return "no HIP device, or the device is not gfx950 (MI355X)";
    case SVDQ_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

int svdq_device_check(int hip_device) { return check_device(hip_device); }

int svdq_quantize_act(int fmt, int dtype, int M, int K, int r, const void* X, const float* smooth_inv,
                      const void* lora_down, uint8_t* act_codes, void* act_scales, float* lora_act,
                      void* stream) {
  if (fmt != SVDQ_INT4_G64 && fmt != SVDQ_FP4_E2M1_B32) return SVDQ_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return SVDQ_ERR_INVALID_ARG;
  if (M < 0 || M > (1 << 23) || !k_ok(K) || !rank_ok(r)) return SVDQ_ERR_SHAPE;
  if (M == 0) return SVDQ_OK;
  if (!X || !smooth_inv || !act_codes || !act_scales) return SVDQ_ERR_INVALID_ARG;
  if (r > 0 && (!lora_down || !lora_act)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(smooth_inv) || !aligned16(act_codes) || !aligned16(act_scales))
    return SVDQ_ERR_ALIGN;
  if (r > 0 && (!aligned16(lora_down) || !aligned16(lora_act))) return SVDQ_ERR_ALIGN;
  const int dc = check_current_device();
  if (dc != SVDQ_OK) return dc;
  (void)hipGetLastError();
  return finish(svdq::launch_quantize_act(fmt, dtype, M, K, r, X, smooth_inv, lora_down, act_codes,
                                          act_scales, lora_act, (hipStream_t)stream));
}

int svdq_gemm_w4a4(int fmt, int dtype, int M, int N, int K, int r, const uint8_t* act_codes,
                   const void* act_scales, const float* lora_act, const uint8_t* w_codes,
                   const void* w_scales, const void* lora_up, const void* bias, int epi, void* Y,
                   void* stream) {
  if (fmt != SVDQ_INT4_G64 && fmt != SVDQ_FP4_E2M1_B32) return SVDQ_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return SVDQ_ERR_INVALID_ARG;
  if (epi != SVDQ_EPI_NONE && epi != SVDQ_EPI_GELU_TANH) return SVDQ_ERR_INVALID_ARG;
  if (M < 0 || M > (1 << 23) || N < 128 || N > 65536 || (N % 128) != 0 || !k_ok(K) || !rank_ok(r))
    return SVDQ_ERR_SHAPE;
  if (M == 0) return SVDQ_OK;
  if (!act_codes || !act_scales || !w_codes || !w_scales || !Y) return SVDQ_ERR_INVALID_ARG;
  if (r > 0 && (!lora_act || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(act_codes) || !aligned16(act_scales) || !aligned16(w_codes) ||
      !aligned16(w_scales) || !aligned16(Y) || (bias && !aligned16(bias)))
    return SVDQ_ERR_ALIGN;
  if (r > 0 && (!aligned16(lora_act) || !aligned16(lora_up))) return SVDQ_ERR_ALIGN;
  const int dc = check_current_device();
  if (dc != SVDQ_OK) return dc;
  (void)hipGetLastError();
  return finish(svdq::launch_gemm_w4a4(fmt, dtype, M, N, K, r, act_codes, act_scales, lora_act, w_codes,
                                       w_scales, lora_up, bias, epi, Y, (hipStream_t)stream));
}

size_t svdq_gemm_w4a4_splitk_workspace(int fmt, int M, int N, int K) {
  if ((fmt != SVDQ_INT4_G64 && fmt != SVDQ_FP4_E2M1_B32) || M < 1 || M > (1 << 23) || N < 128 || N > 65536 ||
      (N % 128) != 0 || !k_ok(K))
    return 0;
  return svdq::splitk_bytes(fmt, M, N, K);
}

int svdq_gemm_w4a4_splitk(int fmt, int dtype, int M, int N, int K, int r, const uint8_t* act_codes,
                          const void* act_scales, const float* lora_act, const uint8_t* w_codes,
                          const void* w_scales, const void* lora_up, const void* bias, int epi, void* Y,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (fmt != SVDQ_INT4_G64 && fmt != SVDQ_FP4_E2M1_B32) return SVDQ_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return SVDQ_ERR_INVALID_ARG;
  if (epi != SVDQ_EPI_NONE && epi != SVDQ_EPI_GELU_TANH) return SVDQ_ERR_INVALID_ARG;
  if (M < 0 || M > (1 << 23) || N < 128 || N > 65536 || (N % 128) != 0 || !k_ok(K) || !rank_ok(r))
    return SVDQ_ERR_SHAPE;
  if (M == 0) return SVDQ_OK;
  if (!act_codes || !act_scales || !w_codes || !w_scales || !Y) return SVDQ_ERR_INVALID_ARG;
  if (r > 0 && (!lora_act || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(act_codes) || !aligned16(act_scales) || !aligned16(w_codes) ||
      !aligned16(w_scales) || !aligned16(Y) || (bias && !aligned16(bias)) || (workspace && !aligned16(workspace)))
    return SVDQ_ERR_ALIGN;
  if (r > 0 && (!aligned16(lora_act) || !aligned16(lora_up))) return SVDQ_ERR_ALIGN;
  const int dc = check_current_device();
  if (dc != SVDQ_OK) return dc;
  (void)hipGetLastError();
  return finish(svdq::launch_gemm_w4a4_split(fmt, dtype, M, N, K, r, act_codes, act_scales, lora_act, w_codes,
                                             w_scales, lora_up, bias, epi, Y, workspace, workspace_bytes,
                                             (hipStream_t)stream));
}

int svdq_gemm_w4a4_qkv(int fmt, int dtype, int M, int N, int K, int r, const uint8_t* act_codes,
                       const void* act_scales, const float* lora_act, const uint8_t* w_codes,
                       const void* w_scales, const void* lora_up, const void* bias,
                       const void* qk_norm_w, const float* rope, float eps, void* Y, void* stream) {
  if (fmt != SVDQ_INT4_G64) return SVDQ_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return SVDQ_ERR_INVALID_ARG;
  if (!(eps >= 0.0f) || eps > 1.0f) return SVDQ_ERR_INVALID_ARG;   // also rejects NaN
  if (M < 0 || M > (1 << 23) || N < 384 || N > 65536 || (N % 384) != 0 || !k_ok(K) || !rank_ok(r))
    return SVDQ_ERR_SHAPE;
  if (M == 0) return SVDQ_OK;
  if (!act_codes || !act_scales || !w_codes || !w_scales || !Y || !qk_norm_w || !rope)
    return SVDQ_ERR_INVALID_ARG;
  if (r > 0 && (!lora_act || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(act_codes) || !aligned16(act_scales) || !aligned16(w_codes) ||
      !aligned16(w_scales) || !aligned16(Y) || (bias && !aligned16(bias)) ||
      !aligned16(qk_norm_w) || !aligned16(rope))
    return SVDQ_ERR_ALIGN;
  if (r > 0 && (!aligned16(lora_act) || !aligned16(lora_up))) return SVDQ_ERR_ALIGN;
  const int dc = check_current_device();
  if (dc != SVDQ_OK) return dc;
  (void)hipGetLastError();
  const svdq::QkvEpilogue qe{qk_norm_w, rope, eps, N / 384};
  return finish(svdq::launch_gemm_w4a4(fmt, dtype, M, N, K, r, act_codes, act_scales, lora_act, w_codes,
                                       w_scales, lora_up, bias, 2, Y, (hipStream_t)stream, &qe));
}

size_t svdq_gemm_w4a4_mlp_workspace(int M, int N, int r2) { return mlp_partial_bytes(M, N, r2); }

int svdq_gemm_w4a4_mlp(int fmt, int dtype, int M, int N, int K, int r, const uint8_t* act_codes,
                       const void* act_scales, const float* lora_act, const uint8_t* w_codes,
                       const void* w_scales, const void* lora_up, const void* bias,
                       const float* smooth_inv2, const void* lora_down2, int r2, uint8_t* act_codes2,
                       void* act_scales2, float* lora_act2, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return mlp_chain(fmt, dtype, M, N, K, r, act_codes, act_scales, lora_act, w_codes, w_scales, lora_up, bias,
                   smooth_inv2, lora_down2, r2, act_codes2, act_scales2, lora_act2, workspace, workspace_bytes,
                   false, stream);
}

int svdq_gemm_w4a4_mlp_noalloc(int fmt, int dtype, int M, int N, int K, int r, const uint8_t* act_codes,
                               const void* act_scales, const float* lora_act, const uint8_t* w_codes,
                               const void* w_scales, const void* lora_up, const void* bias,
                               const float* smooth_inv2, const void* lora_down2, int r2, uint8_t* act_codes2,
                               void* act_scales2, float* lora_act2, void* stream) {
  return mlp_chain(fmt, dtype, M, N, K, r, act_codes, act_scales, lora_act, w_codes, w_scales, lora_up, bias,
                   smooth_inv2, lora_down2, r2, act_codes2, act_scales2, lora_act2, nullptr, 0, true, stream);
}

int svdq_quantize_act_nvfp4(int dtype, int M, int K, int r, const void* X, const float* smooth_inv,
                            const void* lora_down, float act_gscale, uint8_t* act_codes,
                            uint8_t* act_scales, float* lora_act, void* stream) {
  if (!dtype_ok(dtype)) return SVDQ_ERR_INVALID_ARG;
  if (M < 0 || M > (1 << 23) || !k_nv_ok(K) || !rank_ok(r)) return SVDQ_ERR_SHAPE;
  if (!positive_finite(act_gscale) || !positive_finite(6.0f * act_gscale)) return SVDQ_ERR_INVALID_ARG;
  if (M == 0) return SVDQ_OK;
  if (!X || !smooth_inv || !act_codes || !act_scales) return SVDQ_ERR_INVALID_ARG;
  if (r > 0 && (!lora_down || !lora_act)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(smooth_inv) || !aligned16(act_codes) || !aligned16(act_scales))
    return SVDQ_ERR_ALIGN;
  if (r > 0 && (!aligned16(lora_down) || !aligned16(lora_act))) return SVDQ_ERR_ALIGN;
  const int dc = check_current_device();
  if (dc != SVDQ_OK) return dc;
  (void)hipGetLastError();
  return finish(svdq::launch_quantize_act(SVDQ_NVFP4_G16, dtype, M, K, r, X, smooth_inv, lora_down, act_codes,
                                          act_scales, lora_act, (hipStream_t)stream, act_gscale));
}

int svdq_gemm_nvfp4(int dtype, int M, int N, int K, int r, const uint8_t* act_codes,
                    const uint8_t* act_scales, const float* lora_act, const uint8_t* w_codes,
                    const uint8_t* w_scales, const void* lora_up, const void* bias, float alpha,
                    int epilogue, void* Y, void* stream) {
  if (!dtype_ok(dtype)) return SVDQ_ERR_INVALID_ARG;
  if (epilogue != SVDQ_EPI_NONE && epilogue != SVDQ_EPI_GELU_TANH) return SVDQ_ERR_INVALID_ARG;
  if (!std::isfinite(alpha)) return SVDQ_ERR_INVALID_ARG;
  if (M < 0 || M > (1 << 23) || N < 128 || N > 65536 || (N % 128) != 0 || !k_nv_ok(K) || !rank_ok(r))
    return SVDQ_ERR_SHAPE;
  if (M == 0) return SVDQ_OK;
  if (!act_codes || !act_scales || !w_codes || !w_scales || !Y) return SVDQ_ERR_INVALID_ARG;
  if (r > 0 && (!lora_act || !lora_up)) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(act_codes) || !aligned16(act_scales) || !aligned16(w_codes) || !aligned16(w_scales) ||
      !aligned16(Y) || (bias && !aligned16(bias)))
    return SVDQ_ERR_ALIGN;
  if (r > 0 && (!aligned16(lora_act) || !aligned16(lora_up))) return SVDQ_ERR_ALIGN;
  const int dc = check_current_device();
  if (dc != SVDQ_OK) return dc;
  (void)hipGetLastError();
  return finish(svdq::launch_gemm_nvfp4(dtype, M, N, K, r, act_codes, act_scales, lora_act, w_codes, w_scales,
                                        lora_up, bias, alpha, epilogue, Y, (hipStream_t)stream));
}

int awq_gemv_w4a16(int dtype, int M, int N, int K, int group, const void* x, const uint8_t* w_codes,
                   const void* scales, const void* zeros, const void* bias, void* y, void* stream) {
  if (!dtype_ok(dtype)) return SVDQ_ERR_INVALID_ARG;
  if (group != 64) return SVDQ_ERR_SHAPE;
  if (M < 0 || M > 8 || N < 1 || N > (1 << 20) || K < 64 || (K % 64) != 0 || M * K > 32768)
    return SVDQ_ERR_SHAPE;
  if (M == 0) return SVDQ_OK;
  if (!x || !w_codes || !scales || !zeros || !y) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_codes) || !aligned16(scales) || !aligned16(zeros) ||
      !aligned16(y) || !aligned16(bias))
    return SVDQ_ERR_ALIGN;
  const int dc = check_current_device();
  if (dc != SVDQ_OK) return dc;
  (void)hipGetLastError();
  return finish(svdq::launch_awq_gemv(dtype, M, N, K, x, w_codes, scales, zeros, bias, y,
                                      (hipStream_t)stream));
}

int svdq_clock_probe(int workgroups, unsigned long long ticks, unsigned long long* out, int* wall_khz,
                     void* stream) {
  if (workgroups < 1 || workgroups > 4096 || ticks < 1 || ticks > 100000000ull) return SVDQ_ERR_SHAPE;
  if (!out || !wall_khz) return SVDQ_ERR_INVALID_ARG;
  if (!aligned16(out)) return SVDQ_ERR_ALIGN;
  const int dc = check_current_device();
  if (dc != SVDQ_OK) return dc;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return SVDQ_ERR_HIP;
  (void)hipGetLastError();
  hipLaunchKernelGGL(clock_probe_kernel, dim3(workgroups), dim3(64), 0, (hipStream_t)stream, out, ticks);
  return finish(hipGetLastError());
}

}  // extern "C"
