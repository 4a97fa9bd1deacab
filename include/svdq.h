/*
 * svdq.h -- C ABI of the MI355X (gfx950) SVDQuant W4A4 + AWQ W4A16 library.
 *
 * The layer this library runs is the SVDQuant linear layer: activation
 * outliers migrated into the weights by a per-channel smoothing, a small
 * 16-bit low-rank branch holding the hardest part of the weight, and the
 * residual quantized to 4 bits, so the main product runs with 4-bit weights
 * AND 4-bit activations (dothoosh.com "How Nunchaku Lite halves
 * diffusion-model VRAM", SVDQuant paragraph; nextgz.net "Hugging Face brings
 * Nunchaku Lite to Diffusers", section "Why W4A4 differs from weight-only
 * backends"). As on the pages' fused kernels, the low-rank down-projection
 * is fused with the activation quantizer and the up-projection with the
 * 4-bit GEMM (dothoosh.com article, fused-kernel paragraph), giving two
 * calls per layer:
 *
 *     svdq_quantize_act:  X -> (act_codes, act_scales, lora_act = X . lora_down^T)
 *     svdq_gemm_w4a4:     Y = act(lora_act . lora_up^T + dequant(act) dequant(W)^T + bias)
 *
 * plus the AWQ W4A16 GEMV of the modulation / adaptive-norm projections
 * (dothoosh.com article, kernel-family list, the awq_w4a16 entry).
 *
 * Conventions for every entry point:
 *   - Ownership: the caller owns every buffer; all pointers are DEVICE
 *     pointers (HIP device memory) unless stated. The library allocates
 *     nothing, keeps no per-call state and only uses the pointers for the
 *     work it enqueues.
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL is the
 *     null stream) and the call returns without synchronizing.
 *   - Errors: arguments are checked on the host BEFORE anything is enqueued;
 *     the call returns an svdq_status and never aborts or prints. Order of
 *     checks: enum values, sizes (SVDQ_ERR_SHAPE), null pointers
 *     (SVDQ_ERR_INVALID_ARG), 16-byte alignment of every pointer
 *     (SVDQ_ERR_ALIGN), then the device (SVDQ_ERR_UNSUPPORTED_DEVICE: the
 *     current HIP device is not gfx950, or there is none), then the launch
 *     (SVDQ_ERR_HIP). A call with M == 0 validates and returns SVDQ_OK
 *     without enqueuing work (pointers may then be NULL).
 *   - Layouts are row-major and K-contiguous: X [M][K], W [N][K]
 *     (nn.Linear layout), Y [M][N]. 4-bit codes are packed two per byte,
 *     the even-k code in the low nibble. INT4 codes are two's complement
 *     (the quantizers produce -7..7; -8 is accepted).
 *   - Thread safety: calls may be made concurrently from several threads;
 *     the only global state is a per-device architecture cache.
 */
#ifndef SVDQ_MI355X_H
#define SVDQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVDQ_OK = 0,
  SVDQ_ERR_INVALID_ARG = -1,       /* NULL pointer or bad enum value */
  SVDQ_ERR_SHAPE = -2,             /* size outside what the kernels support */
  SVDQ_ERR_ALIGN = -3,             /* a pointer is not 16-byte aligned */
  SVDQ_ERR_UNSUPPORTED_DEVICE = -4,/* no HIP device, or not gfx950 */
  SVDQ_ERR_HIP = -5                /* the HIP runtime reported a launch error */
} svdq_status;

/* 4-bit formats. The pages ship INT4 and a 4-bit float (NVFP4, group 16)
 * (dothoosh.com article, kernel-family list and quantization_config block).
 * SVDQ_INT4_G64: symmetric INT4, one fp16 scale per 64 values along K.
 * SVDQ_FP4_E2M1_B32: OCP E2M1 codes, one E8M0 (power-of-two) scale byte per
 *   32 values along K -- the block-scaled form CDNA4's matrix cores consume.
 * SVDQ_NVFP4_G16: the pages' own float format: OCP E2M1 codes, one OCP FP8
 *   E4M3 scale byte per 16 values along K and one fp32 scale per tensor; it
 *   has entry points of its own (svdq_quantize_act_nvfp4, svdq_gemm_nvfp4),
 *   which carry the per-tensor scales. */
typedef enum { SVDQ_INT4_G64 = 0, SVDQ_FP4_E2M1_B32 = 1, SVDQ_NVFP4_G16 = 2 } svdq_format;

/* Epilogue applied after the bias: identity, or GELU in its tanh form
 * y/2 (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))) for MLP up-projections
 * (the GELU/MLP fusion of the full engine, dothoosh.com article, paragraph on
 * model-specific fused paths). */
typedef enum { SVDQ_EPI_NONE = 0, SVDQ_EPI_GELU_TANH = 1 } svdq_epilogue;

/* The layer's 16-bit compute type (the quantization_config's compute_dtype,
 * dothoosh.com article, quantization_config block; "bfloat16" in the pages'
 * example). Below, "h16" is this type: it is the type of X, lora_down,
 * lora_up, bias, qk_norm_w and Y, and of the GEMV's x, bias and y.
 * Conversions to h16 round to nearest, ties to even; the low-rank products
 * run on the h16 matrix instructions with fp32 accumulation. lora_act, the
 * low-rank activations between the two calls, is fp32 whatever dtype is.
 * Stored scales keep their format's own type whatever dtype is (INT4 and AWQ:
 * fp16). A value outside this enum is SVDQ_ERR_INVALID_ARG. */
typedef enum { SVDQ_F16 = 0, SVDQ_BF16 = 1 } svdq_dtype;

/* Returns SVDQ_OK iff HIP device `hip_device` exists and is a gfx950 part.
 * This is the library's capability check: a clear error instead of wrong
 * output on hardware the kernels were not built for (dothoosh.com article,
 * hardware-support paragraph). Result is cached per device. */
int svdq_device_check(int hip_device);

/* Static string for a status code (never NULL). */
const char* svdq_status_str(int status);

/* Library version as 10000*major + 100*minor + patch. */
int svdq_version(void);

/*
 * svdq_quantize_act -- fused activation smoothing, low-rank down-projection
 * and per-group 4-bit activation quantization (one pass over X).
 *
 *   x_hat[m,k]   = fl32(fp32(X[m,k]) * smooth_inv[k])          (IEEE multiply)
 *   lora_act[m,j]= sum_k X[m,k] * lora_down[j,k]             (h16 inputs, fp32 accumulate)
 *   INT4_G64, per row m and group g of 64 along K:
 *     amax = max |x_hat|;  s = fp16_rne(min(fl32(amax / 7), 65504));
 *     q = s == 0 ? 0 : clamp(rint_even(fl32(x_hat / s)), -7, 7)   (IEEE division)
 *   FP4_E2M1_B32, per row m and block of 32 along K:
 *     amax == 0 -> scale byte 0, codes 0; else e = min integer with
 *     6 * 2^e >= amax, clamped to [-127, 127]; scale byte = e + 127;
 *     code = E2M1 nearest to x_hat / 2^e (ties to even mantissa), sign bit
 *     from x_hat's sign.
 * Codes and scales are bit-exact functions of (X, smooth_inv); lora_act is a
 * float result (fp32 accumulation in a fixed but unspecified order, stored in
 * fp32).
 *
 * Arguments:
 *   fmt         svdq_format.
 *   dtype       svdq_dtype.
 *   M           rows (tokens), 0 <= M <= 2^23.
 *   K           input channels; K % 128 == 0, 128 <= K <= 65536.
 *   r           low-rank width; r % 16 == 0, 0 <= r <= 128.
 *   X           h16 [M][K].
 *   smooth_inv  fp32 [K], the smoothing multiplier (1/lambda).
 *   lora_down   h16 [r][K] (carries diag(smooth_inv)); may be NULL iff r == 0.
 *   act_codes   out, u8 [M][K/2]. With few rows and a long K the call splits K
 *               across workgroups and first parks fp32 low-rank partial sums in
 *               the tails of these rows (scratch owned by the call until its
 *               work on `stream` completes; the final content is the codes).
 *   act_scales  out, fp16 [M][K/64] (INT4_G64) or u8 [M][K/32] (FP4_E2M1_B32).
 *   lora_act    out, fp32 [M][r]; may be NULL iff r == 0.
 *   stream      hipStream_t.
 */
int svdq_quantize_act(int fmt, int dtype, int M, int K, int r,
                      const void* X, const float* smooth_inv, const void* lora_down,
                      uint8_t* act_codes, void* act_scales, float* lora_act,
                      void* stream);

/*
 * svdq_gemm_w4a4 -- the 4-bit GEMM with the low-rank up-projection, scale
 * dequantization, bias and epilogue fused:
 *
 *   Y[m,n] = act( sum_j lora_act[m,j] lora_up[n,j]
 *               + sum_g s_x[m,g] s_w[n,g] sum_{k in g} q_x[m,k] q_w[n,k]
 *               + bias[n] )                                 -> h16 (RNE)
 *
 * INT4_G64 multiplies the codes exactly (int8 matrix cores, int32 per
 * group) and applies s_x s_w in fp32; FP4_E2M1_B32 uses the block-scaled
 * FP4 matrix instruction with the E8M0 scales applied in hardware and fp32
 * accumulation. The low-rank product takes each fp32 lora_act value as a pair
 * of h16 operands, hi = h16(v) and lo = h16(v - hi), on two matrix
 * instructions with fp32 accumulation: hi + lo is v within 2^-22 |v| for fp16
 * (2^-18 |v| for bf16), where one h16 value would be off by up to 2^-11 |v|
 * (2^-8 |v|). |lora_act| must stay below the h16 maximum.
 *
 * Arguments:
 *   fmt         svdq_format.
 *   M           rows, 0 <= M <= 2^23 (any value; tails are masked).
 *   N           output channels; N % 128 == 0, N <= 65536.
 *   K           input channels; K % 128 == 0, 128 <= K <= 65536.
 *   r           low-rank width; r % 16 == 0, 0 <= r <= 128.
 *   act_codes   u8 [M][K/2] (from svdq_quantize_act).
 *   act_scales  fp16 [M][K/64] or u8 [M][K/32].
 *   lora_act    fp32 [M][r] (from svdq_quantize_act); may be NULL iff r == 0.
 *   w_codes     u8 [N][K/2].
 *   w_scales    fp16 [N][K/64] or u8 [N][K/32].
 *   lora_up     h16 [N][r]; may be NULL iff r == 0.
 *   bias        h16 [N], or NULL for no bias.
 *   epi         svdq_epilogue.
 *   Y           out, h16 [M][N].
 *   stream      hipStream_t.
 */
int svdq_gemm_w4a4(int fmt, int dtype, int M, int N, int K, int r,
                   const uint8_t* act_codes, const void* act_scales, const float* lora_act,
                   const uint8_t* w_codes, const void* w_scales, const void* lora_up,
                   const void* bias, int epi, void* Y, void* stream);

/*
 * svdq_gemm_w4a4_splitk -- svdq_gemm_w4a4 (epi NONE or GELU_TANH) for shapes
 * with too few output tiles to fill the GPU (few tokens, long K, e.g. an MLP
 * down-projection at M 1024): K is cut into S near-equal runs of whole 128-code
 * steps, S (a power of two, at most 8) workgroups per output tile each write
 * the fp32 partial sum of their run into `workspace` ([S][M][N]; the low-rank
 * product joins the first run), and a second kernel adds the S partials in
 * run order and applies bias and epilogue as svdq_gemm_w4a4 does. The same
 * float result up to the order of the fp32 additions (deterministic). INT4
 * only: with SVDQ_FP4_E2M1_B32, with a shape that does not split, with a NULL
 * workspace or with workspace_bytes below
 * svdq_gemm_w4a4_splitk_workspace(...), the call runs svdq_gemm_w4a4 itself.
 *
 * Arguments as svdq_gemm_w4a4, and
 *   workspace        device memory (16-byte aligned) owned by the call until its
 *                    work on `stream` completes; contents on entry do not matter.
 *   workspace_bytes  its size.
 */
int svdq_gemm_w4a4_splitk(int fmt, int dtype, int M, int N, int K, int r,
                          const uint8_t* act_codes, const void* act_scales, const float* lora_act,
                          const uint8_t* w_codes, const void* w_scales, const void* lora_up,
                          const void* bias, int epi, void* Y, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Workspace bytes svdq_gemm_w4a4_splitk splits K with for this shape:
 * S M N 4, or 0 when the shape (or format) does not split or is invalid. */
size_t svdq_gemm_w4a4_splitk_workspace(int fmt, int M, int N, int K);

/*
 * svdq_gemm_w4a4_qkv -- svdq_gemm_w4a4 for a fused Q|K|V projection, with the
 * per-head RMSNorm of Q and K and the rotary position embedding applied in the
 * same epilogue (the pages' structural rewrite that fuses the QKV projection
 * with the Q/K norm and the rotary embedding: dothoosh.com article,
 * structural-rewrites paragraph). With lin[m,n] the svdq_gemm_w4a4 result
 * before rounding (bias included, no activation), heads of D = 128 channels
 * and H = N / 384 heads per third:
 *
 *   V third   (n >= 2 H D):  Y = lin
 *   Q, K      (per head):    u[d] = lin[d] / sqrt(mean_d lin^2 + eps) * w[d]
 *                            Y[2i]   = u[2i] cos[m,i] - u[2i+1] sin[m,i]
 *                            Y[2i+1] = u[2i] sin[m,i] + u[2i+1] cos[m,i]
 *                                                         -> h16 (RNE)
 *
 * Float results (fp32 arithmetic, hardware rsqrt); INT4_G64 only.
 *
 * Arguments as svdq_gemm_w4a4 (fmt must be SVDQ_INT4_G64, no activation), and
 *   N           output channels; N % 384 == 0 (Q, K, V thirds of 128-channel heads).
 *   qk_norm_w   h16 [2][128]: the RMSNorm weights of Q, then of K.
 *   rope        fp32 [M][64][2]: (cos, sin) of token m for channel pair i.
 *   eps         RMSNorm epsilon, 0 <= eps <= 1.
 * Errors: SVDQ_ERR_INVALID_ARG for another format, a bad eps or a NULL
 * qk_norm_w / rope; otherwise as svdq_gemm_w4a4.
 */
int svdq_gemm_w4a4_qkv(int fmt, int dtype, int M, int N, int K, int r,
                       const uint8_t* act_codes, const void* act_scales, const float* lora_act,
                       const uint8_t* w_codes, const void* w_scales, const void* lora_up,
                       const void* bias, const void* qk_norm_w, const float* rope, float eps,
                       void* Y, void* stream);

/*
 * svdq_gemm_w4a4_mlp -- the fused MLP chain: an MLP up-projection with GELU
 * whose output never reaches memory; its 16-bit result U goes straight into
 * the down-projection's activation quantizer (the pages' GELU / MLP fused
 * kernels of the full engine: dothoosh.com article, generic-path paragraph).
 * Exactly the composition of the unfused calls, without Y:
 *
 *   U = h16_rne( svdq_gemm_w4a4(..., SVDQ_EPI_GELU_TANH) )      (not stored)
 *   act_codes2, act_scales2, lora_act2 = svdq_quantize_act(INT4_G64, U,
 *                                          smooth_inv2, lora_down2)
 *
 * The codes and scales equal the unfused path's bit for bit (the same U, the
 * same quantizer rule); lora_act2 is summed over the up-projection's tiles of
 * columns (128, or 256 for the large FP4 tile) in fp32, in a fixed order
 * (deterministic), and stored in fp32. Two kernels: the GEMM with the
 * quantizer in its epilogue, and the sum of the per-tile partials of the
 * low-rank down-projection, kept in `workspace`.
 *
 * Arguments as svdq_gemm_w4a4 for the up-projection (fmt: SVDQ_INT4_G64 or
 * SVDQ_FP4_E2M1_B32, the up-projection's own format; the down-projection's
 * codes are INT4 g64 either way; GELU is implied; there is no Y), and
 *   smooth_inv2      fp32 [N], the down-projection's smoothing multiplier.
 *   lora_down2       h16 [r2][N], its low-rank down factor; NULL iff r2 == 0.
 *   r2               its low-rank width; r2 % 16 == 0, 0 <= r2 <= 128.
 *   act_codes2       out, u8 [M][N/2]   (INT4 codes of U, the down-projection's K = N).
 *   act_scales2      out, fp16 [M][N/64].
 *   lora_act2        out, fp32 [M][r2]; NULL iff r2 == 0.
 *   workspace        device memory of at least svdq_gemm_w4a4_mlp_workspace(M, N, r2)
 *                    bytes (fp32 partials), owned by the caller; NULL iff r2 == 0.
 *   workspace_bytes  its size (SVDQ_ERR_SHAPE if too small).
 */
size_t svdq_gemm_w4a4_mlp_workspace(int M, int N, int r2);
int svdq_gemm_w4a4_mlp(int fmt, int dtype, int M, int N, int K, int r,
                       const uint8_t* act_codes, const void* act_scales, const float* lora_act,
                       const uint8_t* w_codes, const void* w_scales, const void* lora_up,
                       const void* bias, const float* smooth_inv2, const void* lora_down2, int r2,
                       uint8_t* act_codes2, void* act_scales2, float* lora_act2,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * svdq_gemm_w4a4_mlp_noalloc -- svdq_gemm_w4a4_mlp for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, the same arguments
 * without `workspace` / `workspace_bytes`, bit-identical results. The fp32
 * partials live in a device array of the library instead: 64 MiB
 * (67108864 bytes), one copy per GPU, created when the library's code is
 * loaded on that GPU and held until the process ends. The call allocates
 * nothing and calls no allocating routine.
 *
 * Limit: svdq_gemm_w4a4_mlp_workspace(M, N, r2) <= 67108864 (e.g. M 4096,
 * N 12288, r2 32 needs 50331648), else SVDQ_ERR_SHAPE; r2 == 0 uses no scratch.
 * Every call on one GPU shares the array and overwrites it (the partials are
 * written in full before they are read, so nothing needs clearing): calls
 * that overlap on one GPU -- on two streams, or from two threads without
 * ordering -- race and give wrong results. Calls on one stream are ordered
 * and safe.
 */
int svdq_gemm_w4a4_mlp_noalloc(int fmt, int dtype, int M, int N, int K, int r,
                               const uint8_t* act_codes, const void* act_scales, const float* lora_act,
                               const uint8_t* w_codes, const void* w_scales, const void* lora_up,
                               const void* bias, const float* smooth_inv2, const void* lora_down2, int r2,
                               uint8_t* act_codes2, void* act_scales2, float* lora_act2, void* stream);

/*
 * svdq_quantize_act_nvfp4 -- svdq_quantize_act for NVFP4 (the pages' svdq_w4a4
 * precision "nvfp4" with group size 16: dothoosh.com article,
 * quantization_config block). Smoothing and the low-rank down-projection as
 * in svdq_quantize_act; then, per block of 16 values of x_hat along K, with
 * the activations' per-tensor scale g (fixed offline from calibration data):
 *
 *   s    = E4M3_rne( fl32( amax / fl32(6 g) ) )   saturating at 448 (0x7E);
 *   d    = fl32( E4M3(s) * g );
 *   code = E2M1_rne( fl32( x_hat / d ) )          (IEEE division; nearest,
 *          ties to even mantissa, saturating at 6, sign from x_hat; all codes
 *          0 where d == 0).
 *
 * A value is E2M1(code) * E4M3(s) * g. Codes and scales are bit-exact.
 *
 * Arguments as svdq_quantize_act, except:
 *   K           K % 256 == 0, 256 <= K <= 65536.
 *   act_gscale  g, finite and > 0 (else SVDQ_ERR_INVALID_ARG).
 *   act_scales  out, u8 [M][K/16] E4M3 bytes (sign bit 0).
 */
int svdq_quantize_act_nvfp4(int dtype, int M, int K, int r,
                            const void* X, const float* smooth_inv, const void* lora_down,
                            float act_gscale, uint8_t* act_codes, uint8_t* act_scales,
                            float* lora_act, void* stream);

/*
 * svdq_gemm_nvfp4 -- svdq_gemm_w4a4 for NVFP4 operands:
 *
 *   Y[m,n] = act( alpha * sum_k (E2M1(q_x[m,k]) E4M3(s_x[m,k/16]))
 *                               (E2M1(q_w[n,k]) E4M3(s_w[n,k/16]))
 *               + sum_j lora_act[m,j] lora_up[n,j] + bias[n] )     -> h16 (RNE)
 *
 * with alpha = act_gscale * w_gscale (the two per-tensor scales; the caller
 * forms the product). gfx950 has no matrix instruction for E4M3 scales per
 * 16, so both operands are dequantized exactly to fp16 and multiplied on the
 * fp16 matrix cores with fp32 accumulation.
 *
 * Arguments as svdq_gemm_w4a4, except:
 *   K           K % 256 == 0, 256 <= K <= 65536.
 *   act_scales  u8 [M][K/16], w_scales u8 [N][K/16]: E4M3 bytes; the sign bit
 *               is ignored (scales are magnitudes).
 *   alpha       finite (else SVDQ_ERR_INVALID_ARG).
 */
int svdq_gemm_nvfp4(int dtype, int M, int N, int K, int r,
                    const uint8_t* act_codes, const uint8_t* act_scales, const float* lora_act,
                    const uint8_t* w_codes, const uint8_t* w_scales, const void* lora_up,
                    const void* bias, float alpha, int epilogue, void* Y, void* stream);

/*
 * awq_gemv_w4a16 -- 4-bit weights, 16-bit activations, memory-bound GEMV for
 * the modulation / adaptive-norm projections (dothoosh.com article,
 * kernel-family list: awq_w4a16; quantization_config block: int4, group 64):
 *
 *   y[m,n] = sum_k x[m,k] * (q[n,k] - z[n,k/G]) * s[n,k/G] + bias[n]   -> h16 (RNE)
 *
 * with fp32 accumulation; the bias is added to the fp32 total before the one
 * rounding to h16.
 *
 * Arguments:
 *   M       rows of x, 0 <= M <= 8.
 *   N       output channels, 1 <= N <= 2^20.
 *   K       input channels; K % 64 == 0, K >= 64, M * K <= 32768 (x is staged
 *           in LDS).
 *   group   group size along K; must be 64.
 *   dtype   svdq_dtype (x, bias and y).
 *   x       h16 [M][K].
 *   w_codes u8 [N][K/2], unsigned nibbles, even k in the low nibble.
 *   scales  fp16 [N][K/64].
 *   zeros   fp16 [N][K/64], in code units (any fp16 value).
 *   bias    h16 [N], or NULL for none.
 *   y       out, h16 [M][N].
 *   stream  hipStream_t.
 */
int awq_gemv_w4a16(int dtype, int M, int N, int K, int group,
                   const void* x, const uint8_t* w_codes, const void* scales,
                   const void* zeros, const void* bias, void* y, void* stream);

/*
 * svdq_clock_probe -- measures the shader clock, for reporting next to
 * timings (the clock a kernel ran at decides its share of the chip's peak).
 * Each of `workgroups` one-wave workgroups counts shader cycles (s_memtime)
 * while the constant-rate real-time counter (s_memrealtime) advances by
 * `ticks`; the clock in MHz is cycles / ticks * wall_khz / 1000.
 *
 * Arguments:
 *   workgroups  1 .. 4096 (256 puts about one on every CU).
 *   ticks       real-time ticks to wait, 1 .. 10^8.
 *   out         out, device u64 [workgroups][2]: (cycles, ticks) per workgroup.
 *   wall_khz    out, HOST int: the real-time counter's rate in kHz.
 *   stream      hipStream_t.
 */
int svdq_clock_probe(int workgroups, unsigned long long ticks, unsigned long long* out, int* wall_khz,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_MI355X_H */
