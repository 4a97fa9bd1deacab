"""Oracle for the SVDQ W4A4 linear layer: offline preparation (smoothing,
low-rank split, residual quantization) and the run-time reference
(smoothing, low-rank down-projection, 4-bit activation quantization, group-
scaled 4-bit GEMM, low-rank up-projection, bias, GELU).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources. The method is one sentence repeated on the pages: outliers move from
the activations into the weights, a small 16-bit low-rank branch holds the
hardest part of each weight matrix, and the residual is quantized to 4 bits
(dothoosh.com "How Nunchaku Lite halves diffusion-model VRAM", SVDQuant
paragraph; news.hamidun.com "Nunchaku Lite: 4-bit image generation in
Diffusers", section "What are Nunchaku and SVDQuant"; nextgz.net "Hugging Face
brings Nunchaku Lite to Diffusers", section "Why W4A4 differs from
weight-only backends"). The fused kernels put the low-rank down-projection
next to the activation quantizer and the up-projection next to the 4-bit
GEMM (dothoosh.com article, fused-kernel paragraph). Both INT4 and a 4-bit
float format exist (dothoosh.com article, kernel-family list and the
quantization_config block: rank 32, group size 16 for the float format, 64
for INT4 AWQ).

Notation: X is M x K (tokens x input channels), W is N x K (nn.Linear
layout: out x in), Y = X W^T + b is M x N. Groups run along K.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
FP16_MAX = 65504.0

# OCP E2M1 magnitudes by 3-bit code (exponent bits << 1 | mantissa bit).
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])

FORMATS = ("int4_g64", "fp4_b32", "nvfp4_g16")

# 6 * 448: the largest E2M1 magnitude times the largest E4M3 value.
NVFP4_RANGE = 2688.0


def _group(fmt: str) -> int:
    if fmt == "int4_g64":
        return 64
    if fmt == "fp4_b32":
        return 32
    if fmt == "nvfp4_g16":
        return 16
    raise ValueError(f"unknown format {fmt!r}")


# --------------------------------------------------------------------------
# Storage: two 4-bit codes per byte, the even-k code in the low nibble.
# [reading: the pages give no packing; this is the canonical layout.]
# --------------------------------------------------------------------------

def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """codes [..., K] (INT4 values -8..7 or 4-bit patterns 0..15) -> u8 [..., K/2]."""
    c = np.asarray(codes).astype(np.int64)
    if c.shape[-1] % 2:
        raise ValueError("last dimension must be even")
    nib = (c & 0xF).astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray, signed: bool) -> np.ndarray:
    """u8 [..., K/2] -> [..., K]; signed=True reads two's-complement INT4."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int16)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    if signed:
        out = np.where(out >= 8, out - 16, out)
    return out.astype(np.int8)


# --------------------------------------------------------------------------
# Offline preparation (oracle only; its outputs are inputs to both sides).
# --------------------------------------------------------------------------

def smoothing_factors(X_cal: np.ndarray, W: np.ndarray, alpha: float) -> np.ndarray:
    """Per-input-channel smoothing, returned as the fp32 multiplier applied to
    activations (smooth_inv = 1/lambda).

    Outlier migration (dothoosh.com article, SVDQuant paragraph) with the
    plainest rule that has an exponent alpha [reading]: lambda_k =
    a_k^alpha / w_k^(1-alpha), a_k = max_m |X_cal[m,k]|, w_k = max_n |W[n,k]|;
    lambda_k = 1 where a_k or w_k is 0. smooth_inv = fp32_rne(1 / lambda).
    """
    a = np.max(np.abs(np.asarray(X_cal, dtype=np.float64)), axis=0)
    w = np.max(np.abs(np.asarray(W, dtype=np.float64)), axis=0)
    lam = np.ones_like(a)
    ok = (a > 0) & (w > 0)
    lam[ok] = a[ok] ** alpha / w[ok] ** (1.0 - alpha)
    return (1.0 / lam).astype(np.float32)


def lowrank_factors(W_hat_kn: np.ndarray, rank: int):
    """Rank-r split of the smoothed weight (K x N) by a thin SVD.

    "SVDQuant" names the decomposition; the 16-bit branch holds "the hardest
    part" of the matrix (dothoosh.com article, SVDQuant paragraph), read as the
    top-r singular triplets. [reading: all of Sigma goes into L1.]
    Returns (L1 [K][r], L2 [r][N], singular values) in float64.
    """
    U, S, Vt = np.linalg.svd(W_hat_kn, full_matrices=False)
    L1 = U[:, :rank] * S[:rank]
    L2 = Vt[:rank, :]
    return L1, L2, S


def prep_svdq_layer(W: np.ndarray, smooth_inv: np.ndarray, rank: int, fmt: str,
                    act_gscale=None, dtype: str = "float16") -> dict:
    """Offline preparation of one SVDQ W4A4 layer.

    W fp16 [N][K]; smooth_inv fp32 [K]. Steps (each a reading of the pages'
    one-sentence description, dothoosh.com article, SVDQuant paragraph):
      1. lambda'_k = 1 / float64(smooth_inv_k) exactly, W_hat = diag(lambda') W_kn,
         so X_hat W_hat = X W holds in real arithmetic.
      2. L1, L2 = rank-r SVD split of W_hat.
      3. lora_down = h16((diag(smooth_inv) L1)^T) [r][K] -- the low-rank branch
         consumes the caller's X directly; lora_up = h16(L2^T) [N][r], with h16
         the compute dtype: fp16, or bf16 (stored as float32 holding bf16 values).
      4. Residual with the rounded factors: R = W_hat - diag(lambda') lora_down^T lora_up^T,
         so the 16-bit rounding of the factors is absorbed by the 4-bit part.
      5. Quantize R^T (N x K) along K with the same rule the activations use;
         for NVFP4 with the per-tensor scale nvfp4_global_scale(max |R|), and
         the activations' per-tensor scale act_gscale (from calibration,
         nvfp4_act_global_scale) is stored with the layer.
    """
    if fmt not in FORMATS:
        raise ValueError(fmt)
    if dtype not in ("float16", "bfloat16"):
        raise ValueError(dtype)
    h16 = (lambda a: a.astype(np.float16)) if dtype == "float16" else \
          (lambda a: bf16_round(a.astype(np.float32)))
    W = np.asarray(W)
    N, K = W.shape
    si64 = np.asarray(smooth_inv, dtype=np.float32).astype(np.float64)
    lam = 1.0 / si64
    W_hat = W.astype(np.float64).T * lam[:, None]                 # K x N
    if rank > 0:
        L1, L2, _ = lowrank_factors(W_hat, rank)
        lora_down = h16((L1 * si64[:, None]).T)                    # r x K
        lora_up = h16(np.ascontiguousarray(L2.T))                  # N x r
        low = (lam[:, None] * lora_down.T.astype(np.float64)) @ lora_up.T.astype(np.float64)
    else:
        lora_down = h16(np.zeros((0, K)))
        lora_up = h16(np.zeros((N, 0)))
        low = 0.0
    R = W_hat - low                                                # K x N
    Rt = np.ascontiguousarray(R.T).astype(np.float32)
    w_gscale = None
    if fmt == "nvfp4_g16":
        if act_gscale is None:
            raise ValueError("nvfp4_g16 needs the activations' per-tensor scale")
        w_gscale = nvfp4_global_scale(np.max(np.abs(Rt)))
        act_gscale = np.float32(act_gscale)
    codes, scales = quantize(Rt, fmt, w_gscale)
    return {
        "act_gscale": act_gscale,
        "w_gscale": w_gscale,
        "fmt": fmt,
        "rank": rank,
        "smooth_inv": np.asarray(smooth_inv, dtype=np.float32),
        "lora_down": np.ascontiguousarray(lora_down),
        "lora_up": lora_up,
        "w_codes": pack_nibbles(codes),
        "w_scales": scales,
        "w_codes_unpacked": codes,
        "residual_kn": R,
    }


# --------------------------------------------------------------------------
# Run-time reference: what the GPU must reproduce.
# --------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round to bfloat16 (8 significant bits, fp32's exponent range) to
    nearest, ties to the even mantissa; returns the values as float32.
    Worked from the fp32 bit pattern: adding 0x7FFF plus the lowest kept bit
    and dropping the low 16 bits is round-half-even on the discarded half
    (a carry moves into the exponent, up to infinity). NaN stays NaN."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(f), f, out).astype(np.float32)


def as_f32_16bit(X16) -> np.ndarray:
    """A 16-bit input (fp16 array, or float32 array holding bf16 values) as float32."""
    X = np.asarray(X16)
    if X.dtype == np.float16:
        return X.astype(np.float32)
    X = X.astype(np.float32)
    if (X.view(np.uint32) & 0xFFFF).any():
        raise ValueError("a float32 16-bit input must hold bfloat16 values")
    return X


def smooth_act(X16: np.ndarray, smooth_inv: np.ndarray) -> np.ndarray:
    """x_hat = fl32(fp32(x) * smooth_inv[k]): one IEEE fp32 multiply, never
    fused with anything (runtime half of outlier migration). X16: fp16, or
    float32 holding bf16 values (the bfloat16 compute dtype)."""
    return as_f32_16bit(X16) * np.asarray(smooth_inv, dtype=np.float32)[None, :]


def quantize_int4_g64(v: np.ndarray):
    """Symmetric INT4 per group of 64 along the last axis.

    Rule [reading; the pages only say 4-bit with a group size]:
      amax = max |v| over the group (exact);
      s32 = fl32(amax / 7) (IEEE division);
      s16 = fp16_rne(min(s32, 65504))  -- stored scale, saturating;
      q = 0 if s16 == 0, else clamp(rint_half_even(fl32(v / fp32(s16))), -7, 7).
    Codes are measured against the stored fp16 scale so that q * s16 is the
    dequantized value. Returns (codes int8 [rows][K], scales fp16 [rows][K/64]).
    """
    v = np.asarray(v, dtype=np.float32)
    rows, K = v.shape
    if K % 64:
        raise ValueError("K must be a multiple of 64")
    g = v.reshape(rows, K // 64, 64)
    amax = np.max(np.abs(g), axis=2)
    s32 = amax / F32(7.0)
    s16 = np.minimum(s32, F32(FP16_MAX)).astype(np.float16)
    s = s16.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        quo = g / s
    q = np.clip(np.rint(quo), -7, 7)
    q = np.where(s == 0, 0, q)
    return q.astype(np.int8).reshape(rows, K), s16


def _e8m0_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with 6 * 2^e >= amax (amax > 0), from the exact
    binary exponent: with e0 = floor(log2 amax), e = e0 - 2 if
    amax <= 1.5 * 2^e0 else e0 - 1."""
    _, ex = np.frexp(amax.astype(np.float64))      # amax = m * 2^ex, m in [0.5, 1)
    e0 = ex.astype(np.int64) - 1
    return np.where(amax.astype(np.float64) <= 1.5 * np.ldexp(1.0, e0), e0 - 2, e0 - 1)


def quantize_fp4_b32(v: np.ndarray):
    """FP4 E2M1 with one E8M0 power-of-two scale per block of 32 along the last axis.

    The pages' float format is NVFP4 with group 16 (dothoosh.com article,
    quantization_config block); the block-32 E8M0 form is the one CDNA4's
    block-scaled matrix instructions consume natively [reading]. Rule:
      amax = max |v| over the block; amax == 0 -> scale code 0, all codes 0;
      else e = the smallest integer with 6 * 2^e >= amax (no clipping),
      clamped to [-127, 127]; scale code = e + 127;
      u = fl32(v / 2^e); magnitude = nearest of {0, .5, 1, 1.5, 2, 3, 4, 6},
      ties to the even mantissa bit, saturating at 6; sign bit = signbit(v)
      (so -0 and small negatives encode as 0x8).
    Nibble = sign << 3 | exponent << 1 | mantissa (OCP E2M1).
    Returns (codes uint8 [rows][K] in 0..15, scales uint8 [rows][K/32]).
    """
    v = np.asarray(v, dtype=np.float32)
    rows, K = v.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    g = v.reshape(rows, K // 32, 32)
    amax = np.max(np.abs(g), axis=2)
    zero = amax == 0
    e = np.clip(_e8m0_exponent(np.where(zero, F32(1.0), amax)), -127, 127)
    scale_code = np.where(zero, 0, e + 127).astype(np.uint8)
    pow2 = np.ldexp(F32(1.0), e.astype(np.int32)).astype(np.float32)[:, :, None]
    code = e2m1_encode(g / pow2)
    code = np.where(zero[:, :, None], 0, code).astype(np.uint8)
    return code.reshape(rows, K), scale_code


def e2m1_encode(u: np.ndarray) -> np.ndarray:
    """fp32 values -> OCP E2M1 nibbles: magnitude = nearest of
    {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even mantissa bit, saturating
    at 6; sign bit = signbit(u)."""
    a = np.abs(np.asarray(u, dtype=np.float32))
    mag = ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
           + (a > 2.5) + (a >= 3.5) + (a > 5.0)).astype(np.uint8)
    return (mag | (np.signbit(u).astype(np.uint8) << 3)).astype(np.uint8)


# --------------------------------------------------------------------------
# NVFP4: E2M1 codes, one E4M3 scale per 16 values, one fp32 scale per tensor.
# --------------------------------------------------------------------------

def e4m3_value(code) -> np.ndarray:
    """OCP FP8 E4M3 (bias 7, no infinities, S.1111.111 is NaN) byte -> float64."""
    c = np.asarray(code, dtype=np.int64)
    sgn = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    val = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.ldexp(1.0, e - 10))
    return np.where((c & 0x7F) == 0x7F, np.nan, sgn * val)


def e4m3_rne(a: np.ndarray) -> np.ndarray:
    """Non-negative fp32 values -> E4M3 byte by round-to-nearest-even,
    saturating at 448 (0x7E). Quantum 2^(e-3) in binade [2^e, 2^(e+1)),
    e >= -6, and 2^-9 below 2^-6; a carry into the next binade is exact."""
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    if (a < 0).any() or np.isnan(a).any():
        raise ValueError("e4m3_rne takes non-negative numbers")
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    q = np.ldexp(1.0, e - 3)
    r = np.rint(a / q) * q                          # exact: a / q is a scaled fp32
    r = np.minimum(r, 448.0)
    # encode r (a representable value) to its byte
    _, er = np.frexp(np.where(r > 0, r, 1.0))
    er = er.astype(np.int64) - 1
    normal = r >= 2.0 ** -6
    code_n = ((er + 7) << 3) | np.rint(r / np.ldexp(1.0, er) * 8 - 8).astype(np.int64)
    code_s = np.rint(r / 2.0 ** -9).astype(np.int64)
    return np.where(normal, code_n, code_s).astype(np.uint8)


def nvfp4_global_scale(amax) -> np.float32:
    """Per-tensor fp32 scale g = fl32(amax / 2688) so that the largest block
    scale lands on the largest E4M3 value [reading: the pages give NVFP4's
    name and group size only; this is the usual two-level recipe]. 1 when
    amax is 0."""
    a = np.float32(amax)
    return np.float32(1.0) if a == 0 else np.float32(a / np.float32(NVFP4_RANGE))


def nvfp4_act_global_scale(X_cal16: np.ndarray, smooth_inv: np.ndarray) -> np.float32:
    """The activations' per-tensor scale, fixed offline from calibration rows
    (the kernels have no whole-tensor pass): g_x = nvfp4_global_scale of the
    largest smoothed calibration value."""
    return nvfp4_global_scale(np.max(np.abs(smooth_act(X_cal16, smooth_inv))))


def quantize_nvfp4_g16(v: np.ndarray, gscale):
    """NVFP4 per block of 16 along the last axis with per-tensor scale g.

    Rule [reading; dothoosh.com article, quantization_config block: precision
    nvfp4, group size 16]:
      amax = max |v| over the block;
      s = E4M3_rne(fl32(amax / fl32(6 g))), saturating at 448;
      d = fl32(E4M3(s) * g); codes = E2M1_rne(fl32(v / d)) (IEEE division),
      all codes 0 where d == 0.
    Value of a code: E2M1(code) * E4M3(s) * g.
    Returns (codes uint8 [rows][K] in 0..15, scales uint8 [rows][K/16]).
    """
    v = np.asarray(v, dtype=np.float32)
    rows, K = v.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    g = np.float32(gscale)
    blk = v.reshape(rows, K // 16, 16)
    amax = np.max(np.abs(blk), axis=2)
    d6 = np.float32(np.float32(6.0) * g)
    sf = (amax / d6).astype(np.float32)
    scode = e4m3_rne(sf)
    d = (e4m3_value(scode).astype(np.float32) * g).astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = (blk / d).astype(np.float32)
    code = np.where(d == 0, 0, e2m1_encode(np.where(d == 0, 0, u))).astype(np.uint8)
    return code.reshape(rows, K), scode


def quantize(v: np.ndarray, fmt: str, gscale=None):
    if fmt == "int4_g64":
        return quantize_int4_g64(v)
    if fmt == "fp4_b32":
        return quantize_fp4_b32(v)
    if fmt == "nvfp4_g16":
        if gscale is None:
            raise ValueError("nvfp4_g16 needs the per-tensor scale")
        return quantize_nvfp4_g16(v, gscale)
    raise ValueError(fmt)


def quantize_act_ref(X16: np.ndarray, smooth_inv: np.ndarray, fmt: str, gscale=None):
    """Smoothing + 4-bit activation quantization. Returns (codes unpacked,
    packed codes u8 [M][K/2], scales). gscale: NVFP4's per-tensor scale."""
    codes, scales = quantize(smooth_act(X16, smooth_inv), fmt, gscale)
    return codes, pack_nibbles(codes), scales


def lora_act_ref(X16: np.ndarray, lora_down: np.ndarray) -> np.ndarray:
    """Low-rank down-projection X . lora_down^T in float64 ([M][r]).
    lora_down already carries diag(smooth_inv) [reading: equal to X_hat L1 in
    real arithmetic with one rounding fewer]."""
    return np.asarray(X16, dtype=np.float64) @ np.asarray(lora_down, dtype=np.float64).T


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: str, gscale=None) -> np.ndarray:
    """Unpacked codes [rows][K] and scales -> float64 values (exact).
    gscale: NVFP4's per-tensor scale."""
    codes = np.asarray(codes)
    rows, K = codes.shape
    G = _group(fmt)
    if fmt == "int4_g64":
        s = np.asarray(scales, dtype=np.float16).astype(np.float64)
        return (codes.astype(np.float64).reshape(rows, K // G, G) * s[:, :, None]).reshape(rows, K)
    c = codes.astype(np.int64)
    mag = E2M1_VALUES[c & 7]
    val = np.where(c & 8, -mag, mag)
    if fmt == "nvfp4_g16":
        p = e4m3_value(scales) * float(np.float32(gscale))
    else:
        p = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)
    return (val.reshape(rows, K // G, G) * p[:, :, None]).reshape(rows, K)


def gelu_tanh(y: np.ndarray) -> np.ndarray:
    """GELU, tanh form, float64: y/2 * (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3)))."""
    y = np.asarray(y, dtype=np.float64)
    return 0.5 * y * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (y + 0.044715 * y ** 3)))


def _finish(y: np.ndarray, bias, epilogue: str) -> np.ndarray:
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    if epilogue == "gelu_tanh":
        return gelu_tanh(y)
    if epilogue != "none":
        raise ValueError(epilogue)
    return y


def gemm_ref(act_codes, act_scales, lora_act, w_codes, w_scales, lora_up, bias,
             fmt: str, epilogue: str = "none", rows=None, cols=None,
             act_gscale=None, w_gscale=None) -> np.ndarray:
    """The fused 4-bit GEMM entry point's contract, float64:
    Y = act(lora_act . lora_up^T + sum_g s_x[m,g] s_w[n,g] (q_x[m,g,:] . q_w[n,g,:]) + bias).

    act_codes / w_codes are unpacked ([M][K], [N][K]); lora_act [M][r] is the
    value handed to the GEMM (the quantizer's fp32 output). rows / cols pick a
    subset of outputs for spot checks at full size. act_gscale / w_gscale are
    NVFP4's per-tensor scales (each dequantized value carries its own).
    """
    ac = np.asarray(act_codes)
    ascl = np.asarray(act_scales)
    la = np.asarray(lora_act, dtype=np.float64)
    wc = np.asarray(w_codes)
    wscl = np.asarray(w_scales)
    lu = np.asarray(lora_up, dtype=np.float64)
    b = None if bias is None else np.asarray(bias, dtype=np.float64)
    if rows is not None:
        ac, ascl, la = ac[rows], ascl[rows], la[rows]
    if cols is not None:
        wc, wscl, lu = wc[cols], wscl[cols], lu[cols]
        b = None if b is None else b[cols]
    Xq = dequantize(ac, ascl, fmt, act_gscale)
    Wq = dequantize(wc, wscl, fmt, w_gscale)
    y = la @ lu.T + Xq @ Wq.T
    return _finish(y, b, epilogue)


def forward_ref(X16, layer: dict, act_codes, act_scales, bias, epilogue: str = "none",
                rows=None, cols=None) -> np.ndarray:
    """Whole-layer reference on given activation codes, float64:
    Y = act((X lora_down^T) lora_up^T + dequant(Q(X_hat)) dequant(Q(R))^T + bias).
    The low-rank branch uses the exact X (not the quantizer's lora_act)."""
    X = np.asarray(X16, dtype=np.float64)
    if rows is not None:
        X = X[rows]
    la = X @ np.asarray(layer["lora_down"], dtype=np.float64).T
    wc = layer["w_codes_unpacked"] if "w_codes_unpacked" in layer else \
        unpack_nibbles(layer["w_codes"], signed=(layer["fmt"] == "int4_g64"))
    return gemm_ref(act_codes if rows is None else np.asarray(act_codes)[rows],
                    act_scales if rows is None else np.asarray(act_scales)[rows],
                    la, wc, layer["w_scales"], layer["lora_up"], bias, layer["fmt"],
                    epilogue, rows=None, cols=cols, act_gscale=layer.get("act_gscale"),
                    w_gscale=layer.get("w_gscale"))


def dense_ref(X16, W16, bias, epilogue: str = "none") -> np.ndarray:
    """The unquantized layer in float64: act(X W^T + b)."""
    y = np.asarray(X16, dtype=np.float64) @ np.asarray(W16, dtype=np.float64).T
    return _finish(y, bias, epilogue)
