"""Seeded synthetic workloads for the SVDQuant W4A4 linear layer and the
AWQ W4A16 modulation GEMV.

The pages measure whole text-to-image pipelines on trained checkpoints, which
are not available here; these draws stand in for them with DiT-shaped layers
(hidden size 3072, 4096 image tokens at 1024x1024) and the activation outlier
structure that motivates the method (a few input channels carrying values
tens of times larger than the rest; dothoosh.com "How Nunchaku Lite halves
diffusion-model VRAM", paragraph on why outliers make 4-bit hard).

Every array comes from numpy's PCG64 seeded with SeedSequence([seed, cfg_id,
stream]); streams: 0 = X, 1 = W, 2 = bias, 3 = outlier-channel choice,
4 = calibration X, 5 = GEMV x, 6 = GEMV W, 7 = synthetic quantized
parameters for timing runs, 8 = Q/K norm weights of the fused QKV epilogue,
9 = dense weights of the synthetic DiT block, 10 = its inputs.

Nothing here computes the method: no smoothing, no SVD, no quantization and
no forward pass.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

STREAM_X, STREAM_W, STREAM_BIAS, STREAM_OUTLIERS, STREAM_XCAL = 0, 1, 2, 3, 4
STREAM_GEMV_X, STREAM_GEMV_W, STREAM_QPARAMS, STREAM_QKV_EPI = 5, 6, 7, 8
STREAM_DIT_W, STREAM_DIT_X = 9, 10
DIT_CFG_ID = 20


@dataclass(frozen=True)
class LayerConfig:
    """One SVDQ W4A4 linear layer workload (X: M x K, W: N x K, rank r)."""
    name: str
    cfg_id: int
    M: int
    K: int
    N: int
    rank: int
    fmt: str            # "int4_g64", "fp4_b32" or "nvfp4_g16"
    epilogue: str       # "none", "gelu_tanh" or "qkv_norm_rope"
    x_dist: str         # "normal" or "gelu_normal"
    outlier_frac: float
    outlier_scale: float
    w_std: float = 0.02
    bias_std: float = 0.01
    alpha: float = 0.5

    @property
    def group(self) -> int:
        return {"int4_g64": 64, "fp4_b32": 32, "nvfp4_g16": 16}[self.fmt]


@dataclass(frozen=True)
class GemvConfig:
    """One AWQ W4A16 GEMV workload (x: M x K, W: N x K, group along K)."""
    name: str
    cfg_id: int
    M: int
    K: int
    N: int
    group: int = 64
    w_std: float = 0.02


CONFIGS = {
    # Tiny single layer, small enough for the oracle's SVD and exact checks.
    "tiny": LayerConfig("tiny", 0, 256, 512, 512, 16, "int4_g64", "none",
                        "normal", 0.01, 50.0),
    # DiT attention QKV projection, Q,K,V concatenated along the output dim.
    "qkv": LayerConfig("qkv", 1, 4096, 3072, 9216, 32, "int4_g64", "none",
                       "normal", 0.005, 30.0),
    # The same projection with the per-head Q/K RMSNorm and rotary embedding fused
    # into its epilogue (24 heads of 128 per third).
    "qkv_normrope": LayerConfig("qkv_normrope", 11, 4096, 3072, 9216, 32, "int4_g64",
                                "qkv_norm_rope", "normal", 0.005, 30.0),
    # DiT MLP up-projection in FP4 E2M1 with block-32 E8M0 scales, GELU(tanh).
    "mlp_up": LayerConfig("mlp_up", 2, 4096, 3072, 12288, 32, "fp4_b32",
                          "gelu_tanh", "normal", 0.005, 30.0),
    # DiT MLP down-projection; input is a GELU output.
    "mlp_down": LayerConfig("mlp_down", 3, 4096, 12288, 3072, 32, "int4_g64",
                            "none", "gelu_normal", 0.005, 30.0),
    # Same at a 512x512 image (1024 tokens): exposes low-rank overhead.
    "mlp_down_m1024": LayerConfig("mlp_down_m1024", 31, 1024, 12288, 3072, 32,
                                  "int4_g64", "none", "gelu_normal", 0.005, 30.0),
    # The two remaining linears of one DiT block, INT4 (block stream).
    "attn_out": LayerConfig("attn_out", 41, 4096, 3072, 3072, 32, "int4_g64",
                            "none", "normal", 0.005, 30.0),
    "mlp_up_int4": LayerConfig("mlp_up_int4", 42, 4096, 3072, 12288, 32,
                               "int4_g64", "gelu_tanh", "normal", 0.005, 30.0),
    # The MLP up-projection in the pages' own float format: NVFP4 (E2M1, E4M3
    # scale per 16, fp32 scale per tensor), GELU(tanh).
    "mlp_up_nvfp4": LayerConfig("mlp_up_nvfp4", 43, 4096, 3072, 12288, 32,
                                "nvfp4_g16", "gelu_tanh", "normal", 0.005, 30.0),
    # Modulation projection of a DiT block: six 3072-wide vectors at M = 1.
    "gemv": GemvConfig("gemv", 4, 1, 3072, 18432, 64),
}

# The linear stream of one DiT block at 4096 tokens, hidden 3072.
BLOCK_STREAM = ("qkv", "attn_out", "mlp_up_int4", "mlp_down")


def rng_for(seed: int, cfg_id: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg_id, stream])))


def outlier_channels(K: int, frac: float, rng: np.random.Generator) -> np.ndarray:
    """Sorted indices of round-half-even(frac*K) distinct input channels."""
    n_out = int(np.rint(frac * K))
    return np.sort(rng.permutation(K)[:n_out])


def _gelu_erf(z: np.ndarray) -> np.ndarray:
    # Input recipe only (the exact erf form); unrelated to the layer's epilogue.
    from scipy.special import erf
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def _draw_x(cfg: LayerConfig, rows: int, outl: np.ndarray, rng: np.random.Generator) -> np.ndarray:
    z = rng.standard_normal((rows, cfg.K))
    if cfg.x_dist == "gelu_normal":
        z = _gelu_erf(z)
    elif cfg.x_dist != "normal":
        raise ValueError(cfg.x_dist)
    z[:, outl] *= cfg.outlier_scale
    return z.astype(np.float16)


def make_layer_inputs(cfg: LayerConfig, seed: int = 0, M: int | None = None,
                      cal_rows: int | None = None) -> dict:
    """X fp16 [M][K], W fp16 [N][K] (nn.Linear layout), bias fp16 [N],
    X_cal fp16 [cal_rows][K] (independent draw, same outlier channels)."""
    M = cfg.M if M is None else M
    outl = outlier_channels(cfg.K, cfg.outlier_frac, rng_for(seed, cfg.cfg_id, STREAM_OUTLIERS))
    X = _draw_x(cfg, M, outl, rng_for(seed, cfg.cfg_id, STREAM_X))
    W = (rng_for(seed, cfg.cfg_id, STREAM_W).standard_normal((cfg.N, cfg.K)) * cfg.w_std).astype(np.float16)
    bias = (rng_for(seed, cfg.cfg_id, STREAM_BIAS).standard_normal(cfg.N) * cfg.bias_std).astype(np.float16)
    cal_rows = min(cfg.M, 1024) if cal_rows is None else cal_rows
    X_cal = _draw_x(cfg, cal_rows, outl, rng_for(seed, cfg.cfg_id, STREAM_XCAL))
    return {"X": X, "W": W, "bias": bias, "X_cal": X_cal, "outliers": outl}


def make_gemv_inputs(cfg: GemvConfig, seed: int = 0, M: int | None = None) -> dict:
    """x fp16 [M][K] ~ N(0,1); W fp16 [N][K] ~ N(0, w_std^2)."""
    M = cfg.M if M is None else M
    x = rng_for(seed, cfg.cfg_id, STREAM_GEMV_X).standard_normal((M, cfg.K)).astype(np.float16)
    W = (rng_for(seed, cfg.cfg_id, STREAM_GEMV_W).standard_normal((cfg.N, cfg.K)) * cfg.w_std).astype(np.float16)
    return {"x": x, "W": W}


def _nibble_bytes(lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    return ((lo.astype(np.uint8) & 0xF) | ((hi.astype(np.uint8) & 0xF) << 4)).astype(np.uint8)


def random_quantized_layer(cfg: LayerConfig, seed: int = 0, M: int | None = None) -> dict:
    """Random, plausibly scaled layer parameters in the library's storage
    formats, for timing runs and for GEMM checks that do not need a
    calibrated weight. Codes are uniform over the format's values, scales
    sit where a N(0, 0.02^2) weight would put them.

    Returns X fp16 [M][K], smooth_inv fp32 [K], lora_down fp16 [r][K],
    w_codes u8 [N][K/2], w_scales (fp16 [N][K/64] or u8 [N][K/32]),
    lora_up fp16 [N][r], bias fp16 [N].
    """
    M = cfg.M if M is None else M
    K, N, r = cfg.K, cfg.N, cfg.rank
    g = rng_for(seed, cfg.cfg_id, STREAM_QPARAMS)
    outl = outlier_channels(K, cfg.outlier_frac, rng_for(seed, cfg.cfg_id, STREAM_OUTLIERS))
    X = _draw_x(cfg, M, outl, rng_for(seed, cfg.cfg_id, STREAM_X))
    smooth_inv = np.exp(g.normal(0.0, 0.3, K)).astype(np.float32)
    smooth_inv[outl] /= np.float32(np.sqrt(cfg.outlier_scale))
    lora_down = (g.standard_normal((r, K)) * 0.02).astype(np.float16)
    lora_up = (g.standard_normal((N, r)) * 0.1).astype(np.float16)
    bias = (g.standard_normal(N) * cfg.bias_std).astype(np.float16)
    if cfg.fmt == "int4_g64":
        # the whole two's-complement range: -8 is a valid weight code for the GEMM
        # even though the symmetric quantizer never produces it
        lo = g.integers(-8, 8, (N, K // 2))
        hi = g.integers(-8, 8, (N, K // 2))
        w_scales = (g.uniform(0.004, 0.01, (N, K // 64))).astype(np.float16)
    elif cfg.fmt == "fp4_b32":
        lo = g.integers(0, 16, (N, K // 2))
        hi = g.integers(0, 16, (N, K // 2))
        w_scales = g.integers(119, 123, (N, K // 32)).astype(np.uint8)
    elif cfg.fmt == "nvfp4_g16":
        # E4M3 block scales spread over the upper binades (the per-tensor scale
        # puts the largest block near 448), per-tensor scales of an N(0, 0.02^2)
        # weight and of activations whose largest smoothed value is about 50
        lo = g.integers(0, 16, (N, K // 2))
        hi = g.integers(0, 16, (N, K // 2))
        w_scales = g.integers(0x50, 0x7F, (N, K // 16)).astype(np.uint8)
    else:
        raise ValueError(cfg.fmt)
    out = {"X": X, "smooth_inv": smooth_inv, "lora_down": lora_down,
           "w_codes": _nibble_bytes(lo, hi), "w_scales": w_scales,
           "lora_up": lora_up, "bias": bias}
    if cfg.fmt == "nvfp4_g16":
        out["w_gscale"] = np.float32(0.1 / 2688.0)
        out["act_gscale"] = np.float32(50.0 / 2688.0)
    return out


def random_awq_layer(cfg: GemvConfig, seed: int = 0, M: int | None = None) -> dict:
    """Random AWQ parameters in storage format: x fp16 [M][K], codes u8
    [N][K/2] (unsigned nibbles), scales fp16 [N][K/G], zeros fp16 [N][K/G]
    (integers 0..15)."""
    M = cfg.M if M is None else M
    g = rng_for(seed, cfg.cfg_id, STREAM_QPARAMS)
    x = rng_for(seed, cfg.cfg_id, STREAM_GEMV_X).standard_normal((M, cfg.K)).astype(np.float16)
    lo = g.integers(0, 16, (cfg.N, cfg.K // 2))
    hi = g.integers(0, 16, (cfg.N, cfg.K // 2))
    scales = g.uniform(0.004, 0.01, (cfg.N, cfg.K // cfg.group)).astype(np.float16)
    zeros = g.integers(0, 16, (cfg.N, cfg.K // cfg.group)).astype(np.float16)
    return {"x": x, "codes": _nibble_bytes(lo, hi), "scales": scales, "zeros": zeros}


def qkv_epilogue_inputs(M: int, seed: int = 0, head_dim: int = 128) -> dict:
    """Inputs of the fused QKV epilogue: RMSNorm weights of Q and K (fp16, near
    1) and rotary tables for M image tokens. The tokens are taken as a
    ceil(sqrt(M))-wide grid in row-major order; the first half of the channel
    pairs rotate with the token's row, the second half with its column
    (per-axis rotary embedding of image DiTs), frequencies 10000^(-j/(P/2)) for
    pair j of each half (P = head_dim / 2 pairs). rope is fp32 [M][P][2] (cos, sin);
    eps is the RMSNorm epsilon."""
    g = rng_for(seed, 0, STREAM_QKV_EPI)
    q_w = (1.0 + 0.1 * g.standard_normal(head_dim)).astype(np.float16)
    k_w = (1.0 + 0.1 * g.standard_normal(head_dim)).astype(np.float16)
    P = head_dim // 2
    side = int(math.ceil(math.sqrt(max(M, 1))))
    m = np.arange(M)
    row, col = (m // side).astype(np.float64), (m % side).astype(np.float64)
    half = P // 2
    freq = 10000.0 ** (-np.arange(half) / half)
    theta = np.concatenate([row[:, None] * freq[None, :], col[:, None] * freq[None, :]], axis=1)
    rope = np.stack([np.cos(theta), np.sin(theta)], axis=-1).astype(np.float32)
    return {"qk_norm_w": np.stack([q_w, k_w]), "rope": np.ascontiguousarray(rope), "eps": 1e-6}


def dit_block_params(dim: int, cond_dim: int | None = None, mlp_ratio: int = 4,
                     seed: int = 0) -> dict:
    """Dense weights of one synthetic DiT block, fp16 numpy arrays keyed by the
    torch parameter names (nn.Linear layout [out][in]): linears N(0, 1/in),
    biases N(0, 0.02^2), RMSNorm weights near 1, and a modulation projection
    scaled so that shift, scale and gate come out around 0.2."""
    cond_dim = cond_dim or dim
    g = rng_for(seed, DIT_CFG_ID, STREAM_DIT_W)
    hid = mlp_ratio * dim
    shapes = {"self_attention.to_q": (dim, dim), "self_attention.to_k": (dim, dim),
              "self_attention.to_v": (dim, dim), "self_attention.to_out": (dim, dim),
              "mlp.0": (hid, dim), "mlp.2": (dim, hid)}
    out = {}
    for name, (n, k) in shapes.items():
        out[name + ".weight"] = (g.standard_normal((n, k)) / math.sqrt(k)).astype(np.float16)
        out[name + ".bias"] = (g.standard_normal(n) * 0.02).astype(np.float16)
    for name in ("self_attention.norm_q", "self_attention.norm_k"):
        out[name + ".weight"] = (1.0 + 0.1 * g.standard_normal(128)).astype(np.float16)
    out["adaLN_modulation.1.weight"] = (g.standard_normal((6 * dim, cond_dim)) * 0.01).astype(np.float16)
    out["adaLN_modulation.1.bias"] = (g.standard_normal(6 * dim) * 0.02).astype(np.float16)
    return out


def dit_block_inputs(B: int, T: int, dim: int, cond_dim: int | None = None, seed: int = 0,
                     outlier_frac: float = 0.01, outlier_scale: float = 20.0) -> dict:
    """x fp16 [B][T][dim]: N(0, 1) with a few channels scaled up (outliers
    that survive LayerNorm); c fp16 [B][cond_dim] ~ N(0, 1); rope fp32
    [T][64][2] from qkv_epilogue_inputs over a grid of T tokens."""
    cond_dim = cond_dim or dim
    g = rng_for(seed, DIT_CFG_ID, STREAM_DIT_X)
    outl = outlier_channels(dim, outlier_frac, g)
    x = g.standard_normal((B, T, dim))
    x[..., outl] *= outlier_scale
    c = g.standard_normal((B, cond_dim))
    rope = qkv_epilogue_inputs(T, seed)["rope"]
    return {"x": x.astype(np.float16), "c": c.astype(np.float16), "rope": rope}
