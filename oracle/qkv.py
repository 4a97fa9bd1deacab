"""Oracle for the fused QKV epilogue: per-head RMSNorm of Q and K and rotary
position embedding, applied to the output of a fused Q|K|V projection.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source. The pages list, among the structural rewrites the Nunchaku Lite
loader applies to a pipeline, one that fuses the QKV projection with the Q/K
normalisation and the rotary embedding (dothoosh.com "How Nunchaku Lite
halves diffusion-model VRAM", structural-rewrites paragraph, the rewrite
spelled fused_qkv_norm_rottary there), alongside fusing Q, K and V into one
projection. The pages name the rewrite only; the readings used here:

  - Q, K and V are concatenated along the output axis, each H heads of D
    channels (the DiT shapes: hidden 3072 = 24 heads of 128);
  - the norm is RMSNorm over the D channels of each head of Q and of K,
    x / sqrt(mean(x^2) + eps) * w[d], with one learned weight vector for Q
    and one for K (shared by the heads), eps = 1e-6 by default;
  - the rotary embedding rotates the channel pairs (2i, 2i+1) of every Q and
    K head by a per-token angle: (a, b) -> (a cos - b sin, a sin + b cos),
    with cos and sin given per token and pair (so any position scheme, 1-D or
    per-axis 2-D/3-D for image tokens, is the caller's table);
  - the bias of the projection is added before the norm; V passes unchanged.

Everything is float64.
"""
from __future__ import annotations

import numpy as np


def rms_norm_heads(y: np.ndarray, head_dim: int, weight: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over each head of head_dim channels along the last axis:
    y / sqrt(mean over the head of y^2 + eps) * weight (weight [head_dim])."""
    y = np.asarray(y, dtype=np.float64)
    lead = y.shape[:-1]
    h = y.reshape(*lead, -1, head_dim)
    ms = np.mean(h * h, axis=-1, keepdims=True)
    out = h / np.sqrt(ms + eps) * np.asarray(weight, dtype=np.float64)
    return out.reshape(y.shape)


def rope_pairs(y: np.ndarray, head_dim: int, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate channel pairs (2i, 2i+1) of every head of y [M][H*head_dim] by the
    token's angle: cos, sin are [M][head_dim / 2]."""
    y = np.asarray(y, dtype=np.float64)
    M = y.shape[0]
    h = y.reshape(M, -1, head_dim // 2, 2)
    a, b = h[..., 0], h[..., 1]
    c = np.asarray(cos, dtype=np.float64)[:, None, :]
    s = np.asarray(sin, dtype=np.float64)[:, None, :]
    out = np.stack([a * c - b * s, a * s + b * c], axis=-1)
    return out.reshape(y.shape)


def qkv_epilogue_ref(y_lin: np.ndarray, head_dim: int, q_norm_w: np.ndarray, k_norm_w: np.ndarray,
                     cos: np.ndarray, sin: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """y_lin [M][3 H head_dim] (projection output with bias) -> Q and K parts
    RMS-normalised per head and rotated; V part unchanged."""
    y = np.asarray(y_lin, dtype=np.float64)
    n = y.shape[1]
    assert n % (3 * head_dim) == 0
    third = n // 3
    q = rope_pairs(rms_norm_heads(y[:, :third], head_dim, q_norm_w, eps), head_dim, cos, sin)
    k = rope_pairs(rms_norm_heads(y[:, third:2 * third], head_dim, k_norm_w, eps), head_dim, cos, sin)
    return np.concatenate([q, k, y[:, 2 * third:]], axis=1)
