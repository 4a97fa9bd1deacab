"""Oracle for the AWQ W4A16 GEMV used by the modulation / adaptive-norm
projections: 4-bit weights, 16-bit activations, memory-bound (dothoosh.com
"How Nunchaku Lite halves diffusion-model VRAM", kernel-family list, the
awq_w4a16 entry; quantization_config block: precision int4, group size 64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Storage [reading: the pages give none]: codes u8 [N][K/2], unsigned nibbles,
the even-k code in the low nibble; scales and zeros fp16 [N][K/G]; the
weight is w = (q - z) * s with z in code units.
"""
from __future__ import annotations

import numpy as np

from .svdq import pack_nibbles, unpack_nibbles


def awq_prep(W16: np.ndarray, group: int = 64) -> dict:
    """Asymmetric min-max 4-bit quantization per (row n, group g) in float64.

    [reading: AWQ's activation-aware scale search needs calibration data the
    pages do not give; any (q, s, z) is a valid GEMV input, so plain min-max
    is used.] s = fp16((max - min) / 15) (1 where that is 0);
    z = clamp(rint(-min / s), 0, 15) as fp16; q = clamp(rint(w / s) + z, 0, 15).
    """
    W = np.asarray(W16, dtype=np.float64)
    N, K = W.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    g = W.reshape(N, K // group, group)
    mn = g.min(axis=2)
    mx = g.max(axis=2)
    s16 = ((mx - mn) / 15.0).astype(np.float16)
    s16 = np.where(s16 == 0, np.float16(1.0), s16)
    s = s16.astype(np.float64)
    z = np.clip(np.rint(-mn / s), 0, 15)
    q = np.clip(np.rint(g / s[:, :, None]) + z[:, :, None], 0, 15).astype(np.int64)
    q = q.reshape(N, K)
    return {"codes": pack_nibbles(q), "codes_unpacked": q.astype(np.uint8),
            "scales": s16, "zeros": z.astype(np.float16), "group": group}


def awq_dequantize(codes_packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                   group: int = 64) -> np.ndarray:
    """(q - z) * s per element, float64, [N][K]."""
    q = unpack_nibbles(codes_packed, signed=False).astype(np.float64)
    N, K = q.shape
    s = np.asarray(scales, dtype=np.float64)
    z = np.asarray(zeros, dtype=np.float64)
    return ((q.reshape(N, K // group, group) - z[:, :, None]) * s[:, :, None]).reshape(N, K)


def gemv_ref(x16: np.ndarray, codes_packed: np.ndarray, scales: np.ndarray,
             zeros: np.ndarray, group: int = 64, bias=None) -> np.ndarray:
    """y[m,n] = sum_k x[m,k] (q[n,k] - z[n,k/G]) s[n,k/G] (+ bias[n]), float64 [M][N]."""
    Wd = awq_dequantize(codes_packed, scales, zeros, group)
    y = np.asarray(x16, dtype=np.float64) @ Wd.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y
