"""Oracle for the synthetic DiT block that drives the 4-bit linear layers end
to end.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages describe the quantized model as the dense diffusion transformer
with its linears swapped: the attention and MLP projections of the repeated
blocks to SVDQ W4A4, the modulation projection adaLN_modulation.1 to AWQ
W4A16, optionally to_q/to_k/to_v fused with the Q/K norm and rotary embedding
(dothoosh.com "How Nunchaku Lite halves diffusion-model VRAM",
quantization_config block and its target names; structural-rewrites
paragraphs). They name the modules, not the block; the readings used here
are those of the DiT adaLN-Zero block:

  mod = W_mod SiLU(c) + b_mod, split into shift1, scale1, gate1, shift2, scale2, gate2
  h   = LN(x) (1 + scale1) + shift1
  q, k, v = projections of h; q, k RMS-normalised per 128-channel head
            (weights, eps 1e-6) and rotated pairwise by the token's cos / sin
  x   = x + gate1 * to_out(softmax(q k^T / sqrt(128)) v)        (per head)
  h   = LN(x) (1 + scale2) + shift2
  x   = x + gate2 * (W_2 GELU_tanh(W_1 h + b_1) + b_2)            (mlp.0, mlp.2)

with LN the LayerNorm without affine parameters, eps 1e-6.

Each linear is an entry of `params`:
  {"kind": "dense", "W": [N][K], "b": [N] | None}       exact, float64, no rounding
  {"kind": "svdq", "layer": prep_svdq_layer(...), "b": fp16 [N] | None,
   "epilogue": "none" | "gelu_tanh"}
  {"kind": "svdq_qkv", "layer": ..., "b": ..., "qk_norm_w": fp16 [2][128], "eps": float}
  {"kind": "awq", "awq": awq_prep(...), "b": fp16 [N] | None}
plus "self_attention.norm_q" / "self_attention.norm_k" weight arrays when Q,
K and V are separate. A 4-bit entry may carry "dtype": "bfloat16" (default
"float16"): the layer's 16-bit type. A 4-bit layer takes its input rounded to
that type and returns its output rounded to it (the storage types of the
layers); the rest is float64.
"""
from __future__ import annotations

import numpy as np

from .awq import gemv_ref
from .qkv import qkv_epilogue_ref, rms_norm_heads, rope_pairs
from .svdq import bf16_round, forward_ref, gelu_tanh, quantize_act_ref

HEAD_DIM = 128


def _r16(a, dtype: str = "float16") -> np.ndarray:
    """Round to the layer's 16-bit type: fp16 array, or float32 holding bf16 values."""
    a = np.asarray(a, dtype=np.float64)
    if dtype == "bfloat16":
        return bf16_round(a.astype(np.float32))
    return a.astype(np.float16)


def layer_norm(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) over the last axis (biased variance)."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """q, k, v [B][T][H][d] -> softmax over keys of q k^T / sqrt(d), times v,
    per batch and head; [B][T][H][d]."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    d = q.shape[-1]
    s = np.einsum("bthd,bshd->bhts", q, k) / np.sqrt(d)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.einsum("bhts,bshd->bthd", p, v)


def linear(x: np.ndarray, e: dict, rope=None) -> np.ndarray:
    """One linear of the block on rows x [M][K] -> [M][N] float64."""
    kind = e["kind"]
    if kind == "dense":
        y = np.asarray(x, dtype=np.float64) @ np.asarray(e["W"], dtype=np.float64).T
        return y if e.get("b") is None else y + np.asarray(e["b"], dtype=np.float64)
    dt = e.get("dtype", "float16")
    X16 = _r16(x, dt)
    if kind == "awq":
        a = e["awq"]
        return _r16(gemv_ref(X16, a["codes"], a["scales"], a["zeros"], a["group"], bias=e.get("b")), dt)
    layer = e["layer"]
    codes, _, scales = quantize_act_ref(X16, layer["smooth_inv"], layer["fmt"], layer.get("act_gscale"))
    if kind == "svdq":
        return _r16(forward_ref(X16, layer, codes, scales, e.get("b"), e.get("epilogue", "none")), dt)
    if kind == "svdq_qkv":
        y = forward_ref(X16, layer, codes, scales, e.get("b"))
        w = np.asarray(e["qk_norm_w"])
        return _r16(qkv_epilogue_ref(y, HEAD_DIM, w[0], w[1], rope[..., 0], rope[..., 1], e["eps"]), dt)
    raise ValueError(kind)


def _rope_heads(y: np.ndarray, rope_rows: np.ndarray, weight) -> np.ndarray:
    """RMSNorm per head then pairwise rotation, y [M][H*d]."""
    y = rms_norm_heads(y, HEAD_DIM, weight, 1e-6)
    return rope_pairs(y, HEAD_DIM, rope_rows[..., 0], rope_rows[..., 1])


def dit_block_ref(x, c, rope, params: dict, eps: float = 1e-6, capture: dict | None = None,
                  outputs: dict | None = None):
    """x [B][T][D], c [B][C], rope [T][64][2] -> block output [B][T][D] float64.

    capture, when given, receives (input rows, output rows) of each linear
    under its name, float64, the input before any rounding. outputs, when
    given, supplies the output rows of the linears it names in place of
    computing them (teacher forcing: the rest of the block then runs on those
    values), so the block's own arithmetic can be checked apart from the
    4-bit layers."""
    x = np.asarray(x, dtype=np.float64)
    B, T, D = x.shape
    H = D // HEAD_DIM
    rope_rows = np.tile(np.asarray(rope, dtype=np.float64), (B, 1, 1))        # [B*T][64][2]

    def lin(name, rows, **kw):
        if outputs is not None and name in outputs:
            y = np.array(outputs[name], dtype=np.float64).reshape(rows.shape[0], -1)
        else:
            # the layer's 16-bit values, carried on in float64 like the rest of the block
            y = np.asarray(linear(rows, params[name], **kw), dtype=np.float64)
        if capture is not None:
            capture[name] = (np.array(rows, dtype=np.float64), y)
        return y

    mod = lin("adaLN_modulation.1", silu(c))                                   # [B][6D]
    sh1, sc1, g1, sh2, sc2, g2 = (m[:, None, :] for m in np.split(mod, 6, axis=-1))

    h = (layer_norm(x, eps) * (1 + sc1) + sh1).reshape(B * T, D)
    if "self_attention.to_qkv" in params:
        y = lin("self_attention.to_qkv", h, rope=rope_rows)
        q, k, v = y[:, :D], y[:, D:2 * D], y[:, 2 * D:]
    else:
        q = _rope_heads(lin("self_attention.to_q", h), rope_rows, params["self_attention.norm_q"])
        k = _rope_heads(lin("self_attention.to_k", h), rope_rows, params["self_attention.norm_k"])
        v = lin("self_attention.to_v", h)
    o = attention(*(t.reshape(B, T, H, HEAD_DIM) for t in (q, k, v))).reshape(B * T, D)
    x = x + g1 * lin("self_attention.to_out", o).reshape(B, T, D)

    h = (layer_norm(x, eps) * (1 + sc2) + sh2).reshape(B * T, D)
    u = lin("mlp.0", h)
    if params["mlp.0"].get("epilogue", "none") != "gelu_tanh":
        u = gelu_tanh(u)
    x = x + g2 * lin("mlp.2", u).reshape(B, T, D)
    return x
