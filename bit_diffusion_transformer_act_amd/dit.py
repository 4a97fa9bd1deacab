"""A synthetic DiT transformer block whose linear layers take the 4-bit modules.

The pages describe the quantized model as the dense diffusion transformer
with its linears swapped (dothoosh.com "How Nunchaku Lite halves
diffusion-model VRAM": generic-path paragraph; quantization_config block,
whose targets are the attention projections of the repeated blocks, e.g.
layers.0.self_attention.to_q, and the modulation projection
adaLN_modulation.1; structural-rewrites paragraphs for to_qkv with the Q/K
norm and rotary embedding). The block here has that shape, with the module
names of the pages' example, and no trained weights:

  mod = adaLN_modulation(c) = Linear(SiLU(c))  -> shift, scale, gate (x2)
  x  += gate1 * self_attention(LN(x) (1 + scale1) + shift1, rope)
  x  += gate2 * mlp(LN(x) (1 + scale2) + shift2),  mlp = Linear, GELU(tanh), Linear

Readings (the pages name the modules only): the DiT adaLN-Zero block;
LayerNorm without affine, eps 1e-6; attention heads of 128 channels with
RMSNorm of Q and K (weights, eps 1e-6) and rotation of channel pairs
(2i, 2i+1) by per-token cos/sin; softmax(q k^T / sqrt(128)) v.

The linears run on the library's kernels once quantize_model /
fuse_qkv_norm_rope have swapped them in. The rest of the block (LayerNorm,
modulation arithmetic, attention, residuals) is plain torch arithmetic in
fp32 (fp64 for fp64 inputs): it is not part of the 4-bit linear layers. The
inputs of a 4-bit layer are rounded to its 16-bit compute type (fp16 or
bf16), which those layers take.
"""
from __future__ import annotations

import math

import torch
import torch.nn.functional as F
from torch import nn

from .modules import AWQLinear, SVDQLinear, SVDQLinearQKV

HEAD_DIM = 128


def _glue_dtype(t: torch.Tensor):
    return torch.float64 if t.dtype == torch.float64 else torch.float32


def _linear(mod: nn.Module, x: torch.Tensor) -> torch.Tensor:
    """Apply a dense or 4-bit linear; the result comes back in x's dtype."""
    if isinstance(mod, (SVDQLinear, AWQLinear)):
        return mod(x.to(mod.io_dtype)).to(x.dtype)
    return mod(x.to(mod.weight.dtype)).to(x.dtype)


class RMSNorm(nn.Module):
    """x / sqrt(mean(x^2) + eps) * weight over the last axis."""

    def __init__(self, dim: int, eps: float = 1e-6):
        super().__init__()
        self.eps = eps
        self.weight = nn.Parameter(torch.ones(dim))

    def forward(self, x):
        return x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + self.eps) * self.weight.to(x.dtype)


def apply_rope(x: torch.Tensor, rope: torch.Tensor) -> torch.Tensor:
    """x [B, T, H, 128]; rope [T, 64, 2] (cos, sin per token and channel pair):
    (a, b) -> (a cos - b sin, a sin + b cos) for the pairs (2i, 2i+1)."""
    p = x.unflatten(-1, (HEAD_DIM // 2, 2))
    a, b = p[..., 0], p[..., 1]
    c = rope[..., 0].to(x.dtype)[None, :, None, :]
    s = rope[..., 1].to(x.dtype)[None, :, None, :]
    return torch.stack([a * c - b * s, a * s + b * c], dim=-1).flatten(-2)


class SelfAttention(nn.Module):
    def __init__(self, dim: int, eps: float = 1e-6):
        super().__init__()
        if dim % HEAD_DIM:
            raise ValueError("dim must be a whole number of 128-channel heads")
        self.heads = dim // HEAD_DIM
        self.to_q = nn.Linear(dim, dim)
        self.to_k = nn.Linear(dim, dim)
        self.to_v = nn.Linear(dim, dim)
        self.norm_q = RMSNorm(HEAD_DIM, eps)
        self.norm_k = RMSNorm(HEAD_DIM, eps)
        self.to_out = nn.Linear(dim, dim)

    def forward(self, h: torch.Tensor, rope: torch.Tensor) -> torch.Tensor:
        B, T, D = h.shape
        H = self.heads
        if isinstance(getattr(self, "to_qkv", None), SVDQLinearQKV):
            q, k, v = (t.to(h.dtype).reshape(B, T, H, HEAD_DIM)
                       for t in self.to_qkv(h.to(self.to_qkv.io_dtype), rope))
        else:
            q, k, v = (_linear(m, h).reshape(B, T, H, HEAD_DIM)
                       for m in (self.to_q, self.to_k, self.to_v))
            q = apply_rope(self.norm_q(q), rope)
            k = apply_rope(self.norm_k(k), rope)
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))      # B H T d
        att = torch.softmax(q @ k.transpose(-1, -2).contiguous() / math.sqrt(HEAD_DIM), dim=-1)
        o = (att @ v).transpose(1, 2).reshape(B, T, D)
        return _linear(self.to_out, o)


class DiTBlock(nn.Module):
    """forward(x [B, T, dim], c [B, cond_dim], rope [T, 64, 2]) -> [B, T, dim]."""

    def __init__(self, dim: int, cond_dim: int | None = None, mlp_ratio: int = 4, eps: float = 1e-6):
        super().__init__()
        cond_dim = cond_dim or dim
        self.dim, self.eps = dim, eps
        self.self_attention = SelfAttention(dim, eps)
        self.mlp = nn.Sequential(nn.Linear(dim, mlp_ratio * dim), nn.GELU(approximate="tanh"),
                                 nn.Linear(mlp_ratio * dim, dim))
        self.adaLN_modulation = nn.Sequential(nn.SiLU(), nn.Linear(cond_dim, 6 * dim))

    def _ln(self, x):
        return F.layer_norm(x, (self.dim,), eps=self.eps)

    def forward(self, x: torch.Tensor, c: torch.Tensor, rope: torch.Tensor) -> torch.Tensor:
        gd = _glue_dtype(x)
        xg = x.to(gd)
        mod = _linear(self.adaLN_modulation[1], self.adaLN_modulation[0](c.to(gd)))
        sh1, sc1, g1, sh2, sc2, g2 = mod[:, None, :].chunk(6, dim=-1)
        xg = xg + g1 * self.self_attention(self._ln(xg) * (1 + sc1) + sh1, rope)
        h = self._ln(xg) * (1 + sc2) + sh2
        for m in self.mlp:
            h = _linear(m, h) if isinstance(m, (nn.Linear, SVDQLinear)) else m(h)
        xg = xg + g2 * h
        return xg.to(x.dtype)


class DiTStack(nn.Module):
    """`depth` DiT blocks under the names layers.0, layers.1, ..."""

    def __init__(self, depth: int, dim: int, cond_dim: int | None = None, mlp_ratio: int = 4):
        super().__init__()
        self.layers = nn.ModuleList(DiTBlock(dim, cond_dim, mlp_ratio) for _ in range(depth))

    def forward(self, x, c, rope):
        for blk in self.layers:
            x = blk(x, c, rope)
        return x
