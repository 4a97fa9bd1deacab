"""torch modules that stand in for nn.Linear: the SVDQ W4A4 linear layer and
the AWQ W4A16 linear layer, plus the patcher that swaps them in.

The generic path of the pages (dothoosh.com "How Nunchaku Lite halves
diffusion-model VRAM", generic-path paragraph; quantization_config block and
the sentence after it) patches the targeted nn.Linear modules of an unchanged
model before the checkpoint is loaded, so the quantized model keeps the dense
model's module names and every tool that walks the module tree still works.
Here `quantize_model` replaces each targeted nn.Linear by an empty
SVDQLinear / AWQLinear of the same name whose buffers (the packed 4-bit
codes, their scales, the low-rank factors, the smoothing vector) are then
filled by `load_state_dict`. The weights are produced offline by the
checkpoint's quantizer; this library only runs them.

Every forward call runs the library's HIP kernels: there is no CPU or
dequantize-to-dense fallback, and a module on a CPU tensor raises.
"""
from __future__ import annotations

import numpy as np
import torch
from torch import nn

from . import ops
from .config import QuantConfig, parse_quantization_config


def _as_rows(x: torch.Tensor, K: int, name: str, dtype=torch.float16) -> torch.Tensor:
    if x.device.type != "cuda":
        raise RuntimeError(f"{name}: input is on {x.device}; the 4-bit kernels run only on a HIP device")
    if x.dtype != dtype:
        raise TypeError(f"{name}: input dtype {x.dtype}, expected {dtype}")
    if x.shape[-1] != K:
        raise ValueError(f"{name}: input has {x.shape[-1]} channels, expected {K}")
    return x.reshape(-1, K).contiguous()


class SVDQLinear(nn.Module):
    """y = x W^T + b with W held as smoothing + low-rank branch + 4-bit residual.

    Buffers (the layout the C ABI takes, N = out_features, K = in_features;
    16-bit ones in the layer's compute dtype, float16 or bfloat16):
      smooth_inv fp32 [K]; lora_down [r][K]; lora_up [N][r];
      w_codes u8 [N][K/2] (even-k code in the low nibble);
      w_scales fp16 [N][K/64] (int4_g64), E8M0 u8 [N][K/32] (fp4_b32) or
      E4M3 u8 [N][K/16] (nvfp4_g16);
      bias [N] when bias=True;
      nvfp4_g16 only: act_gscale and w_gscale, fp32 scalars (the per-tensor
      scales of the activations, fixed from calibration, and of the weight).
    epilogue "gelu_tanh" applies the tanh-approximated GELU inside the GEMM.
    """

    def __init__(self, in_features: int, out_features: int, rank: int = 32,
                 fmt: str = "int4_g64", bias: bool = True, epilogue: str = "none",
                 device=None, dtype=torch.float16):
        super().__init__()
        if dtype not in (torch.float16, torch.bfloat16):
            raise ValueError("the compute dtype is torch.float16 or torch.bfloat16")
        self.io_dtype = dtype
        if fmt not in ops.ALL_FORMATS:
            raise ValueError(f"unknown format {fmt!r}")
        if epilogue not in ops.EPILOGUES:
            raise ValueError(f"unknown epilogue {epilogue!r}")
        if in_features % 128 or out_features % 128:
            raise ValueError("SVDQLinear needs in_features and out_features divisible by 128")
        if fmt == "nvfp4_g16" and in_features % 256:
            raise ValueError("nvfp4_g16 needs in_features divisible by 256")
        if rank % 16 or not 0 <= rank <= 128:
            raise ValueError("rank must be a multiple of 16 in [0, 128]")
        K, N = in_features, out_features
        self.in_features, self.out_features, self.rank = K, N, rank
        self.fmt, self.epilogue = fmt, epilogue
        sdt, sg = {"int4_g64": (torch.float16, 64), "fp4_b32": (torch.uint8, 32),
                   "nvfp4_g16": (torch.uint8, 16)}[fmt]
        kw = {"device": device}
        self.register_buffer("smooth_inv", torch.ones(K, dtype=torch.float32, **kw))
        self.register_buffer("lora_down", torch.zeros(rank, K, dtype=dtype, **kw))
        self.register_buffer("lora_up", torch.zeros(N, rank, dtype=dtype, **kw))
        self.register_buffer("w_codes", torch.zeros(N, K // 2, dtype=torch.uint8, **kw))
        self.register_buffer("w_scales", torch.zeros(N, K // sg, dtype=sdt, **kw))
        if bias:
            self.register_buffer("bias", torch.zeros(N, dtype=dtype, **kw))
        else:
            self.bias = None
        if fmt == "nvfp4_g16":
            # fp32 scalars kept on the host: the kernels take them by value, and
            # reading a device scalar would synchronize every call
            self.register_buffer("act_gscale", torch.ones((), dtype=torch.float32))
            self.register_buffer("w_gscale", torch.ones((), dtype=torch.float32))
            self._gs, self._alpha = (1.0, 1.0), 1.0
            self.register_load_state_dict_post_hook(SVDQLinear._cache_gscales)

    @staticmethod
    def _cache_gscales(module, incompatible_keys):
        a, w = np.float32(module.act_gscale.cpu()), np.float32(module.w_gscale.cpu())
        module._gs = (float(a), float(w))
        module._alpha = float(a * w)        # the fp32 product the GEMM scales its 4-bit sum by

    def _apply(self, fn, *args, **kwargs):
        # the per-tensor scales stay on the host whatever device the module moves to
        out = super()._apply(fn, *args, **kwargs)
        if self.fmt == "nvfp4_g16":
            self.act_gscale = self.act_gscale.cpu()
            self.w_gscale = self.w_gscale.cpu()
        return out

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"rank={self.rank}, fmt={self.fmt}, epilogue={self.epilogue}, dtype={self.io_dtype}")

    def quantize_input(self, x: torch.Tensor):
        """The first fused call: 4-bit codes, scales and the low-rank activation."""
        X = _as_rows(x, self.in_features, "SVDQLinear", self.io_dtype)
        ld = self.lora_down if self.rank else None
        if self.fmt == "nvfp4_g16":
            return ops.svdq_quantize_act_nvfp4(X, self.smooth_inv, ld, self._gs[0])
        return ops.svdq_quantize_act(X, self.smooth_inv, ld, self.fmt)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        codes, scales, la = self.quantize_input(x)
        lu = self.lora_up if self.rank else None
        if self.fmt == "nvfp4_g16":
            y = ops.svdq_gemm_nvfp4(codes, scales, la, self.w_codes, self.w_scales, lu, self.bias,
                                    self._alpha, self.epilogue, dtype=self.io_dtype)
        else:
            y = ops.svdq_gemm_w4a4(codes, scales, la, self.w_codes, self.w_scales, lu, self.bias,
                                   self.fmt, self.epilogue, dtype=self.io_dtype)
        return y.reshape(*x.shape[:-1], self.out_features)


class SVDQLinearQKV(SVDQLinear):
    """The fused to_qkv of the pages' structural rewrite (dothoosh.com article,
    structural-rewrites paragraphs): to_q, to_k and to_v concatenated along the
    output dimension in Q, K, V order, with the per-head RMSNorm of Q and K
    (heads of 128 channels, weights qk_norm_w fp16 [2][128]: row 0 for Q,
    row 1 for K) and the rotation of channel pairs (2i, 2i+1) done in the GEMM
    epilogue. forward(x, rope) takes rope fp32 [tokens][64][2] (cos, sin per
    token and pair) broadcast over the leading batch dimensions of x, or
    [rows][64][2] for every row, and returns q, k, v of [..., dim] each.
    Only the int4_g64 format has the fused epilogue."""

    def __init__(self, dim: int, rank: int = 32, fmt: str = "int4_g64", bias: bool = True,
                 eps: float = 1e-6, device=None, dtype=torch.float16):
        if fmt != "int4_g64":
            raise ValueError("the fused QKV epilogue is built for int4_g64 only")
        if dim % 128:
            raise ValueError("dim must be a whole number of 128-channel heads")
        super().__init__(dim, 3 * dim, rank, fmt, bias, "none", device, dtype)
        self.dim, self.eps = dim, float(eps)
        self.register_buffer("qk_norm_w", torch.ones(2, 128, dtype=dtype, device=device))

    def forward(self, x: torch.Tensor, rope: torch.Tensor):
        codes, scales, la = self.quantize_input(x)
        M = codes.shape[0]
        if rope.dim() != 3 or tuple(rope.shape[1:]) != (64, 2) or M % rope.shape[0]:
            raise ValueError(f"rope must be [tokens][64][2] with tokens dividing {M} rows")
        rope = rope.to(torch.float32)
        if rope.shape[0] != M:
            rope = rope.repeat(M // rope.shape[0], 1, 1)
        y = ops.svdq_gemm_w4a4_qkv(codes, scales, la, self.w_codes, self.w_scales,
                                   self.lora_up if self.rank else None, self.bias,
                                   self.qk_norm_w, rope.contiguous(), self.eps, self.fmt,
                                   dtype=self.io_dtype)
        y = y.reshape(*x.shape[:-1], 3 * self.dim)
        return y.split(self.dim, dim=-1)


class AWQLinear(nn.Module):
    """y = x W^T + b with W held as AWQ 4-bit codes: w = (q - z) s per group of
    64 along K. Buffers: w_codes u8 [N][K/2] (unsigned, even-k code in the low
    nibble), scales and zeros fp16 [N][K/64], bias [N] in the compute dtype
    (float16 or bfloat16, that of the input). For the
    memory-bound modulation projections: at most 8 rows per call of the GEMV,
    larger inputs go through it 8 rows at a time."""

    MAX_ROWS = 8

    def __init__(self, in_features: int, out_features: int, group_size: int = 64,
                 bias: bool = True, device=None, dtype=torch.float16):
        super().__init__()
        if dtype not in (torch.float16, torch.bfloat16):
            raise ValueError("the compute dtype is torch.float16 or torch.bfloat16")
        self.io_dtype = dtype
        if group_size != 64:
            raise ValueError("AWQLinear supports group_size 64")
        if in_features % 64:
            raise ValueError("in_features must be a multiple of 64")
        K, N = in_features, out_features
        self.in_features, self.out_features, self.group_size = K, N, group_size
        kw = {"device": device}
        self.register_buffer("w_codes", torch.zeros(N, K // 2, dtype=torch.uint8, **kw))
        self.register_buffer("scales", torch.zeros(N, K // 64, dtype=torch.float16, **kw))
        self.register_buffer("zeros", torch.zeros(N, K // 64, dtype=torch.float16, **kw))
        if bias:
            self.register_buffer("bias", torch.zeros(N, dtype=dtype, **kw))
        else:
            self.bias = None

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, group_size=64, "
                f"dtype={self.io_dtype}")

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        X = _as_rows(x, self.in_features, "AWQLinear", self.io_dtype)
        M, N = X.shape[0], self.out_features
        rows = max(1, min(self.MAX_ROWS, 32768 // self.in_features))
        y = torch.empty((M, N), dtype=self.io_dtype, device=X.device)
        for m0 in range(0, M, rows):
            ops.awq_gemv_w4a16(X[m0:m0 + rows], self.w_codes, self.scales, self.zeros, 64,
                               out=y[m0:m0 + rows], bias=self.bias)
        return y.reshape(*x.shape[:-1], N)


def _set_child(root: nn.Module, name: str, new: nn.Module):
    parent_name, _, leaf = name.rpartition(".")
    parent = root.get_submodule(parent_name) if parent_name else root
    setattr(parent, leaf, new)


def quantize_model(model: nn.Module, config, device=None, fuse_gelu: bool = True) -> list:
    """Replace the nn.Linear modules named by config's targets, in place.

    config: a QuantConfig, or the transformer config / quantization_config
    block as a dict or JSON text. A module named by svdq_w4a4 becomes an
    SVDQLinear, by awq_w4a16 an AWQLinear; the rest stay dense. With
    fuse_gelu, an nn.GELU(approximate="tanh") that directly follows an
    SVDQLinear inside an nn.Sequential moves into that layer's GEMM epilogue
    and is replaced by nn.Identity. Returns the names replaced. Buffers are
    empty: fill them with load_state_dict.
    """
    q = config if isinstance(config, QuantConfig) else parse_quantization_config(config)
    io = torch.bfloat16 if q.compute_dtype == "bfloat16" else torch.float16
    done = []
    for name, mod in list(model.named_modules()):
        if not isinstance(mod, nn.Linear):
            continue
        how = q.method_for(name)
        if how is None:
            continue
        dev = device if device is not None else mod.weight.device
        has_bias = mod.bias is not None
        if how == "svdq":
            new = SVDQLinear(mod.in_features, mod.out_features, q.svdq.rank, q.svdq.fmt,
                             has_bias, device=dev, dtype=io)
        else:
            new = AWQLinear(mod.in_features, mod.out_features, q.awq.group_size, has_bias,
                            device=dev, dtype=io)
        _set_child(model, name, new)
        done.append(name)
    if fuse_gelu:
        for seq in model.modules():
            if not isinstance(seq, nn.Sequential):
                continue
            kids = list(seq._modules.items())
            for (_, a), (bname, b) in zip(kids, kids[1:]):
                if (isinstance(a, SVDQLinear) and a.epilogue == "none"
                        and type(a) is SVDQLinear and isinstance(b, nn.GELU)
                        and b.approximate == "tanh"):
                    a.epilogue = "gelu_tanh"
                    seq._modules[bname] = nn.Identity()
    return done


def _norm_pair_hook(module, state_dict, prefix, local_metadata, strict, missing, unexpected, errors):
    """Load-time adapter: the dense checkpoint's norm_q.weight / norm_k.weight
    become the fused module's qk_norm_w rows."""
    kq, kk = prefix + "norm_q.weight", prefix + "norm_k.weight"
    if kq in state_dict and kk in state_dict:
        wq, wk = state_dict.pop(kq), state_dict.pop(kk)
        # load_state_dict converts to the buffer's own dtype
        state_dict.setdefault(prefix + "to_qkv.qk_norm_w", torch.stack([wq.reshape(-1), wk.reshape(-1)]))


def fuse_qkv_norm_rope(model: nn.Module) -> list:
    """The structural rewrite of the pages (dothoosh.com article,
    structural-rewrites paragraphs), in place: every module whose to_q, to_k
    and to_v are int4_g64 SVDQLinear layers of one width and whose norm_q /
    norm_k hold 128-element RMSNorm weights gets a single SVDQLinearQKV named
    to_qkv instead (Q, K, V concatenated along the output axis, in that
    order), and loses those five children. A load_state_dict pre-hook moves a
    checkpoint's norm_q.weight / norm_k.weight into to_qkv.qk_norm_w. The
    4-bit weights of to_qkv are those of the concatenated projection (one
    smoothing vector and one low-rank branch for the three), as the
    quantizer's grouped target config produces them. Returns the names of the
    rewritten modules."""
    done = []
    for name, mod in list(model.named_modules()):
        parts = [getattr(mod, a, None) for a in ("to_q", "to_k", "to_v")]
        nq, nk = getattr(mod, "norm_q", None), getattr(mod, "norm_k", None)
        if not all(type(p) is SVDQLinear for p in parts) or nq is None or nk is None:
            continue
        q = parts[0]
        if any(p.fmt != "int4_g64" or p.in_features != q.in_features or p.out_features != q.in_features
               or p.rank != q.rank or (p.bias is None) != (q.bias is None) or p.io_dtype != q.io_dtype
               for p in parts):
            continue
        if getattr(nq, "weight", None) is None or nq.weight.numel() != 128 or nk.weight.numel() != 128:
            continue
        eps = float(getattr(nq, "eps", 1e-6) or 1e-6)
        fused = SVDQLinearQKV(q.in_features, q.rank, q.fmt, q.bias is not None, eps,
                              device=q.w_codes.device, dtype=q.io_dtype)
        with torch.no_grad():
            fused.qk_norm_w.copy_(torch.stack([nq.weight.reshape(-1), nk.weight.reshape(-1)]))
        for a in ("to_q", "to_k", "to_v", "norm_q", "norm_k"):
            delattr(mod, a)
        mod.to_qkv = fused
        mod.register_load_state_dict_pre_hook(_norm_pair_hook)
        done.append(name)
    return done
