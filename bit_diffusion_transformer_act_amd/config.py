"""The quantization_config block of a Nunchaku Lite transformer config.

A Nunchaku Lite checkpoint is an ordinary Diffusers repository whose
transformer config.json carries one extra block (dothoosh.com "How Nunchaku
Lite halves diffusion-model VRAM", quantization_config block and the list
that follows it): quant_method "nunchaku_lite", a compute_dtype, and two
sub-blocks, svdq_w4a4 (precision, group_size, rank, targets: the attention and
MLP projections) and awq_w4a16 (precision, group_size, targets: the
modulation / adaptive-norm projections). This module parses and validates
that block against what the MI355X library implements:

  svdq_w4a4 precision "int4" with group_size 64  -> INT4, fp16 scale per 64
  svdq_w4a4 precision "nvfp4" with group_size 16 -> NVFP4: E2M1, E4M3 scale per
                                                    16, fp32 scale per tensor
  svdq_w4a4 precision "mxfp4" with group_size 32 -> FP4 E2M1, E8M0 scale per 32
  awq_w4a16 precision "int4" with group_size 64  -> the AWQ GEMV
  compute_dtype "float16" or "bfloat16"           -> the 16-bit type of the
                                                    activations, the low-rank
                                                    branch, biases and outputs
Target entries are module names; "..." entries (an elision in the pages'
example) are ignored, and shell-style wildcards are accepted.
"""
from __future__ import annotations

import fnmatch
import json
from dataclasses import dataclass


class UnsupportedQuantConfig(ValueError):
    """The block is well formed but asks for something this library does not run."""


@dataclass(frozen=True)
class SvdqSpec:
    fmt: str                  # "int4_g64", "fp4_b32" or "nvfp4_g16"
    rank: int
    targets: tuple


@dataclass(frozen=True)
class AwqSpec:
    group_size: int
    targets: tuple


@dataclass(frozen=True)
class QuantConfig:
    compute_dtype: str
    svdq: SvdqSpec | None
    awq: AwqSpec | None

    def method_for(self, module_name: str) -> str | None:
        """"svdq", "awq" or None for a module name (svdq wins a double match)."""
        for spec, tag in ((self.svdq, "svdq"), (self.awq, "awq")):
            if spec is not None and any(fnmatch.fnmatchcase(module_name, t) for t in spec.targets):
                return tag
        return None


def _targets(block: dict, where: str) -> tuple:
    t = block.get("targets", [])
    if not isinstance(t, (list, tuple)) or not all(isinstance(x, str) for x in t):
        raise ValueError(f"{where}.targets must be a list of module names")
    return tuple(x for x in t if x.strip() not in ("...", "…"))


def parse_quantization_config(cfg) -> QuantConfig:
    """cfg: the transformer config (dict or JSON text) holding a
    "quantization_config" key, or the block itself."""
    if isinstance(cfg, (str, bytes)):
        cfg = json.loads(cfg)
    if not isinstance(cfg, dict):
        raise ValueError("quantization config must be a JSON object")
    q = cfg.get("quantization_config", cfg)
    if q.get("quant_method") != "nunchaku_lite":
        raise ValueError(f"quant_method must be 'nunchaku_lite', got {q.get('quant_method')!r}")
    cdt = q.get("compute_dtype", "float16")
    if cdt in ("bfloat16", "bf16"):
        cdt = "bfloat16"
    elif cdt in ("float16", "fp16", "half"):
        cdt = "float16"
    else:
        raise ValueError(f"unknown compute_dtype {cdt!r}")

    svdq = None
    if "svdq_w4a4" in q:
        b = q["svdq_w4a4"]
        prec, gs, rank = b.get("precision"), b.get("group_size"), b.get("rank", 32)
        if prec == "int4" and gs == 64:
            fmt = "int4_g64"
        elif prec == "nvfp4" and gs == 16:
            fmt = "nvfp4_g16"
        elif prec == "mxfp4" and gs == 32:
            fmt = "fp4_b32"
        else:
            raise UnsupportedQuantConfig(f"svdq_w4a4 precision {prec!r} with group_size {gs!r}")
        if not isinstance(rank, int) or rank < 0 or rank > 128 or rank % 16:
            raise UnsupportedQuantConfig(f"svdq_w4a4 rank {rank!r}: must be a multiple of 16 in [0, 128]")
        svdq = SvdqSpec(fmt, rank, _targets(b, "svdq_w4a4"))

    awq = None
    if "awq_w4a16" in q:
        b = q["awq_w4a16"]
        if b.get("precision", "int4") != "int4" or b.get("group_size", 64) != 64:
            raise UnsupportedQuantConfig("awq_w4a16 must be precision 'int4' with group_size 64")
        awq = AwqSpec(64, _targets(b, "awq_w4a16"))
    if svdq is None and awq is None:
        raise ValueError("quantization_config has neither svdq_w4a4 nor awq_w4a16")
    return QuantConfig(cdt, svdq, awq)
