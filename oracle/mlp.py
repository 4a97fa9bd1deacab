"""Oracle for the fused MLP chain: the MLP up-projection with GELU, whose
output goes straight into the down-projection's activation quantizer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages list GELU / MLP kernels among the model-specific fused paths of
the full engine (dothoosh.com "How Nunchaku Lite halves diffusion-model
VRAM", generic-path paragraph). Reading: the fused chain computes exactly
what the two unfused steps compute, without storing the up-projection's
output — the up-projection's 16-bit output U (GELU applied) is the input of
the down-projection's quantizer (its smoothing, low-rank down-projection and
4-bit activation quantization), so the contract is the composition of the
pinned functions below, and nothing else.
"""
from __future__ import annotations

import numpy as np

from .svdq import bf16_round, gemm_ref, lora_act_ref, quantize_act_ref


def mlp_chain_ref(act_codes, act_scales, lora_act, w_codes, w_scales, lora_up, bias, fmt: str,
                  smooth_inv2, lora_down2, fmt2: str = "int4_g64", dtype: str = "float16", rows=None):
    """Up-projection (codes unpacked, as gemm_ref takes them) with GELU, then the
    down-projection's quantizer. Returns (U16 [M][N], codes2 unpacked,
    codes2 packed, scales2, lora_act2 float64 [M][r2]); with rows, only those
    rows (every row of the chain is independent of the others)."""
    y = gemm_ref(act_codes, act_scales, lora_act, w_codes, w_scales, lora_up, bias, fmt, "gelu_tanh",
                 rows=rows)
    U16 = bf16_round(y.astype(np.float32)) if dtype == "bfloat16" else y.astype(np.float16)
    codes, packed, scales = quantize_act_ref(U16, smooth_inv2, fmt2)
    return U16, codes, packed, scales, lora_act_ref(U16, lora_down2)
