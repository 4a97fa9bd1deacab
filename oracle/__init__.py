"""CPU oracle for the SVDQuant W4A4 linear layer and the AWQ W4A16 GEMV.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct
numpy implementation of what the HIP library computes. Only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import it; the HIP
library and its Python binding never do, and nothing here calls them.

The method (stated on all five pages, e.g. dothoosh.com "How Nunchaku Lite
halves diffusion-model VRAM", SVDQuant paragraph): activation outliers are
migrated into the weights by a per-channel smoothing, the hardest part of the
smoothed weight is kept as a small 16-bit low-rank branch, and the residual
is quantized to 4 bits; activations are quantized to 4 bits at run time so
the main product is W4A4. The pages give the idea only; every finer rule here
(smoothing formula, how the singular values are split, rounding, scale
formats, nibble order) is a reading, listed in each function's docstring.

Precision: the offline preparation and the forward pass are float64; the
activation and weight quantizers are float32 with IEEE round-to-nearest-even
division and multiplication, exactly as the GPU must reproduce them.

Every function here is pinned by CPU tests against closed forms, invariants,
brute force or hand-worked fixtures (tests/test_oracle_*.py, tests/golden/).
"""
from .svdq import (  # noqa: F401
    FP16_MAX,
    E2M1_VALUES,
    pack_nibbles,
    unpack_nibbles,
    smoothing_factors,
    lowrank_factors,
    prep_svdq_layer,
    smooth_act,
    bf16_round,
    as_f32_16bit,
    quantize_int4_g64,
    quantize_fp4_b32,
    quantize_nvfp4_g16,
    e2m1_encode,
    e4m3_value,
    e4m3_rne,
    nvfp4_global_scale,
    nvfp4_act_global_scale,
    quantize,
    quantize_act_ref,
    lora_act_ref,
    dequantize,
    gelu_tanh,
    gemm_ref,
    forward_ref,
    dense_ref,
)
from .awq import awq_prep, awq_dequantize, gemv_ref  # noqa: F401
from .qkv import rms_norm_heads, rope_pairs, qkv_epilogue_ref  # noqa: F401
from .block import layer_norm, silu, attention, dit_block_ref  # noqa: F401
from .mlp import mlp_chain_ref  # noqa: F401
