"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This package draws random numbers and lays them out; it holds none of the
quantization method's arithmetic (no smoothing, no SVD, no quantizer, no
forward). Both sides receive the same arrays from here.
"""
from .inputs import (  # noqa: F401
    BLOCK_STREAM,
    CONFIGS,
    LayerConfig,
    GemvConfig,
    rng_for,
    outlier_channels,
    make_layer_inputs,
    make_gemv_inputs,
    random_quantized_layer,
    random_awq_layer,
    qkv_epilogue_inputs,
    dit_block_params,
    dit_block_inputs,
)
