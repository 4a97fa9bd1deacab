"""MI355X (gfx950) SVDQuant W4A4 linear layer and AWQ W4A16 GEMV.

The kernels live in the HIP library libsvdq_mi355x.so (C ABI in
include/svdq.h); this package is its thin torch binding. Build the library
with bit_diffusion_transformer_act_amd.build.build().
"""
from .ops import (  # noqa: F401
    EPILOGUES,
    EXPORTED_SYMBOLS,
    FORMATS,
    SvdqError,
    awq_gemv_w4a16,
    lib,
    svdq_clock_probe,
    svdq_device_check,
    svdq_gemm_w4a4,
    svdq_gemm_w4a4_qkv,
    svdq_gemm_w4a4_splitk,
    svdq_gemm_w4a4_splitk_workspace,
    svdq_gemm_w4a4_mlp,
    svdq_gemm_w4a4_mlp_noalloc,
    svdq_gemm_nvfp4,
    svdq_quantize_act_nvfp4,
    svdq_linear,
    svdq_quantize_act,
    svdq_status_str,
    svdq_version,
)
