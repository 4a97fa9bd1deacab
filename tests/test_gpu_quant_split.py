"""The activation quantizer with K split across workgroups (few 16-row blocks,
long K): codes and scales bit-exact against the oracle, lora_act within
tolerance of the oracle's float64 low-rank product (rounded to the 16-bit
type), for every format and both 16-bit types, with and without the low-rank
branch. M = 256 or 200 with K = 8192 gives 16 or 13 row blocks, so the call
cuts K into 4 slices (8 without the low-rank pass) and, with a rank, first
parks the slices' partial sums in the code rows."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import LORA_TOL, assert_close  # noqa: F401

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
H16 = {"float16": torch.float16, "bfloat16": torch.bfloat16}


@pytest.fixture(scope="module")
def P():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_diffusion_transformer_act_amd as pkg
    assert pkg.svdq_device_check(0) == 0, "cuda:0 is not gfx950"
    return pkg


def to16(a, dtype):
    """host float values -> (the oracle's form of the 16-bit values: fp16 array,
    or float32 array holding bf16 values; device tensor)"""
    t = torch.from_numpy(np.asarray(a, np.float32)).to(H16[dtype])
    host = t.numpy() if dtype == "float16" else t.float().numpy()
    return host, t.to(DEV)


@pytest.mark.parametrize("fmt", ["int4_g64", "fp4_b32", "nvfp4_g16"])
@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
@pytest.mark.parametrize("M,r", [(256, 32), (200, 32), (256, 0), (200, 16)])
def test_quantize_act_k_split(P, fmt, dtype, M, r):
    K = 8192
    rng = np.random.default_rng(1000 + M + r)
    X = rng.standard_normal((M, K)) * 1.5
    X[:, rng.choice(K, 40, replace=False)] *= 25.0          # outlier channels
    X[3, :] = 0.0                                            # an all-zero row: zero scales
    si = np.exp(rng.normal(0.0, 0.3, K)).astype(np.float32)
    Xh, Xd = to16(X, dtype)
    ld_h, ld_d = to16(rng.standard_normal((r, K)) * 0.02, dtype) if r else (None, None)
    ga = oracle.nvfp4_act_global_scale(Xh, si) if fmt == "nvfp4_g16" else None
    _, packed_ref, scales_ref = oracle.quantize_act_ref(Xh, si, fmt, ga)
    if fmt == "nvfp4_g16":
        codes, scales, la = P.svdq_quantize_act_nvfp4(Xd, torch.from_numpy(si).to(DEV), ld_d, float(ga))
    else:
        codes, scales, la = P.svdq_quantize_act(Xd, torch.from_numpy(si).to(DEV), ld_d, fmt)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), packed_ref)
    s = scales.cpu().numpy()
    if fmt == "int4_g64":
        assert np.array_equal(s.view(np.uint16), np.asarray(scales_ref, np.float16).view(np.uint16))
    else:
        assert np.array_equal(s, scales_ref)
    if r:
        assert la.dtype == torch.float32
        assert_close(la.cpu().numpy(), oracle.lora_act_ref(Xh, ld_h), LORA_TOL)
        # deterministic: the slices' partials are added in a fixed order
        if fmt == "nvfp4_g16":
            _, _, la2 = P.svdq_quantize_act_nvfp4(Xd, torch.from_numpy(si).to(DEV), ld_d, float(ga))
        else:
            _, _, la2 = P.svdq_quantize_act(Xd, torch.from_numpy(si).to(DEV), ld_d, fmt)
        assert torch.equal(la, la2)
