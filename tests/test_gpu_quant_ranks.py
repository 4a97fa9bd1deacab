"""The activation quantizer at every rank it accepts (16 to 128 in steps of
16: 16, 8 and 4 waves per workgroup, and one to eight 16-rank blocks of
lora_down passing through the per-wave re-layout one after the other), for
the three formats, at a ragged M: codes and scales bit-exact against the
oracle, lora_act within relative L2 1e-3 of the oracle's float64 product
rounded to fp16."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import LORA_TOL, assert_close  # noqa: F401

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def P():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_diffusion_transformer_act_amd as pkg
    assert pkg.svdq_device_check(0) == 0, "cuda:0 is not gfx950"
    return pkg


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("fmt", ["int4_g64", "fp4_b32", "nvfp4_g16"])
@pytest.mark.parametrize("r", [16, 32, 48, 64, 80, 96, 112, 128])
def test_quantize_act_every_rank(P, fmt, r):
    M, K = 77, 1536
    rng = np.random.default_rng(500 + r)
    X = rng.standard_normal((M, K)) * 2.0
    X[:, rng.choice(K, 12, replace=False)] *= 20.0
    X = X.astype(np.float16)
    si = np.exp(rng.normal(0.0, 0.3, K)).astype(np.float32)
    ld = (rng.standard_normal((r, K)) * 0.02).astype(np.float16)
    ga = oracle.nvfp4_act_global_scale(X, si) if fmt == "nvfp4_g16" else None
    _, packed_ref, scales_ref = oracle.quantize_act_ref(X, si, fmt, ga)
    if fmt == "nvfp4_g16":
        codes, scales, la = P.svdq_quantize_act_nvfp4(dev(X), dev(si), dev(ld), float(ga))
    else:
        codes, scales, la = P.svdq_quantize_act(dev(X), dev(si), dev(ld), fmt)
    assert np.array_equal(host(codes), packed_ref)
    s = host(scales)
    if fmt == "int4_g64":
        assert np.array_equal(s.view(np.uint16), np.asarray(scales_ref, np.float16).view(np.uint16))
    else:
        assert np.array_equal(s, scales_ref)
    la_ref = oracle.lora_act_ref(X, ld).astype(np.float32)
    assert la.shape == (M, r)
    assert_close(host(la), la_ref, LORA_TOL)
