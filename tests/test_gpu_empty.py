"""Zero rows through every entry point of the binding on the GPU: each call
returns outputs with no rows (and the right trailing shapes and dtypes)
without launching anything or raising."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def P():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_diffusion_transformer_act_amd as pkg
    assert pkg.svdq_device_check(0) == 0, "cuda:0 is not gfx950"
    return pkg


def z(*shape, dt=torch.float16):
    return torch.zeros(shape, dtype=dt, device=DEV)


@pytest.mark.parametrize("fmt", ["int4_g64", "fp4_b32"])
def test_quantize_and_gemm_no_rows(P, fmt):
    K, N, r = 512, 256, 16
    si = torch.ones(K, dtype=torch.float32, device=DEV)
    codes, scales, la = P.svdq_quantize_act(z(0, K), si, z(r, K), fmt)
    assert codes.shape == (0, K // 2) and codes.dtype == torch.uint8
    assert scales.shape[0] == 0 and la.shape == (0, r)
    ws = z(N, K // 64) if fmt == "int4_g64" else z(N, K // 32, dt=torch.uint8)
    Y = P.svdq_gemm_w4a4(codes, scales, la, z(N, K // 2, dt=torch.uint8), ws, z(N, r), z(N), fmt, "gelu_tanh")
    assert Y.shape == (0, N) and Y.dtype == torch.float16
    torch.cuda.synchronize()


def test_qkv_and_chain_no_rows(P):
    K, N, r = 512, 768, 16
    si = torch.ones(K, dtype=torch.float32, device=DEV)
    codes, scales, la = P.svdq_quantize_act(z(0, K), si, z(r, K), "int4_g64")
    wc, ws = z(N, K // 2, dt=torch.uint8), z(N, K // 64)
    Y = P.svdq_gemm_w4a4_qkv(codes, scales, la, wc, ws, z(N, r), z(N), z(2, 128),
                             z(0, 64, 2, dt=torch.float32), 1e-6)
    assert Y.shape == (0, N)
    c2, s2, l2 = P.svdq_gemm_w4a4_mlp(codes, scales, la, wc, ws, z(N, r), z(N),
                                      torch.ones(N, dtype=torch.float32, device=DEV), z(16, N))
    assert c2.shape == (0, N // 2) and s2.shape == (0, N // 64) and l2.shape == (0, 16)
    torch.cuda.synchronize()


def test_nvfp4_no_rows(P):
    K, N, r = 512, 256, 16
    si = torch.ones(K, dtype=torch.float32, device=DEV)
    codes, scales, la = P.svdq_quantize_act_nvfp4(z(0, K, dt=torch.bfloat16), si, z(r, K, dt=torch.bfloat16), 0.5)
    assert codes.shape == (0, K // 2) and scales.shape == (0, K // 16) and la.shape == (0, r)
    Y = P.svdq_gemm_nvfp4(codes, scales, la, z(N, K // 2, dt=torch.uint8), z(N, K // 16, dt=torch.uint8),
                          z(N, r, dt=torch.bfloat16), z(N, dt=torch.bfloat16), 1.0, "none")
    assert Y.shape == (0, N) and Y.dtype == torch.bfloat16
    torch.cuda.synchronize()


def test_gemv_no_rows(P):
    K, N = 3072, 1000
    y = P.awq_gemv_w4a16(z(0, K), z(N, K // 2, dt=torch.uint8), z(N, K // 64), z(N, K // 64))
    assert y.shape == (0, N)
    torch.cuda.synchronize()
    assert np.asarray(y.cpu()).size == 0
