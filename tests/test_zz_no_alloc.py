"""The allocation-free fused MLP chain (svdq_gemm_w4a4_mlp_noalloc), through
the C ABI, against the chain with a caller workspace (svdq_gemm_w4a4_mlp):
the same kernels on the same inputs, so codes, scales and lora_act2 must be
equal bit for bit. Two calls in a row share the library's device scratch, the
second on a smaller input; then a call without the low-rank branch."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def P():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_diffusion_transformer_act_amd as pkg
    assert pkg.svdq_device_check(0) == 0, "cuda:0 is not gfx950"
    return pkg


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t.to(dtype) if dtype is not None else t


def _case(P, M, K, N, r, r2, seed, h=torch.float16):
    cfg = synth.LayerConfig(f"noalloc_{M}_{K}_{N}", 95, M, K, N, r, "int4_g64", "gelu_tanh", "normal", 0.005, 30.0)
    up = synth.random_quantized_layer(cfg, seed=seed)
    g = synth.rng_for(seed, 96, 7)
    si2 = dev(np.exp(g.normal(0.0, 0.3, N)).astype(np.float32))
    ld2 = dev((g.standard_normal((r2, N)) * 0.02).astype(np.float16), h) if r2 else None
    codes, scales, la = P.svdq_quantize_act(dev(up["X"], h), dev(up["smooth_inv"]),
                                            dev(up["lora_down"][:r], h) if r else None, "int4_g64")
    args = (codes, scales, la, dev(up["w_codes"]), dev(up["w_scales"]),
            dev(np.ascontiguousarray(up["lora_up"][:, :r]), h) if r else None, dev(up["bias"], h), si2, ld2)
    c1, s1, l1 = P.svdq_gemm_w4a4_mlp(*args, dtype=h)
    c2 = torch.full((M, N // 2), 0xAB, dtype=torch.uint8, device=DEV)
    s2 = torch.full((M, N // 64), float("nan"), dtype=torch.float16, device=DEV)
    l2 = torch.full((M, r2), float("nan"), dtype=torch.float32, device=DEV) if r2 else None
    P.svdq_gemm_w4a4_mlp_noalloc(*args, c2, s2, l2, dtype=h)
    torch.cuda.synchronize()
    assert torch.equal(c2, c1)
    assert torch.equal(s2.view(torch.int16), s1.view(torch.int16))
    if r2:
        assert torch.equal(l2.view(torch.int32), l1.view(torch.int32))
    else:
        assert l1 is None


def test_noalloc_chain_equals_workspace_chain(P):
    _case(P, 4096, 3072, 12288, 32, 32, seed=1)                    # the DiT MLP: 48 MiB of partials
    _case(P, 200, 512, 1024, 16, 48, seed=2)                       # smaller, right after: the scratch is shared
    _case(P, 130, 256, 768, 16, 0, seed=3)                         # no low-rank branch: no scratch
    _case(P, 300, 512, 1024, 32, 16, seed=4, h=torch.bfloat16)     # the bf16 compute dtype


def test_noalloc_chain_rejects_sizes_past_the_scratch(P):
    M, N, K = 8192, 12288, 128
    z = lambda *s, dt=torch.uint8: torch.zeros(s, dtype=dt, device=DEV)
    with pytest.raises(P.SvdqError) as e:
        P.svdq_gemm_w4a4_mlp_noalloc(z(M, K // 2), z(M, K // 64, dt=torch.float16), None, z(N, K // 2),
                                     z(N, K // 64, dt=torch.float16), None, None, z(N, dt=torch.float32),
                                     z(32, N, dt=torch.float16), z(M, N // 2), z(M, N // 64, dt=torch.float16),
                                     z(M, 32, dt=torch.float32))
    assert e.value.status == -2
