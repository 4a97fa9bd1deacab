"""The optional operands of every GEMM entry point left out (no bias, rank 0,
or both), against the oracle: the null-pointer paths of the INT4 kernel's
tile bands, the FP4 256 x 256 kernel, the NVFP4 kernel, the fused QKV
epilogue and the fused MLP chain. Same bar as the other parity tests:
relative L2 2e-3 against the oracle's float64 result; the chain's codes and
scales bit-exact against the unfused pair."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import LORA_TOL, Y_TOL, assert_close, band_rows, rel_l2  # noqa: F401

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


def _case(fmt, M, K, N, r, epi, seed):
    cfg = synth.LayerConfig(f"opt_{fmt}_{M}_{N}_{r}", 90, M, K, N, r, fmt, epi, "normal", 0.005, 30.0)
    p = synth.random_quantized_layer(cfg, seed=seed)
    cu, packed, scales = oracle.quantize_act_ref(p["X"], p["smooth_inv"], fmt, p.get("act_gscale"))
    la = oracle.lora_act_ref(p["X"], p["lora_down"]).astype(np.float32)
    return p, cu, packed, scales, la


def _ref(p, cu, scales, la, fmt, epi, r, use_bias, rows=None):
    M, N = cu.shape[0], p["w_codes"].shape[0]
    wu = oracle.unpack_nibbles(p["w_codes"], signed=(fmt == "int4_g64"))
    kw = dict(act_gscale=p["act_gscale"], w_gscale=p["w_gscale"]) if fmt == "nvfp4_g16" else {}
    la_o = la if r else np.zeros((M, 0))
    lu_o = p["lora_up"] if r else np.zeros((N, 0))
    return oracle.gemm_ref(cu, scales, la_o, wu, p["w_scales"], lu_o, p["bias"] if use_bias else None, fmt, epi,
                           rows=rows, **kw)


@pytest.mark.parametrize("fmt,M,K,N", [("int4_g64", 2000, 512, 3072),   # 64 x 128 tiles
                                       ("int4_g64", 300, 256, 512),     # 64 x 64 tiles
                                       ("int4_g64", 4096, 256, 4096),   # 128 x 128 tiles
                                       ("fp4_b32", 4096, 512, 4096),    # the 256 x 256 FP4 kernel
                                       ("fp4_b32", 300, 256, 512),      # the 128 x 128 FP4 path
                                       ("nvfp4_g16", 1000, 512, 8448),  # 256-wide NVFP4 tiles
                                       ("nvfp4_g16", 200, 512, 384)])   # 128-wide NVFP4 tiles
@pytest.mark.parametrize("r,use_bias", [(0, False), (16, False), (0, True)])
def test_gemm_without_optional_operands(P, fmt, M, K, N, r, use_bias):
    epi = "gelu_tanh" if (M + N) % 2 == 0 else "none"
    p, cu, packed, scales, la = _case(fmt, M, K, N, r, epi, seed=r + 2 * use_bias)
    la_t = dev(la) if r else None
    lu_t = dev(p["lora_up"]) if r else None
    b_t = dev(p["bias"]) if use_bias else None
    if fmt == "nvfp4_g16":
        alpha = float(np.float32(p["act_gscale"]) * np.float32(p["w_gscale"]))
        Y = P.svdq_gemm_nvfp4(dev(packed), dev(scales), la_t, dev(p["w_codes"]), dev(p["w_scales"]), lu_t, b_t,
                              alpha, epi, dtype=torch.float16)
    else:
        Y = P.svdq_gemm_w4a4(dev(packed), dev(scales), la_t, dev(p["w_codes"]), dev(p["w_scales"]), lu_t, b_t,
                             fmt, epi, dtype=torch.float16)
    y = host(Y)
    assert y.dtype == np.float16 and np.isfinite(y).all()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([rng.choice(M, min(M, 48), replace=False), [0, M - 1]]))
    assert_close(y[rows], _ref(p, cu, scales, la, fmt, epi, r, use_bias, rows=rows))


@pytest.mark.parametrize("r,use_bias", [(0, False), (16, False), (0, True)])
def test_qkv_epilogue_without_optional_operands(P, r, use_bias):
    M, K, N = 200, 512, 768
    p, cu, packed, scales, la = _case("int4_g64", M, K, N, r, "none", seed=5 + r)
    e = synth.qkv_epilogue_inputs(M, seed=5)
    Y = P.svdq_gemm_w4a4_qkv(dev(packed), dev(scales), dev(la) if r else None, dev(p["w_codes"]),
                             dev(p["w_scales"]), dev(p["lora_up"]) if r else None,
                             dev(p["bias"]) if use_bias else None, dev(e["qk_norm_w"]), dev(e["rope"]), e["eps"],
                             dtype=torch.float16)
    y_lin = _ref(p, cu, scales, la, "int4_g64", "none", r, use_bias)
    y_ref = oracle.qkv_epilogue_ref(y_lin, 128, e["qk_norm_w"][0], e["qk_norm_w"][1], e["rope"][..., 0],
                                    e["rope"][..., 1], e["eps"])
    y = host(Y)
    assert np.isfinite(y).all()
    for third in range(3):
        sl = slice(third * N // 3, (third + 1) * N // 3)
        assert_close(y[:, sl], y_ref[:, sl], what=third)


@pytest.mark.parametrize("r,r2", [(0, 16), (16, 0), (0, 0)])
def test_chain_without_bias(P, r, r2):
    """The fused chain with no bias (and rank 0 on either side) equals the
    unfused pair: codes and scales bit for bit, lora_act2 within 1e-3."""
    M, K, N = 200, 512, 1024
    p, cu, packed, scales, la = _case("int4_g64", M, K, N, r, "gelu_tanh", seed=9)
    g = synth.rng_for(9, 91, 7)
    si2 = np.exp(g.normal(0.0, 0.3, N)).astype(np.float32)
    ld2 = (g.standard_normal((r2, N)) * 0.02).astype(np.float16)
    args = (dev(packed), dev(scales), dev(la) if r else None, dev(p["w_codes"]), dev(p["w_scales"]),
            dev(p["lora_up"]) if r else None, None)
    y = P.svdq_gemm_w4a4(*args, "int4_g64", "gelu_tanh", dtype=torch.float16)
    c1, s1, l1 = P.svdq_quantize_act(y, dev(si2), dev(ld2) if r2 else None, "int4_g64")
    c2, s2, l2 = P.svdq_gemm_w4a4_mlp(*args, dev(si2), dev(ld2) if r2 else None, dtype=torch.float16)
    assert np.array_equal(host(c2), host(c1))
    assert np.array_equal(host(s2).view(np.uint16), host(s1).view(np.uint16))
    if r2:
        assert_close(host(l2), host(l1), LORA_TOL)
    else:
        assert l2 is None
    # and the up-projection it quantized is the oracle's
    assert_close(host(y), _ref(p, cu, scales, la, "int4_g64", "gelu_tanh", r, False))
