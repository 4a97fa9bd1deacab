"""Every entry point at the largest sizes its contract allows, against the
oracle: K = 65536 with rank 128 (the quantizer then cuts K into 8 slices, and
the slices' fp32 low-rank partial sums fill the last slice's code bytes
exactly), N = 65536 (512 tiles of 128 columns, the 4-bit float paths on their
256-wide tiles), and the GEMV at N = 2^20 rows of weights. Ragged M
throughout. Codes and scales bit-exact; lora_act within relative L2 1e-3 of
the oracle's float64 product rounded to fp16; outputs within 2e-3 of the
oracle's float64 layer. The GEMMs take the oracle's lora_act, so every value
the oracle sees comes from the seeded inputs or from the oracle itself."""
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


def _layer_at(P, fmt, M, K, N, r, epi, cols):
    """Quantize X on the GPU (codes and scales checked on every row, lora_act
    against the oracle's), run the GEMM on the GPU's codes and the oracle's
    lora_act, and return (GPU output on all rows and the given columns, the
    oracle's)."""
    cfg = synth.LayerConfig(f"limit_{fmt}_{K}_{N}", 80, M, K, N, r, fmt, epi, "normal", 0.005, 30.0)
    p = synth.random_quantized_layer(cfg, seed=1)
    ga = p.get("act_gscale")
    cu, c_ref, s_ref = oracle.quantize_act_ref(p["X"], p["smooth_inv"], fmt, ga)
    la_o = oracle.lora_act_ref(p["X"], p["lora_down"]).astype(np.float32)
    if fmt == "nvfp4_g16":
        codes, scales, la = P.svdq_quantize_act_nvfp4(dev(p["X"]), dev(p["smooth_inv"]), dev(p["lora_down"]),
                                                      float(ga))
    else:
        codes, scales, la = P.svdq_quantize_act(dev(p["X"]), dev(p["smooth_inv"]), dev(p["lora_down"]), fmt)
    assert np.array_equal(host(codes), c_ref)
    s = host(scales)
    if fmt == "int4_g64":
        assert np.array_equal(s.view(np.uint16), np.asarray(s_ref, np.float16).view(np.uint16))
    else:
        assert np.array_equal(s, s_ref)
    assert_close(host(la), la_o, LORA_TOL)
    if fmt == "nvfp4_g16":
        Y = P.svdq_gemm_nvfp4(codes, scales, dev(la_o), dev(p["w_codes"]), dev(p["w_scales"]), dev(p["lora_up"]),
                              dev(p["bias"]), float(np.float32(ga) * np.float32(p["w_gscale"])), epi)
        kw = dict(act_gscale=ga, w_gscale=p["w_gscale"])
    else:
        Y = P.svdq_gemm_w4a4(codes, scales, dev(la_o), dev(p["w_codes"]), dev(p["w_scales"]), dev(p["lora_up"]),
                             dev(p["bias"]), fmt, epi)
        kw = {}
    y = host(Y)
    assert y.shape == (M, N) and np.isfinite(y).all()
    wu = oracle.unpack_nibbles(p["w_codes"][cols], signed=(fmt == "int4_g64"))
    y_ref = oracle.gemm_ref(cu, s_ref, la_o, wu, p["w_scales"][cols], p["lora_up"][cols], p["bias"][cols], fmt, epi,
                            **kw)
    return y[:, cols], y_ref


@pytest.mark.parametrize("fmt", ["int4_g64", "fp4_b32", "nvfp4_g16"])
def test_largest_k_and_rank(P, fmt):
    """K 65536, rank 128, M 130 (9 row blocks, the last ragged), N 256: all
    outputs."""
    y, y_ref = _layer_at(P, fmt, 130, 65536, 256, 128, "gelu_tanh", np.arange(256))
    assert_close(y, y_ref)


@pytest.mark.parametrize("fmt,K", [("int4_g64", 128), ("fp4_b32", 512), ("nvfp4_g16", 256)])
def test_largest_n(P, fmt, K):
    """N 65536, M 300 (a ragged last row tile), the smallest K of the
    format's wide-tile path; every row, 2049 columns spread over all tiles
    (first and last of each 256 included where sampled)."""
    cols = np.unique(np.concatenate([np.arange(0, 65536, 32), [65535]]))
    y, y_ref = _layer_at(P, fmt, 300, K, 65536, 16, "none", cols)
    assert_close(y, y_ref)


def test_gemv_largest_n(P):
    """The GEMV at N 2^20 (16384 units of 64 rows), M 3, K 64: every output."""
    g = synth.GemvConfig("gemv_limit", 81, 3, 64, 1 << 20, 64)
    p = synth.random_awq_layer(g, seed=2)
    b = (np.random.default_rng(2).standard_normal(g.N) * 0.1).astype(np.float16)
    y = P.awq_gemv_w4a16(dev(p["x"]), dev(p["codes"]), dev(p["scales"]), dev(p["zeros"]), bias=dev(b))
    y_ref = oracle.gemv_ref(p["x"], p["codes"], p["scales"], p["zeros"], bias=b)
    yh = host(y)
    assert yh.shape == (3, 1 << 20) and np.isfinite(yh).all()
    assert_close(yh, y_ref)


def _bf(a):
    """host values -> float32 array of bf16 values (torch's CPU rounding)"""
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def _dbf(a):
    return torch.from_numpy(np.ascontiguousarray(_bf(a))).to(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("fmt", ["int4_g64", "nvfp4_g16"])
def test_largest_k_and_rank_bf16(P, fmt):
    """The same K 65536 / rank 128 layer in the bf16 compute dtype: inputs are
    the seeded draws rounded to bf16, outputs against the oracle's float64
    result rounded to bf16."""
    M, K, N, r = 130, 65536, 256, 128
    cfg = synth.LayerConfig(f"limit_bf_{fmt}", 82, M, K, N, r, fmt, "none", "normal", 0.005, 30.0)
    p = synth.random_quantized_layer(cfg, seed=3)
    X, ld, lu, b = (_bf(p[k].astype(np.float32)) for k in ("X", "lora_down", "lora_up", "bias"))
    ga = oracle.nvfp4_act_global_scale(X, p["smooth_inv"]) if fmt == "nvfp4_g16" else None
    cu, c_ref, s_ref = oracle.quantize_act_ref(X, p["smooth_inv"], fmt, ga)
    la_o = oracle.lora_act_ref(X, ld).astype(np.float32)
    if fmt == "nvfp4_g16":
        codes, scales, la = P.svdq_quantize_act_nvfp4(_dbf(X), dev(p["smooth_inv"]), _dbf(ld), float(ga))
    else:
        codes, scales, la = P.svdq_quantize_act(_dbf(X), dev(p["smooth_inv"]), _dbf(ld), fmt)
    assert np.array_equal(host(codes), c_ref)
    s = host(scales)
    if fmt == "int4_g64":
        assert np.array_equal(s.view(np.uint16), np.asarray(s_ref, np.float16).view(np.uint16))
    else:
        assert np.array_equal(s, s_ref)
    assert_close(la.float().cpu().numpy(), la_o, LORA_TOL)
    if fmt == "nvfp4_g16":
        Y = P.svdq_gemm_nvfp4(codes, scales, dev(la_o), dev(p["w_codes"]), dev(p["w_scales"]), _dbf(lu), _dbf(b),
                              float(np.float32(ga) * np.float32(p["w_gscale"])), "none")
        kw = dict(act_gscale=ga, w_gscale=p["w_gscale"])
    else:
        Y = P.svdq_gemm_w4a4(codes, scales, dev(la_o), dev(p["w_codes"]), dev(p["w_scales"]), _dbf(lu), _dbf(b),
                             fmt, "none")
        kw = {}
    assert Y.dtype == torch.bfloat16
    y = Y.float().cpu().numpy()
    wu = oracle.unpack_nibbles(p["w_codes"], signed=(fmt == "int4_g64"))
    y_ref = oracle.gemm_ref(cu, s_ref, la_o, wu, p["w_scales"], lu, b, fmt, "none", **kw)
    assert_close(y, oracle.bf16_round(y_ref.astype(np.float32)))
