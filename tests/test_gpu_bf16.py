"""The bfloat16 compute dtype (the pages' compute_dtype) on the GPU against the
oracle, for every entry point: codes and scales bit-exact; layer, GEMM,
fused-QKV and GEMV outputs against the oracle's float64 result rounded to bf16
(the output type is part of the contract), lora_act (fp32 in both dtypes)
against the unrounded result: relative L2 within 1e-3 for lora_act and 2e-3
for outputs, and the per-element bound of tests/parity.py. bf16 inputs are the seeded fp16/fp32 draws
rounded to bf16 by torch's CPU conversion (input preparation)."""
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


def bf(a):
    """host values -> float32 array of bf16 values (torch's CPU rounding)"""
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def dbf(a):
    return torch.from_numpy(np.ascontiguousarray(bf(a))).to(torch.bfloat16).to(DEV)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


_cache = {}


def bf_layer(fmt, M=256, K=512, N=512, r=16, seed=0):
    key = (fmt, M, K, N, r, seed)
    if key not in _cache:
        cfg = synth.LayerConfig(f"bf_{fmt}_{M}_{K}_{N}", 60, M, K, N, r, fmt, "none", "normal", 0.01, 30.0)
        d = synth.make_layer_inputs(cfg, seed=seed)
        X = bf(d["X"].astype(np.float32))
        Xc = bf(d["X_cal"].astype(np.float32))
        si = oracle.smoothing_factors(Xc, d["W"], 0.5)
        ga = oracle.nvfp4_act_global_scale(Xc, si) if fmt == "nvfp4_g16" else None
        layer = oracle.prep_svdq_layer(d["W"], si, r, fmt, act_gscale=ga, dtype="bfloat16")
        _cache[key] = (X, bf(d["bias"].astype(np.float32)), si, ga, layer, d["W"])
    return _cache[key]


def quantize(P, fmt, X, si, ld, ga):
    if fmt == "nvfp4_g16":
        return P.svdq_quantize_act_nvfp4(dbf(X), dev(si), dbf(ld) if ld is not None else None, float(ga))
    return P.svdq_quantize_act(dbf(X), dev(si), dbf(ld) if ld is not None else None, fmt)


@pytest.mark.parametrize("fmt", ["int4_g64", "fp4_b32", "nvfp4_g16"])
@pytest.mark.parametrize("M,r", [(256, 16), (37, 0)])
def test_quantize_act_bf16(P, fmt, M, r):
    X, _, si, ga, layer, _ = bf_layer(fmt, M=M, r=r)
    _, packed_ref, scales_ref = oracle.quantize_act_ref(X, si, fmt, ga)
    codes, scales, la = quantize(P, fmt, X, si, layer["lora_down"] if r else None, ga)
    assert np.array_equal(host(codes), packed_ref)
    sc = host(scales)
    if fmt == "int4_g64":
        assert np.array_equal(sc.view(np.uint16), np.asarray(scales_ref, np.float16).view(np.uint16))
    else:
        assert np.array_equal(sc, scales_ref)
    if r:
        assert la.dtype == torch.float32
        la_ref = oracle.lora_act_ref(X, layer["lora_down"])
        assert_close(host(la), la_ref, LORA_TOL)


def _gemm(P, fmt, layer, packed, scales, la, b, epi, alpha=None):
    lu = dbf(layer["lora_up"]) if layer["rank"] else None
    la_t = dev(la) if layer["rank"] else None
    if fmt == "nvfp4_g16":
        return P.svdq_gemm_nvfp4(dev(packed), dev(scales), la_t, dev(layer["w_codes"]), dev(layer["w_scales"]),
                                 lu, dbf(b), alpha, epi, dtype=torch.bfloat16)
    return P.svdq_gemm_w4a4(dev(packed), dev(scales), la_t, dev(layer["w_codes"]), dev(layer["w_scales"]),
                            lu, dbf(b), fmt, epi, dtype=torch.bfloat16)


@pytest.mark.parametrize("fmt,M,N,epi", [("int4_g64", 200, 512, "none"), ("int4_g64", 256, 512, "gelu_tanh"),
                                         ("fp4_b32", 200, 512, "gelu_tanh"), ("nvfp4_g16", 300, 384, "none"),
                                         ("nvfp4_g16", 256, 512, "gelu_tanh")])
def test_gemm_bf16(P, fmt, M, N, epi):
    X, b, si, ga, layer, _ = bf_layer(fmt, M=M, N=N, r=16)
    cu, packed, scales = oracle.quantize_act_ref(X, si, fmt, ga)
    la = oracle.lora_act_ref(X, layer["lora_down"]).astype(np.float32)
    alpha = float(np.float32(ga) * np.float32(layer["w_gscale"])) if fmt == "nvfp4_g16" else None
    y = _gemm(P, fmt, layer, packed, scales, la, b, epi, alpha)
    assert y.dtype == torch.bfloat16
    y_ref = oracle.gemm_ref(cu, scales, la, layer["w_codes_unpacked"], layer["w_scales"], layer["lora_up"], b,
                            fmt, epi, act_gscale=ga, w_gscale=layer.get("w_gscale"))
    assert_close(host(y), oracle.bf16_round(y_ref.astype(np.float32)))


def test_gemm_fp4_large_tile_bf16(P):
    """The 256 x 256 FP4 kernel (N % 256, K % 512, at least 256 tiles) in bf16,
    on sampled outputs."""
    cfg = synth.LayerConfig("bf_fp4_big", 61, 4096, 512, 4096, 32, "fp4_b32", "gelu_tanh", "normal", 0.005, 30.0)
    p = synth.random_quantized_layer(cfg, seed=1)
    X = bf(p["X"].astype(np.float32))
    ld, lu, b = bf(p["lora_down"].astype(np.float32)), bf(p["lora_up"].astype(np.float32)), bf(p["bias"].astype(np.float32))
    codes, scales, la = P.svdq_quantize_act(dbf(X), dev(p["smooth_inv"]), dbf(ld), "fp4_b32")
    # the GEMM takes the oracle's low-rank activations, the GPU's checked against them
    la_o = oracle.lora_act_ref(X, ld).astype(np.float32)
    assert_close(host(la), la_o, LORA_TOL)
    y = P.svdq_gemm_w4a4(codes, scales, dev(la_o), dev(p["w_codes"]), dev(p["w_scales"]), dbf(lu), dbf(b),
                         "fp4_b32", "gelu_tanh")
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(cfg.M, 16, replace=False))
    cols = np.sort(rng.choice(cfg.N, 64, replace=False))
    cu, c_ref, s_ref = oracle.quantize_act_ref(X[rows], p["smooth_inv"], "fp4_b32")
    assert np.array_equal(host(codes)[rows], c_ref)
    wu = oracle.unpack_nibbles(p["w_codes"][cols], signed=False)
    y_ref = oracle.gemm_ref(cu, s_ref, la_o[rows], wu, p["w_scales"][cols], lu[cols], b[cols], "fp4_b32",
                            "gelu_tanh")
    assert_close(host(y)[np.ix_(rows, cols)], oracle.bf16_round(y_ref.astype(np.float32)))


def test_gemm_qkv_bf16(P):
    M, K, H = 200, 512, 2
    N = 3 * H * 128
    X, b, si, _, layer, _ = bf_layer("int4_g64", M=M, K=K, N=N, r=16, seed=3)
    e = synth.qkv_epilogue_inputs(M, seed=3)
    qkw = bf(e["qk_norm_w"].astype(np.float32))
    cu, packed, scales = oracle.quantize_act_ref(X, si, "int4_g64")
    la = oracle.lora_act_ref(X, layer["lora_down"]).astype(np.float32)
    y = P.svdq_gemm_w4a4_qkv(dev(packed), dev(scales), dev(la), dev(layer["w_codes"]), dev(layer["w_scales"]),
                             dbf(layer["lora_up"]), dbf(b), dbf(qkw), dev(e["rope"]), e["eps"])
    assert y.dtype == torch.bfloat16
    lin = oracle.gemm_ref(cu, scales, la, layer["w_codes_unpacked"], layer["w_scales"], layer["lora_up"], b,
                          "int4_g64")
    y_ref = oracle.qkv_epilogue_ref(lin, 128, qkw[0], qkw[1], e["rope"][..., 0], e["rope"][..., 1], e["eps"])
    assert_close(host(y), oracle.bf16_round(y_ref.astype(np.float32)))


@pytest.mark.parametrize("M,K,N", [(1, 3072, 18432), (6, 2048, 333)])
def test_awq_gemv_bf16(P, M, K, N):
    g = synth.GemvConfig(f"gemv_bf{K}", 44, 1, K, N, 64)
    p = synth.random_awq_layer(g, seed=9, M=M)
    x = bf(p["x"].astype(np.float32))
    b = bf(np.random.default_rng(4).normal(0, 1.0, N).astype(np.float32))
    y = P.awq_gemv_w4a16(dbf(x), dev(p["codes"]), dev(p["scales"]), dev(p["zeros"]), bias=dbf(b))
    assert y.dtype == torch.bfloat16
    y_ref = oracle.gemv_ref(x, p["codes"], p["scales"], p["zeros"], bias=b)
    assert_close(host(y), oracle.bf16_round(y_ref.astype(np.float32)))


def test_mixed_dtypes_rejected(P):
    X, _, si, _, layer, _ = bf_layer("int4_g64")
    with pytest.raises(TypeError):
        P.svdq_quantize_act(dbf(X), dev(si), dev(layer["lora_down"].astype(np.float16)), "int4_g64")
