"""NVFP4 (E2M1 codes, E4M3 scale per 16, fp32 scale per tensor) on the GPU
against the oracle: activation codes and scales bit-exact, lora_act within
1e-3, GEMM and layer outputs within relative L2 2e-3 of the float64 oracle
on the same codes; both tile widths of the GEMM (N % 256 and N % 128), a
ragged M, rank 0, GELU, and the full MLP-up size on sampled outputs."""
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


_cache = {}


def nv_layer(M, K, N, r, seed=0):
    key = (M, K, N, r, seed)
    if key not in _cache:
        cfg = synth.LayerConfig(f"nv_{M}_{K}_{N}_{r}", 50, M, K, N, r, "nvfp4_g16", "none",
                                "normal", 0.01, 30.0)
        d = synth.make_layer_inputs(cfg, seed=seed)
        si = oracle.smoothing_factors(d["X_cal"], d["W"], 0.5)
        ga = oracle.nvfp4_act_global_scale(d["X_cal"], si)
        layer = oracle.prep_svdq_layer(d["W"], si, r, "nvfp4_g16", act_gscale=ga)
        _cache[key] = (d, si, ga, layer)
    return _cache[key]


@pytest.mark.parametrize("M,K,r", [(256, 512, 16), (37, 256, 0), (300, 3072, 32), (1, 1024, 128),
                                   (4100, 512, 16)])
def test_quantize_act_nvfp4(P, M, K, r):
    d, si, ga, layer = nv_layer(M, K, 256, r)
    X = d["X"]
    _, packed_ref, scales_ref = oracle.quantize_act_ref(X, si, "nvfp4_g16", ga)
    codes, scales, la = P.svdq_quantize_act_nvfp4(dev(X), dev(si), dev(layer["lora_down"]) if r else None,
                                                  float(ga))
    assert np.array_equal(host(codes), packed_ref)
    assert np.array_equal(host(scales), scales_ref)
    if r:
        la_ref = oracle.lora_act_ref(X, layer["lora_down"])
        assert_close(host(la), la_ref, LORA_TOL)
    else:
        assert la is None


def test_quantize_act_nvfp4_extremes(P):
    """Saturating block scales (a tiny per-tensor scale), all-zero blocks,
    subnormal E4M3 scales (a huge per-tensor scale) and signed zeros."""
    K = 512
    rng = np.random.default_rng(31)
    X = (rng.standard_normal((64, K)) * 3).astype(np.float16)
    X[5, :16] = 0
    X[6, 16:32] = np.float16(-0.0)
    X[7, :] = np.float16(1e-3)
    si = np.ones(K, np.float32)
    for ga in (np.float32(1e-6), np.float32(0.37), np.float32(1e3)):
        _, packed_ref, scales_ref = oracle.quantize_act_ref(X, si, "nvfp4_g16", ga)
        codes, scales, _ = P.svdq_quantize_act_nvfp4(dev(X), dev(si), None, float(ga))
        assert np.array_equal(host(codes), packed_ref), ga
        assert np.array_equal(host(scales), scales_ref), ga


def test_quantize_act_nvfp4_ties(P):
    """Quotients on an E2M1 rounding boundary (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5)
    or a few fp16 ulps from one, with block divisors that are not powers of two
    (1.25, 1.5, 1.75 at a per-tensor scale of 1): where a reciprocal multiply
    would land on the other side of a tie, the codes must still be those of the
    correctly rounded quotient."""
    M, K = 48, 512
    rng = np.random.default_rng(41)
    bounds = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    X = np.zeros((M, K), np.float16)
    for m in range(M):
        for j in range(K // 16):
            dv = (1.25, 1.5, 1.75)[(m + j) % 3]
            blk = (rng.choice(bounds, 16) * dv).astype(np.float16)
            for t in range(16):                      # a third exact, the rest 1-3 ulps off
                for _ in range(int(rng.integers(0, 4)) if t % 3 else 0):
                    blk[t] = np.nextafter(blk[t], np.float16(np.inf if rng.integers(2) else -np.inf),
                                          dtype=np.float16)
            blk[0] = np.float16(6.0 * dv)            # amax: the block scale is exactly dv
            blk = np.minimum(blk, np.float16(6.0 * dv))
            X[m, 16 * j:16 * j + 16] = blk * rng.choice(np.array([-1, 1], np.float16), 16)
    si = np.ones(K, np.float32)
    _, packed_ref, scales_ref = oracle.quantize_act_ref(X, si, "nvfp4_g16", np.float32(1.0))
    codes, scales, _ = P.svdq_quantize_act_nvfp4(dev(X), dev(si), None, 1.0)
    assert np.array_equal(host(scales), scales_ref)
    assert np.array_equal(host(codes), packed_ref)


def _gemm_case(P, M, K, N, r, epi, seed=1):
    d, si, ga, layer = nv_layer(M, K, N, r, seed)
    codes_u, packed, scales = oracle.quantize_act_ref(d["X"], si, "nvfp4_g16", ga)
    la16 = oracle.lora_act_ref(d["X"], layer["lora_down"]).astype(np.float32)
    y_ref = oracle.gemm_ref(codes_u, scales, la16, layer["w_codes_unpacked"], layer["w_scales"],
                            layer["lora_up"], d["bias"], "nvfp4_g16", epi,
                            act_gscale=ga, w_gscale=layer["w_gscale"])
    alpha = float(np.float32(ga) * np.float32(layer["w_gscale"]))
    y = P.svdq_gemm_nvfp4(dev(packed), dev(scales), dev(la16) if r else None, dev(layer["w_codes"]),
                          dev(layer["w_scales"]), dev(layer["lora_up"]) if r else None, dev(d["bias"]),
                          alpha, epi)
    return host(y), y_ref


@pytest.mark.parametrize("M,K,N,r,epi", [(200, 512, 384, 16, "none"),      # 128-wide tiles
                                         (256, 512, 512, 16, "gelu_tanh"),  # few tiles: 128-wide
                                         (300, 1024, 768, 32, "none"),
                                         (17, 256, 256, 0, "gelu_tanh"),
                                         (520, 768, 1280, 128, "none")])
def test_gemm_nvfp4(P, M, K, N, r, epi):
    y, y_ref = _gemm_case(P, M, K, N, r, epi)
    assert np.isfinite(y).all()
    assert_close(y, y_ref)


def test_gemm_nvfp4_full_size_sampled(P):
    """The MLP up-projection size (M4096 K3072 N12288 r32, GELU) in the launch
    configuration the benchmark times; outputs checked on sampled rows and
    columns, codes of the sampled rows bit-exact."""
    cfg = synth.CONFIGS["mlp_up_nvfp4"]
    p = synth.random_quantized_layer(cfg, seed=0)
    ga, gw = p["act_gscale"], p["w_gscale"]
    codes, scales, la = P.svdq_quantize_act_nvfp4(dev(p["X"]), dev(p["smooth_inv"]), dev(p["lora_down"]),
                                                  float(ga))
    # the GEMM takes the oracle's low-rank activations (all rows), the GPU's checked against them
    la_o = oracle.lora_act_ref(p["X"], p["lora_down"]).astype(np.float32)
    assert_close(host(la), la_o, LORA_TOL)
    y = P.svdq_gemm_nvfp4(codes, scales, dev(la_o), dev(p["w_codes"]), dev(p["w_scales"]), dev(p["lora_up"]),
                          dev(p["bias"]), float(np.float32(ga) * np.float32(gw)), "gelu_tanh")
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(cfg.M, 24, replace=False))
    cols = np.sort(rng.choice(cfg.N, 96, replace=False))
    c_ref_u, c_ref, s_ref = oracle.quantize_act_ref(p["X"][rows], p["smooth_inv"], "nvfp4_g16", ga)
    assert np.array_equal(host(codes)[rows], c_ref)
    assert np.array_equal(host(scales)[rows], s_ref)
    wu = oracle.unpack_nibbles(p["w_codes"][cols], signed=False)
    y_ref = oracle.gemm_ref(c_ref_u, s_ref, la_o[rows], wu, p["w_scales"][cols], p["lora_up"][cols],
                            p["bias"][cols], "nvfp4_g16", "gelu_tanh", act_gscale=ga, w_gscale=gw)
    yh = host(y)
    assert np.isfinite(yh).all()
    assert_close(yh[np.ix_(rows, cols)], y_ref)


def test_gemm_nvfp4_wide_tiles_ragged_sampled(P):
    """256-wide tiles (more than 128 of them) with a ragged last row tile:
    M 1000, N 8448 (4 x 33 tiles); sampled rows (the last ones included) and
    columns against the oracle."""
    cfg = synth.LayerConfig("nv_wide", 62, 1000, 512, 8448, 32, "nvfp4_g16", "gelu_tanh", "normal", 0.005, 30.0)
    p = synth.random_quantized_layer(cfg, seed=4)
    ga, gw = p["act_gscale"], p["w_gscale"]
    codes, scales, la = P.svdq_quantize_act_nvfp4(dev(p["X"]), dev(p["smooth_inv"]), dev(p["lora_down"]),
                                                  float(ga))
    la_o = oracle.lora_act_ref(p["X"], p["lora_down"]).astype(np.float32)
    assert_close(host(la), la_o, LORA_TOL)
    y = P.svdq_gemm_nvfp4(codes, scales, dev(la_o), dev(p["w_codes"]), dev(p["w_scales"]), dev(p["lora_up"]),
                          dev(p["bias"]), float(np.float32(ga) * np.float32(gw)), "gelu_tanh")
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.choice(cfg.M, 20, replace=False), [0, 767, 768, 999]]))
    cols = np.unique(np.concatenate([rng.choice(cfg.N, 80, replace=False), [0, 255, 256, 8447]]))
    c_ref_u, c_ref, s_ref = oracle.quantize_act_ref(p["X"][rows], p["smooth_inv"], "nvfp4_g16", ga)
    assert np.array_equal(host(codes)[rows], c_ref)
    wu = oracle.unpack_nibbles(p["w_codes"][cols], signed=False)
    y_ref = oracle.gemm_ref(c_ref_u, s_ref, la_o[rows], wu, p["w_scales"][cols], p["lora_up"][cols],
                            p["bias"][cols], "nvfp4_g16", "gelu_tanh", act_gscale=ga, w_gscale=gw)
    yh = host(y)
    assert np.isfinite(yh).all()
    assert_close(yh[np.ix_(rows, cols)], y_ref)


def test_nvfp4_layer_module(P):
    from bit_diffusion_transformer_act_amd.modules import SVDQLinear
    M, K, N, r = 333, 1024, 768, 32
    d, si, ga, layer = nv_layer(M, K, N, r, seed=2)
    m = SVDQLinear(K, N, r, "nvfp4_g16", bias=True, epilogue="gelu_tanh", device=DEV)
    sd = {"smooth_inv": si, "lora_down": layer["lora_down"], "lora_up": layer["lora_up"],
          "w_codes": layer["w_codes"], "w_scales": layer["w_scales"], "bias": d["bias"],
          "act_gscale": np.float32(ga), "w_gscale": np.float32(layer["w_gscale"])}
    m.load_state_dict({k: torch.from_numpy(np.ascontiguousarray(v)) for k, v in sd.items()})
    y = m(dev(d["X"]))
    codes_u, _, scales = oracle.quantize_act_ref(d["X"], si, "nvfp4_g16", ga)
    y_ref = oracle.forward_ref(d["X"], layer, codes_u, scales, d["bias"], "gelu_tanh")
    assert_close(host(y), y_ref)
    # the method's point, on this calibrated layer: close to the dense layer
    dense = oracle.dense_ref(d["X"], d["W"], d["bias"], "gelu_tanh")
    assert rel_l2(host(y), dense) < 0.1


def test_nvfp4_errors(P):
    X = torch.zeros((8, 384), dtype=torch.float16, device=DEV)
    with pytest.raises(P.SvdqError):
        P.svdq_quantize_act_nvfp4(X, torch.ones(384, device=DEV), None, 1.0)   # K % 256
    X = torch.zeros((8, 256), dtype=torch.float16, device=DEV)
    with pytest.raises(P.SvdqError):
        P.svdq_quantize_act_nvfp4(X, torch.ones(256, device=DEV), None, 0.0)
