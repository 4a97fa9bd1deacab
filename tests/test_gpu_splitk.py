"""svdq_gemm_w4a4_splitk: the INT4 GEMM with K split across workgroups for
shapes with few output tiles, against the CPU oracle (same bar as the unsplit
GEMM: per-element bound and rel-L2 on every checked row), and its fallbacks
(no split, FP4, a workspace too small), which run the unsplit kernel and must
give its output bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import assert_close, band_rows

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


def layer(cfg, seed, dt=torch.float16):
    """A seeded layer; with bf16, lora_up and bias rounded to bf16 on the host
    (the oracle then sees the values the GPU gets)."""
    p = synth.random_quantized_layer(cfg, seed=seed)
    if dt == torch.bfloat16:
        for k in ("lora_up", "bias"):
            p[k] = torch.from_numpy(np.ascontiguousarray(p[k])).to(torch.bfloat16).float().numpy()
    codes_u, packed, scales = oracle.quantize_act_ref(p["X"], p["smooth_inv"], cfg.fmt)
    la = oracle.lora_act_ref(p["X"], p["lora_down"]).astype(np.float32)
    return p, codes_u, packed, scales, la


def gemm_args(p, packed, scales, la, dt):
    h = lambda a: dev(a).to(dt)
    r = la.shape[1]
    return (dev(packed), dev(scales), dev(la) if r else None, dev(p["w_codes"]), dev(p["w_scales"]),
            h(p["lora_up"]) if r else None, h(p["bias"]))


def test_mlp_down_m1024_full_size(P):
    """The DiT MLP down-projection at M 1024 (K 12288, N 3072): 4 splits of 24
    steps; one row from every 64-row band plus the first and last, all columns."""
    cfg = synth.CONFIGS["mlp_down_m1024"]
    assert P.svdq_gemm_w4a4_splitk_workspace(cfg.M, cfg.N, cfg.K) == 4 * cfg.M * cfg.N * 4
    p, codes_u, packed, scales, la = layer(cfg, seed=21)
    args = gemm_args(p, packed, scales, la, torch.float16)
    y = host(P.svdq_gemm_w4a4_splitk(*args, "int4_g64", cfg.epilogue))
    rows = band_rows(cfg.M, seed=13)
    wu = oracle.unpack_nibbles(p["w_codes"], signed=True)
    y_ref = oracle.gemm_ref(codes_u, scales, la, wu, p["w_scales"], p["lora_up"], p["bias"], "int4_g64",
                            cfg.epilogue, rows=rows)
    assert_close(y[rows], y_ref, what="mlp_down_m1024 split K")
    assert np.isfinite(y).all()


@pytest.mark.parametrize("M,K,N,r,epi,dt,splits", [
    (200, 4096, 512, 16, "none", torch.float16, 4),        # ragged M, 8 steps per split
    (130, 8192, 256, 32, "gelu_tanh", torch.bfloat16, 8),  # GELU, bf16, 8 splits
    (64, 2048, 1024, 0, "none", torch.float16, 2),         # no low-rank branch
    (1, 4480, 128, 48, "none", torch.float16, 4),          # one row; 35 steps: splits of 8 and 9
])
def test_splitk_small_against_oracle(P, M, K, N, r, epi, dt, splits):
    cfg = synth.LayerConfig(f"splitk_{M}_{K}_{N}", 54, M, K, N, r, "int4_g64", epi, "normal", 0.005, 30.0)
    assert P.svdq_gemm_w4a4_splitk_workspace(M, N, K) == splits * M * N * 4
    p, codes_u, packed, scales, la = layer(cfg, seed=5, dt=dt)
    args = gemm_args(p, packed, scales, la, dt)
    Y = P.svdq_gemm_w4a4_splitk(*args, "int4_g64", epi, dtype=dt)
    y = host(Y.float() if dt == torch.bfloat16 else Y)
    wu = oracle.unpack_nibbles(p["w_codes"], signed=True)
    y_ref = oracle.gemm_ref(codes_u, scales, la, wu, p["w_scales"], p["lora_up"], p["bias"], "int4_g64", epi)
    assert_close(y, y_ref, what=cfg.name)


def test_splitk_deterministic_and_close_to_unsplit(P):
    """Two calls give the same bits; against the unsplit kernel only the order
    of the fp32 additions differs, so the outputs agree to an ulp or two of
    fp16 plus a floor far below the oracle bar's (the checks against the
    oracle above are the bar)."""
    cfg = synth.LayerConfig("splitk_det", 55, 512, 8192, 768, 32, "int4_g64", "none", "normal", 0.005, 30.0)
    p, codes_u, packed, scales, la = layer(cfg, seed=6)
    args = gemm_args(p, packed, scales, la, torch.float16)
    ws = torch.full((P.svdq_gemm_w4a4_splitk_workspace(512, 768, 8192),), 0xFF, dtype=torch.uint8, device=DEV)
    y1 = host(P.svdq_gemm_w4a4_splitk(*args, workspace=ws))
    y2 = host(P.svdq_gemm_w4a4_splitk(*args, workspace=ws))
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    y0 = host(P.svdq_gemm_w4a4(*args)).astype(np.float64)
    ulp = np.spacing(np.abs(y0).astype(np.float16)).astype(np.float64)
    # outputs near zero come from cancelling sums, where the fp32 order shows
    # at a tiny fraction of the outputs' rms rather than in fp16 ulps
    rms = np.sqrt(np.mean(y0 ** 2))
    assert np.all(np.abs(y1.astype(np.float64) - y0) <= 2 * ulp + 1e-4 * rms)


@pytest.mark.parametrize("case", ["too_small", "no_split_shape", "fp4"])
def test_splitk_fallbacks_equal_unsplit(P, case):
    fmt = "fp4_b32" if case == "fp4" else "int4_g64"
    M, N = (4096, 1024) if case == "no_split_shape" else (256, 512)   # 256 tiles of 128: no split
    cfg = synth.LayerConfig(f"splitk_fb_{case}", 56, M, 2048, N, 16, fmt, "gelu_tanh", "normal", 0.005, 30.0)
    p, codes_u, packed, scales, la = layer(cfg, seed=7)
    args = gemm_args(p, packed, scales, la, torch.float16)
    need = P.svdq_gemm_w4a4_splitk_workspace(M, N, 2048, fmt)
    if case == "too_small":
        assert need > 0
        ws = torch.empty((need - 16,), dtype=torch.uint8, device=DEV)
    else:
        assert need == 0
        ws = torch.empty((16,), dtype=torch.uint8, device=DEV)
    y = host(P.svdq_gemm_w4a4_splitk(*args, fmt, "gelu_tanh", workspace=ws))
    y0 = host(P.svdq_gemm_w4a4(*args, fmt, "gelu_tanh"))
    assert np.array_equal(y.view(np.uint16), y0.view(np.uint16))
