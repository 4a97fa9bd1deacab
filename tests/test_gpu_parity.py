"""Parity of the HIP library (through the C ABI binding) with the CPU oracle.

Bar: activation codes and scales bit-exact; layer / GEMM / GEMV outputs
within relative L2 2e-3 of the oracle's float64 result on the same codes;
lora_act (fp16) within 1e-3 of the float64 low-rank down-projection. Every oracle
input comes from the seeded generators or from the oracle itself, never from
the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

Y_TOL = 2e-3
LORA_TOL = 1e-3


@pytest.fixture(scope="module")
def P():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import bit_diffusion_transformer_act_amd as pkg
    assert pkg.svdq_device_check(0) == 0, "cuda:0 is not gfx950"
    return pkg


DEV = torch.device("cuda:0")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def scales_equal(gpu, ref, fmt):
    if fmt == "int4_g64":
        return np.array_equal(gpu.view(np.uint16), np.asarray(ref, np.float16).view(np.uint16))
    return np.array_equal(gpu, ref)


_tiny_cache = {}


def tiny_layer(fmt, rank=None):
    key = (fmt, rank)
    if key not in _tiny_cache:
        cfg = synth.CONFIGS["tiny"]
        d = synth.make_layer_inputs(cfg, seed=0)
        si = oracle.smoothing_factors(d["X_cal"], d["W"], cfg.alpha)
        layer = oracle.prep_svdq_layer(d["W"], si, cfg.rank if rank is None else rank, fmt)
        _tiny_cache[key] = (cfg, d, si, layer)
    return _tiny_cache[key]


# ------------------------------------------------------------- quantizer --

@pytest.mark.parametrize("fmt", ["int4_g64", "fp4_b32"])
@pytest.mark.parametrize("M", [256, 200, 17, 1])
def test_quantize_act_tiny(P, fmt, M):
    cfg, d, si, layer = tiny_layer(fmt)
    X = d["X"][:M]
    _, packed_ref, scales_ref = oracle.quantize_act_ref(X, si, fmt)
    codes, scales, la = P.svdq_quantize_act(dev(X), dev(si), dev(layer["lora_down"]), fmt)
    assert np.array_equal(host(codes), packed_ref)
    assert scales_equal(host(scales), scales_ref, fmt)
    la_ref = oracle.lora_act_ref(X, layer["lora_down"])
    assert rel_l2(host(la), la_ref) <= LORA_TOL


@pytest.mark.parametrize("name,fmt", [("qkv", "int4_g64"), ("mlp_up", "fp4_b32"),
                                      ("mlp_down", "int4_g64"), ("mlp_down_m1024", "int4_g64")])
def test_quantize_act_full_size(P, name, fmt):
    cfg = synth.CONFIGS[name]
    p = synth.random_quantized_layer(cfg, seed=1)
    _, packed_ref, scales_ref = oracle.quantize_act_ref(p["X"], p["smooth_inv"], fmt)
    codes, scales, la = P.svdq_quantize_act(dev(p["X"]), dev(p["smooth_inv"]), dev(p["lora_down"]), fmt)
    c = host(codes)
    mism = int((c != packed_ref).sum())
    assert mism == 0, f"{mism} code bytes differ"
    assert scales_equal(host(scales), scales_ref, fmt)
    assert rel_l2(host(la), oracle.lora_act_ref(p["X"], p["lora_down"])) <= LORA_TOL


@pytest.mark.parametrize("fmt", ["int4_g64", "fp4_b32"])
@pytest.mark.parametrize("M,K,r", [
    (48, 40960, 32),    # smooth_inv beyond the LDS budget: the global-load variant
    (37, 2048, 128),    # rank 128: the 4-wave variant, ragged rows
    (300, 1024, 48),    # rank 48: 8 waves, ragged last workgroup
    (4096, 512, 16),    # 256 workgroups: 8 waves per workgroup
])
def test_quantize_act_shapes(P, fmt, M, K, r):
    rng = np.random.default_rng(11)
    X = (rng.standard_normal((M, K)) * 2.0).astype(np.float16)
    si = np.exp(rng.normal(0.0, 0.3, K)).astype(np.float32)
    ld = (rng.standard_normal((r, K)) * 0.02).astype(np.float16)
    _, packed_ref, scales_ref = oracle.quantize_act_ref(X, si, fmt)
    codes, scales, la = P.svdq_quantize_act(dev(X), dev(si), dev(ld), fmt)
    assert np.array_equal(host(codes), packed_ref)
    assert scales_equal(host(scales), scales_ref, fmt)
    assert rel_l2(host(la), oracle.lora_act_ref(X, ld)) <= LORA_TOL


def _adversarial_x(fmt, K=512, M=64, seed=3):
    """Rows built to hit the quantizer's edge cases exactly."""
    rng = np.random.default_rng(seed)
    X = np.zeros((M, K), np.float64)
    G = 64 if fmt == "int4_g64" else 32
    for m in range(M):
        for g0 in range(0, K, G):
            kind = (m + g0 // G) % 7
            grp = np.zeros(G)
            if kind == 0:                      # all zero (and -0)
                grp[::3] = -0.0
            elif kind == 1 and fmt == "int4_g64":   # exact .5 ties at scale 2^e
                s = 2.0 ** rng.integers(-6, 4)
                grp = (rng.integers(-7, 7, G) + 0.5) * s
                grp[0] = 7 * s
            elif kind == 1:                    # exact E2M1 ties at scale 2^e
                e = int(rng.integers(-8, 4))
                ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
                grp = rng.choice(ties, G) * rng.choice([-1, 1], G) * 2.0 ** e
                grp[0] = 6 * 2.0 ** e
            elif kind == 2:                    # fp16 subnormal magnitudes
                grp = rng.integers(-30, 30, G) * 2.0 ** -24
            elif kind == 3:                    # largest fp16 values
                grp = rng.uniform(-65504, 65504, G)
                grp[1] = 65504.0
            elif kind == 4:                    # one outlier, rest tiny
                grp = rng.standard_normal(G) * 1e-3
                grp[rng.integers(G)] = 300.0
            elif kind == 5:                    # single negative value, rest zero
                grp[rng.integers(G)] = -rng.uniform(0.1, 10)
            else:
                grp = rng.standard_normal(G) * 10
            X[m, g0:g0 + G] = grp
    return X.astype(np.float16)


@pytest.mark.parametrize("fmt", ["int4_g64", "fp4_b32"])
@pytest.mark.parametrize("smooth", ["ones", "pow2", "large"])
def test_quantize_act_adversarial(P, fmt, smooth):
    X = _adversarial_x(fmt)
    K = X.shape[1]
    if smooth == "ones":
        si = np.ones(K, np.float32)
    elif smooth == "pow2":
        si = (2.0 ** np.random.default_rng(5).integers(-3, 4, K)).astype(np.float32)
    else:   # pushes amax / 7 above the fp16 maximum: saturating scales
        si = np.full(K, 64.0, np.float32)
    _, packed_ref, scales_ref = oracle.quantize_act_ref(X, si, fmt)
    codes, scales, _ = P.svdq_quantize_act(dev(X), dev(si), None, fmt)
    assert np.array_equal(host(codes), packed_ref)
    assert scales_equal(host(scales), scales_ref, fmt)


# ------------------------------------------------------------------ GEMM --

@pytest.mark.parametrize("fmt", ["int4_g64", "fp4_b32"])
@pytest.mark.parametrize("M,rank,use_bias,epi", [
    (256, 16, True, "none"), (200, 16, False, "none"), (1, 16, True, "gelu_tanh"),
    (129, 0, True, "none"), (256, 32, True, "gelu_tanh"), (37, 128, True, "none")])
def test_gemm_tiny(P, fmt, M, rank, use_bias, epi):
    cfg, d, si, layer = tiny_layer(fmt, rank)
    X = d["X"][:M]
    codes_u, packed, scales = oracle.quantize_act_ref(X, si, fmt)
    la = oracle.lora_act_ref(X, layer["lora_down"]).astype(np.float16)
    bias = d["bias"] if use_bias else None
    wu = layer["w_codes_unpacked"]
    y_ref = oracle.gemm_ref(codes_u, scales, la, wu, layer["w_scales"], layer["lora_up"], bias, fmt, epi)
    Y = P.svdq_gemm_w4a4(dev(packed), dev(scales), dev(la) if rank else None, dev(layer["w_codes"]),
                         dev(layer["w_scales"]), dev(layer["lora_up"]) if rank else None,
                         None if bias is None else dev(bias), fmt, epi)
    assert rel_l2(host(Y), y_ref) <= Y_TOL


@pytest.mark.parametrize("fmt", ["int4_g64", "fp4_b32"])
def test_layer_end_to_end_tiny(P, fmt):
    """GPU quantizer then GPU GEMM against the oracle's whole-layer forward."""
    cfg, d, si, layer = tiny_layer(fmt)
    codes_u, packed_ref, scales_ref = oracle.quantize_act_ref(d["X"], si, fmt)
    y_ref = oracle.forward_ref(d["X"], layer, codes_u, scales_ref, d["bias"])
    L = {"fmt": fmt, "smooth_inv": dev(si), "lora_down": dev(layer["lora_down"]),
         "w_codes": dev(layer["w_codes"]), "w_scales": dev(layer["w_scales"]),
         "lora_up": dev(layer["lora_up"])}
    Y = P.svdq_linear(dev(d["X"]), L, dev(d["bias"]))
    assert rel_l2(host(Y), y_ref) <= Y_TOL
    # and the method's accuracy claim holds on the GPU output as well
    y_dense = oracle.dense_ref(d["X"], d["W"], d["bias"])
    print(f"{fmt}: GPU layer vs dense fp64 rel err {rel_l2(host(Y), y_dense):.3e}")


@pytest.mark.parametrize("name", ["qkv", "mlp_up", "mlp_down", "mlp_down_m1024", "attn_out"])
def test_gemm_full_size_sampled(P, name):
    """Full DiT shapes in the benchmark's launch configuration; outputs
    checked on sampled rows (all columns) against the oracle."""
    cfg = synth.CONFIGS[name]
    fmt = cfg.fmt
    p = synth.random_quantized_layer(cfg, seed=2)
    codes_u, packed, scales = oracle.quantize_act_ref(p["X"], p["smooth_inv"], fmt)
    la = oracle.lora_act_ref(p["X"], p["lora_down"]).astype(np.float16)
    Y = P.svdq_gemm_w4a4(dev(packed), dev(scales), dev(la), dev(p["w_codes"]), dev(p["w_scales"]),
                         dev(p["lora_up"]), dev(p["bias"]), fmt, cfg.epilogue)
    y = host(Y)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([rng.choice(cfg.M, 40, replace=False), [0, cfg.M - 1]]))
    wu = oracle.unpack_nibbles(p["w_codes"], signed=(fmt == "int4_g64"))
    y_ref = oracle.gemm_ref(codes_u, scales, la, wu, p["w_scales"], p["lora_up"], p["bias"], fmt,
                            cfg.epilogue, rows=rows)
    assert rel_l2(y[rows], y_ref) <= Y_TOL
    assert np.isfinite(y).all()


# ------------------------------------------------------------------ GEMV --

@pytest.mark.parametrize("M,N", [(1, 18432), (2, 1000), (8, 96), (3, 17)])
def test_awq_gemv(P, M, N):
    g = synth.CONFIGS["gemv"]
    d = synth.make_gemv_inputs(g, seed=4, M=M)
    aw = oracle.awq_prep(d["W"][:N])
    y_ref = oracle.gemv_ref(d["x"], aw["codes"], aw["scales"], aw["zeros"])
    y = P.awq_gemv_w4a16(dev(d["x"]), dev(aw["codes"]), dev(aw["scales"]), dev(aw["zeros"]))
    assert rel_l2(host(y), y_ref) <= Y_TOL


@pytest.mark.parametrize("M,K,N", [(4, 4096, 512), (1, 12288, 3072), (2, 16384, 300),
                                   (1, 16448, 77), (8, 4096, 130), (1, 64, 5)])
def test_awq_gemv_random_params_other_k(P, M, K, N):
    """Both kernel paths (x in registers for M * ceil(K/4096) <= 4, x in LDS
    otherwise), ragged N, K not a multiple of 4096."""
    g = synth.GemvConfig(f"gemv_k{K}", 40, 1, K, N, 64)
    p = synth.random_awq_layer(g, seed=5, M=M)
    y_ref = oracle.gemv_ref(p["x"], p["codes"], p["scales"], p["zeros"])
    y = P.awq_gemv_w4a16(dev(p["x"]), dev(p["codes"]), dev(p["scales"]), dev(p["zeros"]))
    assert rel_l2(host(y), y_ref) <= Y_TOL


@pytest.mark.parametrize("M", [1, 8])
def test_awq_gemv_fractional_zeros(P, M):
    g = synth.GemvConfig("gemv_fz", 41, 1, 1024, 256, 64)
    p = synth.random_awq_layer(g, seed=6, M=M)
    z = (p["zeros"].astype(np.float32) + np.random.default_rng(1).uniform(-0.5, 0.5, p["zeros"].shape)).astype(np.float16)
    y_ref = oracle.gemv_ref(p["x"], p["codes"], p["scales"], z)
    y = P.awq_gemv_w4a16(dev(p["x"]), dev(p["codes"]), dev(p["scales"]), dev(z))
    assert rel_l2(host(y), y_ref) <= Y_TOL


# ------------------------------------------------------------ semantics --

def test_deterministic_and_stream(P):
    cfg, d, si, layer = tiny_layer("int4_g64")
    L = {"fmt": "int4_g64", "smooth_inv": dev(si), "lora_down": dev(layer["lora_down"]),
         "w_codes": dev(layer["w_codes"]), "w_scales": dev(layer["w_scales"]),
         "lora_up": dev(layer["lora_up"])}
    X = dev(d["X"])
    y1 = host(P.svdq_linear(X, L, None))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y2 = P.svdq_linear(X, L, None)
    s.synchronize()
    assert np.array_equal(y1.view(np.uint16), y2.cpu().numpy().view(np.uint16))


def test_unsupported_device_is_a_clear_error(P, monkeypatch):
    cfg, d, si, layer = tiny_layer("int4_g64")
    monkeypatch.setenv("SVDQ_FORCE_ARCH", "gfx942")
    with pytest.raises(P.SvdqError) as e:
        P.svdq_quantize_act(dev(d["X"]), dev(si), None, "int4_g64")
    assert e.value.status == -4
    monkeypatch.delenv("SVDQ_FORCE_ARCH")
    P.svdq_quantize_act(dev(d["X"]), dev(si), None, "int4_g64")
