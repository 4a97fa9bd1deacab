"""Parity of the HIP library (through the C ABI binding) with the CPU oracle.

Bar: activation codes and scales bit-exact; layer / GEMM / GEMV outputs
within relative L2 2e-3 of the oracle's float64 result on the same codes, and
every compared element within 2 ulp of its type plus 1e-3 rms
(tests/parity.py); lora_act (fp32) within 1e-3 of the float64 low-rank
down-projection under the same element bound. Every oracle input comes from
the seeded generators or from the oracle itself, never from the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import LORA_TOL, Y_TOL, assert_close, band_rows, rel_l2  # noqa: F401

pytestmark = pytest.mark.gpu


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
    assert_close(host(la), la_ref, LORA_TOL)


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
    assert_close(host(la), oracle.lora_act_ref(p["X"], p["lora_down"]), LORA_TOL)


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
    assert_close(host(la), oracle.lora_act_ref(X, ld), LORA_TOL)


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
    la = oracle.lora_act_ref(X, layer["lora_down"]).astype(np.float32)
    bias = d["bias"] if use_bias else None
    wu = layer["w_codes_unpacked"]
    y_ref = oracle.gemm_ref(codes_u, scales, la, wu, layer["w_scales"], layer["lora_up"], bias, fmt, epi)
    Y = P.svdq_gemm_w4a4(dev(packed), dev(scales), dev(la) if rank else None, dev(layer["w_codes"]),
                         dev(layer["w_scales"]), dev(layer["lora_up"]) if rank else None,
                         None if bias is None else dev(bias), fmt, epi)
    assert_close(host(Y), y_ref)


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
    assert_close(host(Y), y_ref)
    # and the method's accuracy claim holds on the GPU output as well
    y_dense = oracle.dense_ref(d["X"], d["W"], d["bias"])
    print(f"{fmt}: GPU layer vs dense fp64 rel err {rel_l2(host(Y), y_dense):.3e}")


@pytest.mark.parametrize("name", ["qkv", "mlp_up", "mlp_down", "mlp_down_m1024", "attn_out", "mlp_up_int4"])
def test_gemm_full_size_sampled(P, name):
    """Full DiT shapes in the benchmark's launch configuration; outputs
    checked against the oracle on one row from every band of 64 (every M-tile
    of the remapped grid) plus the first and last rows, all columns. INT4
    weight codes span -8..7."""
    cfg = synth.CONFIGS[name]
    fmt = cfg.fmt
    p = synth.random_quantized_layer(cfg, seed=2)
    codes_u, packed, scales = oracle.quantize_act_ref(p["X"], p["smooth_inv"], fmt)
    la = oracle.lora_act_ref(p["X"], p["lora_down"]).astype(np.float32)
    Y = P.svdq_gemm_w4a4(dev(packed), dev(scales), dev(la), dev(p["w_codes"]), dev(p["w_scales"]),
                         dev(p["lora_up"]), dev(p["bias"]), fmt, cfg.epilogue)
    y = host(Y)
    rows = band_rows(cfg.M, seed=11)
    wu = oracle.unpack_nibbles(p["w_codes"], signed=(fmt == "int4_g64"))
    if fmt == "int4_g64":
        assert wu.min() == -8
    y_ref = oracle.gemm_ref(codes_u, scales, la, wu, p["w_scales"], p["lora_up"], p["bias"], fmt,
                            cfg.epilogue, rows=rows)
    assert_close(y[rows], y_ref, what=name)
    assert np.isfinite(y).all()


@pytest.mark.parametrize("fmt", ["int4_g64", "fp4_b32"])
@pytest.mark.parametrize("M,N,epi", [
    (2000, 3072, "none"),        # 16 x 24 tiles of 128: the INT4 path's 64 x 128 tiles, ragged M
    (2048, 3072, "gelu_tanh"),   # same band, whole tiles, GELU
    (1000, 1536, "none"),        # 8 x 12 tiles of 128: 64 x 64 tiles, ragged M
])
def test_gemm_tile_bands(P, fmt, M, N, epi):
    """The GEMM picks its INT4 tile size from the number of 128 x 128 tiles;
    each band against the oracle on sampled rows (first and last included)."""
    cfg = synth.LayerConfig(f"band_{M}_{N}", 52, M, 512, N, 32, fmt, epi, "normal", 0.005, 30.0)
    p = synth.random_quantized_layer(cfg, seed=3)
    codes_u, packed, scales = oracle.quantize_act_ref(p["X"], p["smooth_inv"], fmt)
    la = oracle.lora_act_ref(p["X"], p["lora_down"]).astype(np.float32)
    Y = P.svdq_gemm_w4a4(dev(packed), dev(scales), dev(la), dev(p["w_codes"]), dev(p["w_scales"]),
                         dev(p["lora_up"]), dev(p["bias"]), fmt, epi)
    y = host(Y)
    rows = band_rows(M, seed=12, extra=(63, 64, 127, 128))
    wu = oracle.unpack_nibbles(p["w_codes"], signed=(fmt == "int4_g64"))
    y_ref = oracle.gemm_ref(codes_u, scales, la, wu, p["w_scales"], p["lora_up"], p["bias"], fmt, epi,
                            rows=rows)
    assert_close(y[rows], y_ref)
    assert np.isfinite(y).all()


@pytest.mark.parametrize("M,K,epi", [
    (2000, 1024, "gelu_tanh"),   # 8 x 32 tiles of 256: the last row tile holds 208 rows
    (1793, 512, "none"),         # 8 x 32 tiles again: the last row tile holds one row
])
def test_gemm_fp4_big_ragged(P, M, K, epi):
    """The 256 x 256 FP4 kernel (8 waves of 128 x 64) with a ragged last row
    tile, against the oracle on one row of every 64-row band, all columns."""
    N = 8192
    cfg = synth.LayerConfig(f"fp4big_{M}_{K}", 54, M, K, N, 32, "fp4_b32", epi, "normal", 0.005, 30.0)
    p = synth.random_quantized_layer(cfg, seed=5)
    codes_u, packed, scales = oracle.quantize_act_ref(p["X"], p["smooth_inv"], "fp4_b32")
    la = oracle.lora_act_ref(p["X"], p["lora_down"]).astype(np.float32)
    Y = P.svdq_gemm_w4a4(dev(packed), dev(scales), dev(la), dev(p["w_codes"]), dev(p["w_scales"]),
                         dev(p["lora_up"]), dev(p["bias"]), "fp4_b32", epi)
    y = host(Y)
    rows = band_rows(M, seed=13, extra=(1791, 1792) if M > 1792 else ())
    wu = oracle.unpack_nibbles(p["w_codes"], signed=False)
    y_ref = oracle.gemm_ref(codes_u, scales, la, wu, p["w_scales"], p["lora_up"], p["bias"], "fp4_b32", epi,
                            rows=rows)
    assert_close(y[rows], y_ref)
    assert np.isfinite(y).all()


@pytest.mark.parametrize("fmt", ["int4_g64", "fp4_b32"])
@pytest.mark.parametrize("M,K,N", [(200, 384, 512), (200, 640, 512), (4096, 384, 4096)])
def test_gemm_odd_k_steps(P, fmt, M, K, N):
    """K / 128 odd (3 and 5 steps of 128): the last two-step scale group holds
    one step, and the pipelines' wait schedule ends on an odd step. Small M puts
    INT4 on its 64 x 64 tiles and FP4 on the 4-stage 128 x 128 path; M 4096 N 4096
    puts INT4 on its 3-stage 128 x 128 tiles."""
    cfg = synth.LayerConfig(f"oddk_{M}_{K}_{N}", 53, M, K, N, 16, fmt, "none", "normal", 0.005, 30.0)
    p = synth.random_quantized_layer(cfg, seed=4)
    codes_u, packed, scales = oracle.quantize_act_ref(p["X"], p["smooth_inv"], fmt)
    codes, sc, la = P.svdq_quantize_act(dev(p["X"]), dev(p["smooth_inv"]), dev(p["lora_down"]), fmt)
    assert np.array_equal(host(codes), packed)
    assert scales_equal(host(sc), scales, fmt)
    la_o = oracle.lora_act_ref(p["X"], p["lora_down"]).astype(np.float32)
    Y = P.svdq_gemm_w4a4(codes, sc, dev(la_o), dev(p["w_codes"]), dev(p["w_scales"]), dev(p["lora_up"]),
                         dev(p["bias"]), fmt, "none")
    y = host(Y)
    rows = np.arange(M) if M <= 256 else band_rows(M, seed=13)
    wu = oracle.unpack_nibbles(p["w_codes"], signed=(fmt == "int4_g64"))
    y_ref = oracle.gemm_ref(codes_u, scales, la_o, wu, p["w_scales"], p["lora_up"], p["bias"], fmt, "none",
                            rows=rows)
    assert_close(y[rows], y_ref, what=f"{fmt} K{K}")


def test_gemm_int4_extreme_codes(P):
    """INT4 code -8 on both operands: groups of all -8 against all -8 (the
    largest group product, 64 * 64, i.e. 2^20 in the kernel's 256 P accumulation),
    all -8 against all 7, alternating -8 / 7, and random codes, with random fp16
    scales; no low-rank branch, with and without bias."""
    M, K, N = 192, 512, 256
    rng = np.random.default_rng(21)
    G = K // 64
    a = rng.integers(-8, 8, (M, K))
    w = rng.integers(-8, 8, (N, K))
    for g in range(G):
        sl = slice(64 * g, 64 * g + 64)
        kind = g % 4
        if kind == 0:
            a[: M // 2, sl] = -8
            w[: N // 2, sl] = -8
        elif kind == 1:
            a[:, sl] = -8
            w[:, sl] = 7
        elif kind == 2:
            a[:, sl] = np.where(np.arange(64) % 2 == 0, -8, 7)
            w[:, sl] = np.where(np.arange(64) % 3 == 0, 7, -8)
    sa = rng.uniform(0.01, 0.1, (M, G)).astype(np.float16)
    sw = rng.uniform(0.001, 0.01, (N, G)).astype(np.float16)
    bias = (rng.standard_normal(N) * 0.1).astype(np.float16)
    ap, wp = oracle.pack_nibbles(a), oracle.pack_nibbles(w)
    for b in (None, bias):
        Y = P.svdq_gemm_w4a4(dev(ap), dev(sa), None, dev(wp), dev(sw), None, None if b is None else dev(b),
                             "int4_g64", "none")
        y_ref = oracle.gemm_ref(a.astype(np.int8), sa, np.zeros((M, 0)), w.astype(np.int8), sw, np.zeros((N, 0)),
                                b, "int4_g64")
        assert_close(host(Y), y_ref, what="extreme codes")


@pytest.mark.parametrize("M,K,N", [(256, 1024, 512), (2048, 512, 8192)])
def test_gemm_fp4_extreme_scales(P, M, K, N):
    """FP4 E8M0 scale bytes far from 127 on both operands (2^-63 .. 2^63 per
    block), the pairs' exponents summing to about -16 so the outputs stay in
    fp16 range: the hardware's scaling against the oracle's exact dequantized
    product. Random E2M1 codes (all 16 nibbles); the 128 x 128 FP4 path and the
    256 x 256 kernel."""
    rng = np.random.default_rng(31)
    nb = K // 32
    ea = rng.integers(64, 191, nb)                      # per block, shared by the rows
    eb = 254 - 16 - ea                                  # per block, shared by the columns
    sa = (ea[None, :] + rng.integers(-2, 3, (M, nb))).astype(np.uint8)
    sw = (eb[None, :] + rng.integers(-2, 3, (N, nb))).astype(np.uint8)
    a = rng.integers(0, 16, (M, K)).astype(np.uint8)
    w = rng.integers(0, 16, (N, K)).astype(np.uint8)
    Y = P.svdq_gemm_w4a4(dev(oracle.pack_nibbles(a)), dev(sa), None, dev(oracle.pack_nibbles(w)), dev(sw), None,
                         None, "fp4_b32", "none")
    y = host(Y)
    rows = np.arange(M) if M <= 256 else band_rows(M, seed=15)
    y_ref = oracle.gemm_ref(a, sa, np.zeros((M, 0)), w, sw, np.zeros((N, 0)), None, "fp4_b32", rows=rows)
    assert_close(y[rows], y_ref, what="FP4 extreme scales")


# ------------------------------------------------ fused QKV epilogue --

def _qkv_case(P, cfg, seed, rows=None):
    p = synth.random_quantized_layer(cfg, seed=seed)
    e = synth.qkv_epilogue_inputs(cfg.M, seed=seed)
    codes_u, packed, scales = oracle.quantize_act_ref(p["X"], p["smooth_inv"], "int4_g64")
    la = oracle.lora_act_ref(p["X"], p["lora_down"]).astype(np.float32)
    args = (dev(packed), dev(scales), dev(la), dev(p["w_codes"]), dev(p["w_scales"]), dev(p["lora_up"]),
            dev(p["bias"]))
    Y = P.svdq_gemm_w4a4_qkv(*args, dev(e["qk_norm_w"]), dev(e["rope"]), e["eps"])
    Y_plain = P.svdq_gemm_w4a4(*args, "int4_g64", "none")
    wu = oracle.unpack_nibbles(p["w_codes"], signed=True)
    sel = np.arange(cfg.M) if rows is None else rows
    y_lin = oracle.gemm_ref(codes_u, scales, la, wu, p["w_scales"], p["lora_up"], p["bias"], "int4_g64",
                            "none", rows=sel)
    rope = e["rope"][sel]
    y_ref = oracle.qkv_epilogue_ref(y_lin, 128, e["qk_norm_w"][0], e["qk_norm_w"][1], rope[..., 0],
                                    rope[..., 1], e["eps"])
    return host(Y), host(Y_plain), y_ref, sel


def _within_one_ulp(a, b):
    """fp16 arrays equal up to one unit in the last place (the plain GEMM may
    round acc * 2^-8 + bias to fp16 in one step, v_fma_mixlo_f16, where the
    QKV variant rounds to fp32 first)."""
    ia = a.view(np.int16).astype(np.int32)
    ib = b.view(np.int16).astype(np.int32)
    return int(np.abs(ia - ib).max()) <= 1 and np.mean(ia != ib) < 1e-4


def test_gemm_qkv_epilogue_small(P):
    """Ragged M, two heads per third: Q and K normalised and rotated, V equal
    to the plain GEMM's output (to one fp16 ulp)."""
    cfg = synth.LayerConfig("qkv_small", 51, 200, 512, 768, 16, "int4_g64", "none", "normal", 0.005, 30.0)
    y, y_plain, y_ref, _ = _qkv_case(P, cfg, seed=6)
    n3 = cfg.N // 3
    assert_close(y[:, :n3], y_ref[:, :n3])
    assert_close(y[:, n3:2 * n3], y_ref[:, n3:2 * n3])
    assert _within_one_ulp(y[:, 2 * n3:], y_plain[:, 2 * n3:])
    assert_close(y[:, 2 * n3:], y_ref[:, 2 * n3:])


def test_gemm_qkv_epilogue_full_size_sampled(P):
    """The DiT QKV projection (24 heads of 128 per third) in the benchmark's
    launch configuration, checked on one row from every band of 64 (all
    columns: every head of Q, K and V)."""
    cfg = synth.CONFIGS["qkv"]
    rows = band_rows(cfg.M, seed=12)
    y, y_plain, y_ref, sel = _qkv_case(P, cfg, seed=3, rows=rows)
    assert_close(y[sel], y_ref)
    n3 = cfg.N // 3
    assert _within_one_ulp(y[:, 2 * n3:], y_plain[:, 2 * n3:])
    assert np.isfinite(y).all()


def test_gemm_qkv_epilogue_errors(P):
    z = lambda *s, dt=torch.uint8: torch.zeros(s, dtype=dt, device="cuda")
    M, K = 16, 256
    ac, asc = z(M, K // 2), z(M, K // 64, dt=torch.float16)
    nw, rope = z(2, 128, dt=torch.float16), z(M, 64, 2, dt=torch.float32)
    with pytest.raises(P.SvdqError) as e:   # N not a multiple of 384
        P.svdq_gemm_w4a4_qkv(ac, asc, None, z(512, K // 2), z(512, K // 64, dt=torch.float16), None, None,
                             nw, rope)
    assert e.value.status == -2
    with pytest.raises(P.SvdqError) as e:   # FP4 is not supported by this entry point
        P.svdq_gemm_w4a4_qkv(ac, z(M, K // 32), None, z(384, K // 2), z(384, K // 32), None, None,
                             nw, rope, fmt="fp4_b32")
    assert e.value.status == -1


# ------------------------------------------------------------------ GEMV --

@pytest.mark.parametrize("M,N", [(1, 18432), (2, 1000), (8, 96), (3, 17)])
def test_awq_gemv(P, M, N):
    g = synth.CONFIGS["gemv"]
    d = synth.make_gemv_inputs(g, seed=4, M=M)
    aw = oracle.awq_prep(d["W"][:N])
    y_ref = oracle.gemv_ref(d["x"], aw["codes"], aw["scales"], aw["zeros"])
    y = P.awq_gemv_w4a16(dev(d["x"]), dev(aw["codes"]), dev(aw["scales"]), dev(aw["zeros"]))
    assert_close(host(y), y_ref)


@pytest.mark.parametrize("M,K,N", [(4, 4096, 512), (1, 12288, 3072), (2, 16384, 300),
                                   (1, 16448, 77), (8, 4096, 130), (1, 64, 5),
                                   (7, 4160, 1000), (3, 10880, 200), (2, 1088, 4099),
                                   (1, 3072, 2049), (6, 5440, 64), (1, 3072, 1), (1, 3072, 3),
                                   (2, 3072, 1)])
def test_awq_gemv_random_params_other_k(P, M, K, N):
    """Batched x (M up to 8), ragged N (including fewer rows than waves), K
    not a multiple of 64 chunks per unit (the last unit of a row reaches past
    its end; x is staged padded to whole units, up to 96768 bytes of LDS at M 7,
    K 4160), rows in pairs with an odd count, up to the LDS limit M K = 32768;
    at M 1 K 3072 (x in registers) one row and a lone odd row."""
    g = synth.GemvConfig(f"gemv_k{K}", 40, 1, K, N, 64)
    p = synth.random_awq_layer(g, seed=5, M=M)
    y_ref = oracle.gemv_ref(p["x"], p["codes"], p["scales"], p["zeros"])
    y = P.awq_gemv_w4a16(dev(p["x"]), dev(p["codes"]), dev(p["scales"]), dev(p["zeros"]))
    assert_close(host(y), y_ref)


@pytest.mark.parametrize("M,K", [(1, 3072), (2, 3072), (1, 4096)])
def test_awq_gemv_grid_beyond_one_workgroup_per_cu(P, M, K):
    """N 140 001: more rows than 256 workgroups of 8 waves hold at 64 rows a
    wave, so the grid grows (274 workgroups); checked on every 61st row and the
    last 130 rows (each wave's rows are spread over the matrix, row w, w + W,
    ...), including the lone last row of an odd count."""
    N = 140001
    g = synth.GemvConfig(f"gemv_bigN{K}", 45, 1, K, N, 64)
    p = synth.random_awq_layer(g, seed=9, M=M)
    y = host(P.awq_gemv_w4a16(dev(p["x"]), dev(p["codes"]), dev(p["scales"]), dev(p["zeros"])))
    rows = np.unique(np.concatenate([np.arange(0, N, 61), np.arange(N - 130, N)]))
    y_ref = oracle.gemv_ref(p["x"], p["codes"][rows], p["scales"][rows], p["zeros"][rows])
    assert_close(y[:, rows], y_ref)


@pytest.mark.parametrize("M,K,N", [(1, 3072, 2048), (3, 2048, 333)])
@pytest.mark.parametrize("dtype", ["float16", "bfloat16"])
def test_awq_gemv_small_activations(P, M, K, N, dtype):
    """x scaled by 2^-12 (input preparation), so that |x| < 2^-10 almost
    everywhere and many values are fp16 subnormals: the accuracy must not depend
    on the scale of x."""
    g = synth.GemvConfig(f"gemv_s{K}", 43, 1, K, N, 64)
    p = synth.random_awq_layer(g, seed=8, M=M)
    x = (p["x"].astype(np.float32) * np.float32(2.0 ** -12)).astype(np.float16)
    if dtype == "bfloat16":
        xt = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
        x = xt.float().numpy()
        xd = xt.to(DEV)
    else:
        xd = dev(x)
    y_ref = oracle.gemv_ref(x, p["codes"], p["scales"], p["zeros"])
    y = P.awq_gemv_w4a16(xd, dev(p["codes"]), dev(p["scales"]), dev(p["zeros"]))
    if dtype == "bfloat16":
        torch.cuda.synchronize()
        assert_close(y.float().cpu().numpy(), oracle.bf16_round(y_ref.astype(np.float32)))
    else:
        assert_close(host(y), y_ref)


@pytest.mark.parametrize("M", [1, 8])
def test_awq_gemv_fractional_zeros(P, M):
    g = synth.GemvConfig("gemv_fz", 41, 1, 1024, 256, 64)
    p = synth.random_awq_layer(g, seed=6, M=M)
    z = (p["zeros"].astype(np.float32) + np.random.default_rng(1).uniform(-0.5, 0.5, p["zeros"].shape)).astype(np.float16)
    y_ref = oracle.gemv_ref(p["x"], p["codes"], p["scales"], z)
    y = P.awq_gemv_w4a16(dev(p["x"]), dev(p["codes"]), dev(p["scales"]), dev(z))
    assert_close(host(y), y_ref)


@pytest.mark.parametrize("M,K,N", [(1, 3072, 18432), (5, 2048, 333)])
def test_awq_gemv_bias(P, M, K, N):
    """The bias joins the fp32 total before the one fp16 rounding."""
    g = synth.GemvConfig(f"gemv_b{K}", 42, 1, K, N, 64)
    p = synth.random_awq_layer(g, seed=7, M=M)
    b = np.random.default_rng(2).normal(0, 2.0, N).astype(np.float16)
    y_ref = oracle.gemv_ref(p["x"], p["codes"], p["scales"], p["zeros"], bias=b)
    y = P.awq_gemv_w4a16(dev(p["x"]), dev(p["codes"]), dev(p["scales"]), dev(p["zeros"]), bias=dev(b))
    assert_close(host(y), y_ref)


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
