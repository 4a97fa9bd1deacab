"""Pins for the oracle's offline preparation and the method-level claim
(CPU only): smoothing balance and invariance, full-rank exactness,
Eckart-Young truncation error from an independent eigenvalue routine,
residual identity, and "smoothing + low-rank + 4-bit residual beats plain
4-bit" on the tiny DiT-like layer with outlier channels.
"""
import numpy as np
import pytest

import oracle
import synth

TINY = synth.CONFIGS["tiny"]


@pytest.fixture(scope="module")
def tiny():
    d = synth.make_layer_inputs(TINY, seed=0)
    si = oracle.smoothing_factors(d["X_cal"], d["W"], TINY.alpha)
    return d, si


def test_smoothing_balances_channel_maxima(tiny):
    """alpha = 0.5: after migration, max|X_hat| and max|W_hat| agree per channel."""
    d, si = tiny
    a = np.abs(d["X_cal"].astype(np.float64)).max(0) * si.astype(np.float64)
    w = np.abs(d["W"].astype(np.float64)).max(0) / si.astype(np.float64)
    assert np.allclose(a, w, rtol=1e-6)
    # outlier channels are pulled down by about sqrt(outlier scale)
    assert si[d["outliers"]].mean() < 0.5 * np.median(si)


def test_smoothing_invariance(tiny):
    """X_hat W_hat = X W in real arithmetic (float64 here, rel 1e-13)."""
    d, si = tiny
    X = d["X"].astype(np.float64)
    W = d["W"].astype(np.float64)
    lam = 1.0 / si.astype(np.float64)
    lhs = (X * si.astype(np.float64)) @ (W * lam[None, :]).T
    rhs = X @ W.T
    assert np.linalg.norm(lhs - rhs) <= 1e-13 * np.linalg.norm(rhs)


def test_full_rank_split_is_exact(tiny):
    d, si = tiny
    W_hat = d["W"].astype(np.float64).T / si.astype(np.float64)[:, None]
    L1, L2, _ = oracle.lowrank_factors(W_hat, min(W_hat.shape))
    assert np.linalg.norm(W_hat - L1 @ L2) <= 1e-12 * np.linalg.norm(W_hat)


@pytest.mark.parametrize("r", [1, 8, 16, 64])
def test_eckart_young(tiny, r):
    """||W_hat - L1 L2||_F^2 = sum of the discarded sigma^2, with sigma^2 from
    the eigenvalues of W_hat^T W_hat (a different LAPACK routine)."""
    d, si = tiny
    W_hat = d["W"].astype(np.float64).T / si.astype(np.float64)[:, None]
    L1, L2, _ = oracle.lowrank_factors(W_hat, r)
    ev = np.sort(np.linalg.eigvalsh(W_hat.T @ W_hat))[::-1]
    tail = np.sqrt(max(ev[r:].sum(), 0.0))
    assert abs(np.linalg.norm(W_hat - L1 @ L2) - tail) <= 1e-8 * np.linalg.norm(W_hat)
    # and nothing of rank r does better than a random rank-r projection of W_hat
    rng = np.random.default_rng(r)
    Q, _ = np.linalg.qr(rng.standard_normal((W_hat.shape[1], r)))
    assert np.linalg.norm(W_hat - L1 @ L2) <= np.linalg.norm(W_hat - (W_hat @ Q) @ Q.T)


def test_residual_identity_and_quantization_error(tiny):
    d, si = tiny
    layer = oracle.prep_svdq_layer(d["W"], si, TINY.rank, "int4_g64")
    lam = 1.0 / si.astype(np.float64)
    W_hat = d["W"].astype(np.float64).T * lam[:, None]
    low = (lam[:, None] * layer["lora_down"].T.astype(np.float64)) @ layer["lora_up"].T.astype(np.float64)
    assert np.abs(low + layer["residual_kn"] - W_hat).max() <= 1e-14 * np.abs(W_hat).max()
    # every dequantized residual weight lies within half a step of R
    deq = oracle.dequantize(layer["w_codes_unpacked"], layer["w_scales"], "int4_g64")
    R = layer["residual_kn"].T
    s = np.repeat(layer["w_scales"].astype(np.float64), 64, axis=1)
    assert (np.abs(deq - R) <= s / 2 + 1e-7 * np.abs(R) + 1e-30).all()
    assert layer["lora_down"].shape == (TINY.rank, TINY.K)
    assert layer["lora_up"].shape == (TINY.N, TINY.rank)
    assert layer["w_codes"].shape == (TINY.N, TINY.K // 2)


def _layer_error(d, si, rank, fmt):
    ga = oracle.nvfp4_act_global_scale(d["X_cal"], si) if fmt == "nvfp4_g16" else None
    layer = oracle.prep_svdq_layer(d["W"], si, rank, fmt, act_gscale=ga)
    codes, _, scales = oracle.quantize_act_ref(d["X"], si, fmt, ga)
    y = oracle.forward_ref(d["X"], layer, codes, scales, d["bias"])
    y_ref = oracle.dense_ref(d["X"], d["W"], d["bias"])
    return np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref)


@pytest.mark.parametrize("fmt", ["int4_g64", "fp4_b32", "nvfp4_g16"])
def test_method_beats_plain_w4a4(tiny, fmt):
    """The pages' claim (outliers migrate to the weights, a 16-bit low-rank
    branch takes the hardest part, the residual goes to 4 bits) must make
    the layer more accurate than plain W4A4 with the same quantizer."""
    d, si = tiny
    plain = _layer_error(d, np.ones(TINY.K, np.float32), 0, fmt)
    smooth_only = _layer_error(d, si, 0, fmt)
    svdq = _layer_error(d, si, TINY.rank, fmt)
    print(f"{fmt}: plain {plain:.4e}  smooth {smooth_only:.4e}  svdq r16 {svdq:.4e}")
    assert svdq < plain
    assert smooth_only < plain


def test_rank_sweep_reported(tiny):
    """Error against rank (reported; a non-monotone step is a finding)."""
    d, si = tiny
    errs = [_layer_error(d, si, r, "int4_g64") for r in (0, 8, 16, 32)]
    print("rank 0/8/16/32 rel err:", ["%.4e" % e for e in errs])
    assert errs[-1] < errs[0]


def test_nvfp4_residual_within_half_step(tiny):
    """NVFP4 prep: every dequantized residual weight is within half an E2M1
    step (at most one unit of the block divisor, the 4-to-6 gap) of R, or
    clipped at the block's top code; the per-tensor scale is the amax rule."""
    d, si = tiny
    ga = oracle.nvfp4_act_global_scale(d["X_cal"], si)
    layer = oracle.prep_svdq_layer(d["W"], si, TINY.rank, "nvfp4_g16", act_gscale=ga)
    R = layer["residual_kn"].T.astype(np.float32).astype(np.float64)
    assert layer["w_gscale"] == np.float32(np.max(np.abs(R)) / np.float32(2688.0))
    deq = oracle.dequantize(layer["w_codes_unpacked"], layer["w_scales"], "nvfp4_g16", layer["w_gscale"])
    unit = np.repeat(oracle.e4m3_value(layer["w_scales"]) * float(layer["w_gscale"]), 16, axis=1)
    err = np.abs(deq - R)
    assert (err <= unit + 1e-6 * np.abs(R)).all()
    assert np.linalg.norm(deq - R) / np.linalg.norm(R) < 0.15


@pytest.mark.parametrize("alpha", ["0.5", "0.25"])
def test_smoothing_factors_hand_worked(alpha):
    """tests/golden/smoothing.txt: the alpha rule (alpha 0.25 tells a^alpha /
    w^(1 - alpha) from the rule with the exponents exchanged), and lambda = 1
    for an all-zero calibration column and for an all-zero weight column."""
    from tests.golden_io import read_golden
    g = read_golden("smoothing.txt")
    X_cal = np.array([[float(v) for v in row] for row in g["xcal"]], np.float16)
    W = np.array([[float(v) for v in row] for row in g["w"]], np.float16)
    want = np.array([int(h, 16) for h in g[f"si_a{alpha}"][0]], np.uint32)
    si = oracle.smoothing_factors(X_cal, W, float(alpha))
    assert si.dtype == np.float32
    assert np.array_equal(si.view(np.uint32), want), [hex(v) for v in si.view(np.uint32)]
