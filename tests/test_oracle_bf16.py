"""Pins of the oracle's bfloat16 support (the pages' compute_dtype): the
rounding against hand-worked ties, exact rationals and torch's CPU
conversion; the smoothing multiply on bf16 inputs; the offline preparation
with bf16 low-rank factors."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth


def test_bf16_round_hand_worked():
    f = lambda v: float(oracle.bf16_round(np.array([v], np.float32))[0])
    assert f(1 + 2 ** -8) == 1.0                   # halfway, the even neighbour is 1.0
    assert f(1 + 3 * 2 ** -8) == 1 + 2 ** -6       # halfway between 1+2^-7 (odd) and 1+2^-6 (even)
    assert f(1 + 2 ** -8 + 2 ** -20) == 1 + 2 ** -7
    assert f(-(1 + 2 ** -8 - 2 ** -20)) == -1.0
    assert f(3.3895313892515355e38) == 3.3895313892515355e38   # the largest bf16
    assert f(3.4028234663852886e38) == float("inf")            # beyond the last midpoint
    assert np.signbit(oracle.bf16_round(np.array([-0.0], np.float32)))[0]
    assert np.isnan(f(float("nan")))


def _nearest_even_bf16(x: float) -> float:
    """Brute force over the two bf16 neighbours of x with exact rationals."""
    fx = Fraction(x)
    if fx == 0:
        return x
    a = abs(fx)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    e = max(e, -126)                               # subnormals share the quantum 2^-133
    q = Fraction(2) ** (e - 7)
    lo = (abs(fx) // q) * q
    hi = lo + q
    d_lo, d_hi = abs(fx) - lo, hi - abs(fx)
    if d_lo < d_hi or (d_lo == d_hi and (lo / q) % 2 == 0):
        r = lo
    else:
        r = hi
    return float(r) if fx > 0 else -float(r)


def test_bf16_round_brute_force():
    rng = np.random.default_rng(41)
    base = (rng.standard_normal(3000) * 2.0 ** rng.integers(-140, 120, 3000)).astype(np.float32)
    # exact halfway points and their fp32 neighbours
    b = oracle.bf16_round(base).astype(np.float64)
    ties = (b + np.abs(b) * 2.0 ** -8).astype(np.float32)
    x = np.concatenate([base, ties, np.nextafter(ties, np.float32(0)), np.nextafter(ties, np.float32(np.inf))])
    x = x[np.isfinite(x)]
    got = oracle.bf16_round(x)
    for v, g in zip(x.tolist(), got.tolist()):
        assert g == _nearest_even_bf16(v), v


def test_bf16_round_matches_torch_cpu():
    rng = np.random.default_rng(42)
    x = (rng.standard_normal(200000) * 2.0 ** rng.integers(-130, 100, 200000)).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.bf16_round(x).view(np.uint32), want.view(np.uint32))


def test_smooth_act_bf16_inputs():
    X = oracle.bf16_round(np.random.default_rng(43).standard_normal((4, 64)).astype(np.float32) * 7)
    si = np.random.default_rng(44).uniform(0.1, 3, 64).astype(np.float32)
    xh = oracle.smooth_act(X, si)
    for i in range(4):
        for k in range(64):
            assert float(xh[i, k]) == float(np.float32(float(X[i, k]) * float(si[k])))
    with pytest.raises(ValueError):
        oracle.smooth_act(np.full((1, 64), 0.1, np.float32), si)   # not a bf16 value


def test_prep_bf16_factors():
    cfg = synth.CONFIGS["tiny"]
    d = synth.make_layer_inputs(cfg, seed=0)
    si = oracle.smoothing_factors(d["X_cal"], d["W"], cfg.alpha)
    layer = oracle.prep_svdq_layer(d["W"], si, cfg.rank, "int4_g64", dtype="bfloat16")
    for name in ("lora_down", "lora_up"):
        a = layer[name]
        assert a.dtype == np.float32 and not (a.view(np.uint32) & 0xFFFF).any()
    lam = 1.0 / si.astype(np.float64)
    W_hat = d["W"].astype(np.float64).T * lam[:, None]
    low = (lam[:, None] * layer["lora_down"].T.astype(np.float64)) @ layer["lora_up"].T.astype(np.float64)
    assert np.abs(low + layer["residual_kn"] - W_hat).max() <= 1e-14 * np.abs(W_hat).max()
    # the layer keeps the method's accuracy with bf16 factors and bf16 inputs
    X = oracle.bf16_round(d["X"].astype(np.float32))
    codes, _, scales = oracle.quantize_act_ref(X, si, "int4_g64")
    y = oracle.forward_ref(X, layer, codes, scales, d["bias"])
    y_ref = oracle.dense_ref(X, d["W"], d["bias"])
    assert np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref) < 0.08
