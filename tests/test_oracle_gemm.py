"""Pins for the oracle's group-scaled GEMM, forward pass, GELU and AWQ GEMV
(CPU only): hand-worked fixtures, exact rational brute force on tiny shapes,
integer special cases, and closed-form identities.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from golden_io import read_golden


def test_gemm_golden_tiny():
    g = read_golden("gemm_tiny.txt")
    qx = np.concatenate([np.full(64, 1), np.full(64, 2)])[None, :]
    qw = np.concatenate([np.full(64, 3), np.full(64, -1)])[None, :]
    sx = np.array([[0.5, 0.25]], np.float16)
    sw = np.array([[2.0, 4.0]], np.float16)
    b = np.array([0.5], np.float16)
    y0 = oracle.gemm_ref(qx, sx, np.zeros((1, 0)), qw, sw, np.zeros((1, 0)), b, "int4_g64")
    y1 = oracle.gemm_ref(qx, sx, np.array([[2.0]]), qw, sw, np.array([[0.25]], np.float16), b, "int4_g64")
    assert y0[0, 0] == float(g["y_r0"][0][0])
    assert y1[0, 0] == float(g["y_r1"][0][0])


def _frac_gemm(qx, sx, la, qw, sw, lu, bias, fmt):
    """Exact rational evaluation of the group-scaled GEMM contract."""
    M, K = qx.shape
    N = qw.shape[0]
    G = 64 if fmt == "int4_g64" else 32

    def val(c, s, fmt):
        if fmt == "int4_g64":
            return Fraction(int(c)) * Fraction(float(s))
        mag = Fraction(float(oracle.E2M1_VALUES[int(c) & 7]))
        return (-mag if int(c) & 8 else mag) * Fraction(2) ** (int(s) - 127)

    out = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for j in range(la.shape[1]):
                acc += Fraction(float(la[m, j])) * Fraction(float(lu[n, j]))
            for gi in range(K // G):
                part = Fraction(0)
                for k in range(gi * G, (gi + 1) * G):
                    part += val(qx[m, k], sx[m, gi], fmt) * val(qw[n, k], sw[n, gi], fmt)
                acc += part
            out[m, n] = acc + Fraction(float(bias[n]))
    return out


@pytest.mark.parametrize("fmt", ["int4_g64", "fp4_b32"])
def test_gemm_rational_brute_force(fmt):
    rng = np.random.default_rng(7)
    M, N, K, r = 3, 5, 128, 4
    if fmt == "int4_g64":
        qx = rng.integers(-7, 8, (M, K))
        qw = rng.integers(-7, 8, (N, K))
        sx = rng.uniform(0.01, 3, (M, K // 64)).astype(np.float16)
        sw = rng.uniform(0.001, 0.1, (N, K // 64)).astype(np.float16)
    else:
        qx = rng.integers(0, 16, (M, K))
        qw = rng.integers(0, 16, (N, K))
        sx = rng.integers(110, 140, (M, K // 32)).astype(np.uint8)
        sw = rng.integers(110, 140, (N, K // 32)).astype(np.uint8)
    la = rng.standard_normal((M, r)).astype(np.float32)
    lu = rng.standard_normal((N, r)).astype(np.float16)
    b = rng.standard_normal(N).astype(np.float16)
    y = oracle.gemm_ref(qx, sx, la, qw, sw, lu, b, fmt)
    exact = _frac_gemm(qx, sx, la, qw, sw, lu, b, fmt)
    for m in range(M):
        for n in range(N):
            e = float(exact[m, n])
            assert abs(y[m, n] - e) <= 1e-13 * (abs(e) + 1e-300) + 1e-300


def test_gemm_integer_special_case():
    """All scales 1 and rank 0: the contract is an exact integer matmul."""
    rng = np.random.default_rng(8)
    qx = rng.integers(-7, 8, (17, 256))
    qw = rng.integers(-7, 8, (9, 256))
    ones_x = np.ones((17, 4), np.float16)
    ones_w = np.ones((9, 4), np.float16)
    y = oracle.gemm_ref(qx, ones_x, np.zeros((17, 0)), qw, ones_w, np.zeros((9, 0)), None, "int4_g64")
    assert (y == (qx.astype(np.int64) @ qw.astype(np.int64).T)).all()


def test_forward_reduces_to_dense_at_full_rank_zero_residual():
    """With every weight in the low-rank branch and zero 4-bit codes the
    forward pass is X W^T + b on the factors' product."""
    rng = np.random.default_rng(9)
    M, K, N = 8, 64, 16
    X = rng.standard_normal((M, K)).astype(np.float16)
    ld = rng.standard_normal((N, K)).astype(np.float16)     # r = N
    lu = np.eye(N, dtype=np.float16)
    layer = {"fmt": "int4_g64", "lora_down": ld, "lora_up": lu,
             "w_codes_unpacked": np.zeros((N, K), np.int8), "w_scales": np.ones((N, 1), np.float16)}
    b = rng.standard_normal(N).astype(np.float16)
    y = oracle.forward_ref(X, layer, np.zeros((M, K), np.int8), np.ones((M, 1), np.float16), b)
    assert np.allclose(y, oracle.dense_ref(X, ld, b), rtol=1e-13, atol=1e-13)


def test_gelu_tanh_identities():
    y = np.linspace(-12, 12, 20001)
    g = oracle.gelu_tanh(y)
    # gelu(y) - gelu(-y) = y for the tanh form
    assert np.allclose(g - oracle.gelu_tanh(-y), y, rtol=0, atol=1e-12)
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    # close to the exact erf form (the tanh form is an approximation of it)
    erf = np.vectorize(math.erf)
    exact = 0.5 * y * (1 + erf(y / math.sqrt(2)))
    assert np.abs(g - exact).max() < 1e-3
    # tails: identity for large y, zero for very negative y
    assert abs(oracle.gelu_tanh(np.array([30.0]))[0] - 30.0) < 1e-12
    assert abs(oracle.gelu_tanh(np.array([-30.0]))[0]) < 1e-12


def test_awq_golden():
    g = read_golden("awq_gemv.txt")
    q = np.tile(np.arange(16), 4)[None, :]
    codes = oracle.pack_nibbles(q)
    s = np.array([[0.5]], np.float16)
    z = np.array([[8.0]], np.float16)
    x1 = np.ones((1, 64), np.float16)
    x2 = np.zeros((1, 64), np.float16)
    x2[0, 0::2] = 1
    assert oracle.gemv_ref(x1, codes, s, z)[0, 0] == float(g["y_all_ones"][0][0])
    assert oracle.gemv_ref(x2, codes, s, z)[0, 0] == float(g["y_even_ones"][0][0])
    # the bias is a plain per-channel offset: alone when x is zero, added otherwise
    b = np.array([-2.25], np.float16)
    assert oracle.gemv_ref(np.zeros((1, 64), np.float16), codes, s, z, bias=b)[0, 0] == -2.25
    assert oracle.gemv_ref(x1, codes, s, z, bias=b)[0, 0] == float(g["y_all_ones"][0][0]) - 2.25


def test_awq_integer_special_case_and_rational():
    rng = np.random.default_rng(10)
    N, K = 6, 192
    q = rng.integers(0, 16, (N, K))
    codes = oracle.pack_nibbles(q)
    x = rng.integers(-3, 4, (2, K)).astype(np.float16)
    y = oracle.gemv_ref(x, codes, np.ones((N, 3), np.float16), np.zeros((N, 3), np.float16))
    assert (y == x.astype(np.int64) @ q.T).all()
    s = rng.uniform(0.001, 0.1, (N, 3)).astype(np.float16)
    z = rng.integers(0, 16, (N, 3)).astype(np.float16)
    xr = rng.standard_normal((2, K)).astype(np.float16)
    y = oracle.gemv_ref(xr, codes, s, z)
    for m in range(2):
        for n in range(N):
            acc = Fraction(0)
            for gi in range(3):
                part = Fraction(0)
                for k in range(gi * 64, gi * 64 + 64):
                    part += Fraction(float(xr[m, k])) * (int(q[n, k]) - Fraction(float(z[n, gi])))
                acc += part * Fraction(float(s[n, gi]))
            assert abs(y[m, n] - float(acc)) <= 1e-13 * abs(float(acc)) + 1e-12


def test_awq_prep_error_bound():
    d = synth.make_gemv_inputs(synth.CONFIGS["gemv"], seed=0)
    W = d["W"][:64]
    p = oracle.awq_prep(W)
    Wd = oracle.awq_dequantize(p["codes"], p["scales"], p["zeros"])
    s = np.repeat(p["scales"].astype(np.float64), 64, axis=1)
    err = np.abs(Wd - W.astype(np.float64))
    # min-max grid: every weight within one step, nearly all within half a step
    assert (err <= s * 1.0 + 1e-12).all()
    assert (err <= s / 2 * (1 + 1e-3)).mean() > 0.99
    assert set(np.unique(p["zeros"]).tolist()) <= set(range(16))


def test_mlp_chain_is_the_composition_and_pins_hold():
    """The chain adds no arithmetic of its own: with all-zero up-projection codes
    and rank 0 the up-projection is the bias, so U = GELU(bias) in every row, and
    the chain's quantizer sees exactly that (closed form through the pinned GELU
    and quantizer)."""
    M, K, N = 3, 128, 128
    b = (np.arange(N) / 16.0 - 4.0).astype(np.float16)
    z = np.zeros((M, K), np.int64)
    s1 = np.ones((M, K // 64), np.float16)
    U16, codes, packed, scales, la2 = oracle.mlp_chain_ref(
        z, s1, np.zeros((M, 0)), np.zeros((N, K), np.int64), np.ones((N, K // 64), np.float16),
        np.zeros((N, 0)), b, "int4_g64", np.ones(N, np.float32), np.zeros((0, N), np.float16))
    want = oracle.gelu_tanh(b.astype(np.float64)).astype(np.float16)
    assert np.array_equal(U16, np.broadcast_to(want, (M, N)))
    c2, _, s2 = oracle.quantize_act_ref(np.broadcast_to(want, (M, N)), np.ones(N, np.float32), "int4_g64")
    assert np.array_equal(codes, c2) and np.array_equal(scales.view(np.uint16), s2.view(np.uint16))
    assert la2.shape == (M, 0)
