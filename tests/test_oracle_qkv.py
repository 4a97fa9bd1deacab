"""Pins for the fused-QKV-epilogue oracle (oracle/qkv.py): hand-worked
fixtures, closed forms and invariants of RMSNorm and of the pair rotation."""
import numpy as np
import pytest

import oracle
from golden_io import read_golden


@pytest.mark.parametrize("case", ["a", "b"])
def test_golden_cases(case):
    g = read_golden("qkv_norm_rope.txt")
    f = lambda k: np.array([float(t) for t in g[f"{case}_{k}"][0]])
    D = int(g[f"{case}_head_dim"][0][0])
    y = f("y_lin")[None, :]
    out = oracle.qkv_epilogue_ref(y, D, f("q_norm_w"), f("k_norm_w"), f("cos")[None, :],
                                  f("sin")[None, :], eps=float(g[f"{case}_eps"][0][0]))
    np.testing.assert_allclose(out[0], f("out"), rtol=0, atol=1e-12)


def test_rmsnorm_unit_rms_and_eps_closed_form():
    rng = np.random.default_rng(0)
    y = rng.standard_normal((5, 3 * 64)) * 3.0
    n0 = oracle.rms_norm_heads(y, 64, np.ones(64), 0.0).reshape(5, 3, 64)
    np.testing.assert_allclose(np.sqrt(np.mean(n0 ** 2, axis=-1)), 1.0, rtol=1e-13)
    eps = 0.7
    n1 = oracle.rms_norm_heads(y, 64, np.ones(64), eps).reshape(5, 3, 64)
    ms = np.mean(y.reshape(5, 3, 64) ** 2, axis=-1)
    np.testing.assert_allclose(np.mean(n1 ** 2, axis=-1), ms / (ms + eps), rtol=1e-13)


def test_rmsnorm_weight_and_scale():
    rng = np.random.default_rng(1)
    y = rng.standard_normal((4, 2 * 32))
    w = rng.standard_normal(32)
    np.testing.assert_allclose(oracle.rms_norm_heads(y, 32, w, 0.0),
                               np.tile(w, 2) * oracle.rms_norm_heads(y, 32, np.ones(32), 0.0), rtol=1e-13)
    np.testing.assert_allclose(oracle.rms_norm_heads(7.5 * y, 32, w, 0.0),
                               oracle.rms_norm_heads(y, 32, w, 0.0), rtol=1e-12)


def test_rope_identity_quarter_turn_and_norms():
    rng = np.random.default_rng(2)
    y = rng.standard_normal((3, 2 * 16))
    one, zero = np.ones((3, 8)), np.zeros((3, 8))
    np.testing.assert_array_equal(oracle.rope_pairs(y, 16, one, zero), y)
    q = oracle.rope_pairs(y, 16, zero, one).reshape(3, 2, 8, 2)
    p = y.reshape(3, 2, 8, 2)
    np.testing.assert_array_equal(q[..., 0], -p[..., 1])
    np.testing.assert_array_equal(q[..., 1], p[..., 0])
    th = rng.uniform(-10, 10, (3, 8))
    r = oracle.rope_pairs(y, 16, np.cos(th), np.sin(th)).reshape(3, 2, 8, 2)
    np.testing.assert_allclose(np.hypot(r[..., 0], r[..., 1]), np.hypot(p[..., 0], p[..., 1]), rtol=1e-13)


def test_rope_composition():
    rng = np.random.default_rng(3)
    y = rng.standard_normal((2, 16))
    t1, t2 = rng.uniform(-3, 3, (2, 8)), rng.uniform(-3, 3, (2, 8))
    two = oracle.rope_pairs(oracle.rope_pairs(y, 16, np.cos(t1), np.sin(t1)), 16, np.cos(t2), np.sin(t2))
    one = oracle.rope_pairs(y, 16, np.cos(t1 + t2), np.sin(t1 + t2))
    np.testing.assert_allclose(two, one, rtol=1e-12, atol=1e-12)


def test_parts_are_independent_and_v_passes():
    rng = np.random.default_rng(4)
    D, H, M = 8, 2, 3
    y = rng.standard_normal((M, 3 * H * D))
    w = rng.standard_normal(D)
    th = rng.uniform(-3, 3, (M, D // 2))
    a = oracle.qkv_epilogue_ref(y, D, w, 2 * w, np.cos(th), np.sin(th))
    np.testing.assert_array_equal(a[:, 2 * H * D:], y[:, 2 * H * D:])
    y2 = y.copy()
    y2[:, 2 * H * D:] += 5.0
    y2[:, H * D:2 * H * D] *= 3.0   # K: scale invariance of the norm (eps small)
    b = oracle.qkv_epilogue_ref(y2, D, w, 2 * w, np.cos(th), np.sin(th), eps=0.0)
    a0 = oracle.qkv_epilogue_ref(y, D, w, 2 * w, np.cos(th), np.sin(th), eps=0.0)
    np.testing.assert_array_equal(b[:, :H * D], a0[:, :H * D])
    np.testing.assert_allclose(b[:, H * D:2 * H * D], a0[:, H * D:2 * H * D], rtol=1e-12)
