"""Pins for the oracle's quantizers and packing (CPU only).

Each check compares the oracle with something other than itself: hand-worked
fixtures, an independent scalar computation in Python floats (double
rounding of a single fp32 division through float64 is innocuous because
53 >= 2*24 + 2), round trips of on-grid values, and brute force over the
E2M1 grid.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from golden_io import read_golden


def f32(x: float) -> float:
    return struct.unpack("f", struct.pack("f", x))[0]


def f16(x: float) -> float:
    return struct.unpack("e", struct.pack("e", x))[0]


def round_half_even(x: float) -> int:
    return int(round(x))  # Python's round() is ties-to-even


# ---------------------------------------------------------------- packing --

def test_nibble_packing_golden():
    g = read_golden("nibble_pack.txt")
    codes = np.array([int(t) for t in g["codes"][0]])
    expect = np.array([int(t, 16) for t in g["bytes"][0]], dtype=np.uint8)
    packed = oracle.pack_nibbles(codes[None, :])[0]
    assert packed.tolist() == expect.tolist()
    assert oracle.unpack_nibbles(packed[None, :], signed=True)[0].tolist() == codes.tolist()


def test_nibble_roundtrip_random():
    rng = np.random.default_rng(0)
    c = rng.integers(-8, 8, (7, 130))
    assert (oracle.unpack_nibbles(oracle.pack_nibbles(c), signed=True) == c).all()
    u = rng.integers(0, 16, (3, 64))
    assert (oracle.unpack_nibbles(oracle.pack_nibbles(u), signed=False) == u).all()


# ------------------------------------------------------------------- INT4 --

def _int4_scalar(group_vals):
    """Independent scalar INT4 rule on Python floats (fp32 values in)."""
    amax = max(abs(v) for v in group_vals)
    s32 = f32(amax / 7.0)
    s16 = f16(min(s32, 65504.0))
    if s16 == 0.0:
        return [0] * len(group_vals), s16
    return [max(-7, min(7, round_half_even(f32(v / s16)))) for v in group_vals], s16


def test_int4_golden_cases():
    g = read_golden("int4_group.txt")
    for case in ("caseA", "caseB"):
        xs = [float(t) for t in g[case + "_x"][0]]
        qs = [int(t) for t in g[case + "_q"][0]]
        scale = float(g[case + "_scale"][0][0])
        X = np.zeros((1, 64), np.float16)
        X[0, :len(xs)] = xs
        codes, _, scales = oracle.quantize_act_ref(X, np.ones(64, np.float32), "int4_g64")
        assert float(scales[0, 0]) == scale
        assert codes[0, :len(qs)].tolist() == qs
        assert (codes[0, len(qs):] == 0).all()


def test_int4_on_grid_roundtrip():
    rng = np.random.default_rng(1)
    # fp16 scales spread over normal and subnormal fp16 range
    s16 = (2.0 ** rng.uniform(-20, 10, 400)).astype(np.float16)
    s16 = s16[s16 > 0]
    q = rng.integers(-7, 8, (s16.size, 64))
    q[:, 5] = np.where(rng.random(s16.size) < 0.5, 7, -7)     # amax = 7 * s16 exactly
    v = (q * s16.astype(np.float32)[:, None]).astype(np.float32)
    codes, scales = oracle.quantize_int4_g64(v)
    assert (scales[:, 0] == s16).all()
    assert (codes == q).all()


def test_int4_exhaustive_fp16_against_scalar_rule():
    """Every finite fp16 magnitude below a group max, for several group maxima,
    against the scalar rule written independently on Python floats."""
    allh = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)   # +0 .. max finite
    allv = np.concatenate([allh, -allh]).astype(np.float32)
    for amax in (1.0, 0.3330078125, 7.0, 1000.0, 6.1e-05, 3.0e-07):
        A = np.float32(np.float16(amax))
        xs = allv[np.abs(allv) <= A]
        pad = (-xs.size) % 63
        xs = np.concatenate([xs, np.zeros(pad, np.float32)]).reshape(-1, 63)
        grp = np.concatenate([np.full((xs.shape[0], 1), A, np.float32), xs], axis=1)
        codes, scales = oracle.quantize_int4_g64(grp)
        ref_codes, ref_s = _int4_scalar([float(A)] + [0.0])
        assert float(scales[0, 0]) == ref_s
        flat = grp.reshape(-1)
        want = np.array([max(-7, min(7, round_half_even(f32(float(v) / ref_s)))) if ref_s else 0
                         for v in flat])
        assert (codes.reshape(-1) == want).all(), amax


def test_int4_invariants_random():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal((64, 512)) * np.exp(rng.normal(0, 3, (64, 1)))).astype(np.float32)
    codes, s16 = oracle.quantize_int4_g64(v)
    s = np.repeat(s16.astype(np.float64), 64, axis=1)
    assert np.abs(codes).max() <= 7
    err = np.abs(v.astype(np.float64) - codes * s)
    unclamped = np.abs(codes) < 7
    assert (err[unclamped] <= s[unclamped] / 2 * (1 + 1e-6)).all()
    assert ((np.sign(codes) == np.sign(v)) | (codes == 0)).all()
    # odd symmetry: negating a group negates its codes and keeps its scale
    c2, s2 = oracle.quantize_int4_g64(-v)
    assert (c2 == -codes).all() and (s2 == s16).all()


def test_int4_zero_group_and_saturation():
    v = np.zeros((2, 64), np.float32)
    v[1, 0] = 1e9                       # amax/7 above fp16 max: scale saturates
    v[1, 1] = 65504.0 * 3
    codes, s16 = oracle.quantize_int4_g64(v)
    assert s16[0, 0] == 0 and (codes[0] == 0).all()
    assert float(s16[1, 0]) == 65504.0
    assert codes[1, 0] == 7 and codes[1, 1] == 3


def test_smoothing_multiply_is_single_fp32_rounding():
    rng = np.random.default_rng(3)
    X = (rng.standard_normal((4, 64)) * 30).astype(np.float16)
    si = np.exp(rng.normal(0, 2, 64)).astype(np.float32)
    xh = oracle.smooth_act(X, si)
    for i in range(4):
        for k in range(64):
            assert float(xh[i, k]) == f32(float(X[i, k]) * float(si[k]))


# -------------------------------------------------------------------- FP4 --

def test_fp4_golden_table():
    g = read_golden("fp4_e2m1.txt")
    for amax_s, code_s in g["e8m0"]:
        v = np.zeros((1, 32), np.float32)
        v[0, 7] = np.float32(float(amax_s))
        _, sc = oracle.quantize_fp4_b32(v)
        assert int(sc[0, 0]) == int(code_s), amax_s
    for x_s, code_s in g["e2m1"]:
        v = np.zeros((1, 32), np.float32)
        v[0, 0] = 6.0
        v[0, 3] = np.float32(float(x_s))
        codes, sc = oracle.quantize_fp4_b32(v)
        assert sc[0, 0] == 127
        assert int(codes[0, 3]) == int(code_s), x_s


def test_fp4_all_codes_roundtrip_every_exponent():
    grid = oracle.E2M1_VALUES
    # 6 * 2^e must stay finite in fp32, so e <= 125; at e = -127 every value
    # is an exact fp32 subnormal.
    for e in range(-127, 126):
        vals = np.array([grid[c & 7] * (-1 if c & 8 else 1) for c in range(16)], np.float64)
        v = np.zeros((1, 32), np.float64)
        v[0, :16] = vals
        v[0, 16:] = vals[::-1]
        v = v * 2.0 ** e
        v32 = v.astype(np.float32)
        assert (v32.astype(np.float64) == v).all()
        codes, sc = oracle.quantize_fp4_b32(v32)
        assert int(sc[0, 0]) == e + 127
        back = oracle.dequantize(codes, sc, "fp4_b32")
        assert (back == v).all(), e


def _nearest_e2m1(u: float) -> int:
    """Brute force: nearest magnitude, ties to the even code, saturating."""
    best = None
    for c, gv in enumerate(oracle.E2M1_VALUES.tolist()):
        d = abs(Fraction(u) - Fraction(gv))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_fp4_rounding_brute_force():
    rng = np.random.default_rng(4)
    u = np.concatenate([rng.uniform(0, 6, 3000), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0],
                        np.nextafter(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32), 0),
                        np.nextafter(np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32), 7)])
    u = u.astype(np.float32)
    n = u.size
    pad = (-n) % 31
    blocks = np.concatenate([u, np.zeros(pad, np.float32)]).reshape(-1, 31)
    v = np.concatenate([np.full((blocks.shape[0], 1), 6.0, np.float32), blocks], axis=1)
    sgn = np.where(rng.random(v.shape) < 0.5, -1, 1).astype(np.float32)
    sgn[:, 0] = 1
    v = v * sgn
    codes, sc = oracle.quantize_fp4_b32(v)
    assert (sc == 127).all()
    for i in range(v.shape[0]):
        for j in range(32):
            want = _nearest_e2m1(abs(float(v[i, j]))) | (8 if np.signbit(v[i, j]) else 0)
            assert int(codes[i, j]) == want, (float(v[i, j]), int(codes[i, j]), want)


def test_fp4_scale_is_ceiling():
    """6 * 2^(e-1) < amax <= 6 * 2^e across the fp32 range (E8M0 not clamped)."""
    rng = np.random.default_rng(5)
    amax = (2.0 ** rng.uniform(-120, 120, 5000) * rng.uniform(1, 2, 5000)).astype(np.float32)
    amax = np.concatenate([amax, np.float32([1.5 * 2.0 ** k for k in range(-100, 100)]),
                           np.float32([6.0 * 2.0 ** k for k in range(-100, 100)])])
    v = np.zeros((amax.size, 32), np.float32)
    v[:, 3] = amax
    _, sc = oracle.quantize_fp4_b32(v)
    e = sc.astype(np.int64)[:, 0] - 127
    a = amax.astype(np.float64)
    assert (6.0 * np.ldexp(1.0, e) >= a).all()
    assert (6.0 * np.ldexp(1.0, e - 1) < a).all()


def test_fp4_zero_block():
    v = np.zeros((1, 64), np.float32)
    v[0, 40] = -3.0
    codes, sc = oracle.quantize_fp4_b32(v)
    assert sc[0, 0] == 0 and (codes[0, :32] == 0).all()
    assert sc[0, 1] == 126 and codes[0, 40] == (7 | 8)   # -3 / 2^-1 = -6, code 7 is 6.0
