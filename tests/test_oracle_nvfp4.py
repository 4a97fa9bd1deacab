"""Pins of the oracle's NVFP4 format (E2M1 codes, E4M3 scale per 16, fp32
scale per tensor): hand-worked fixtures (tests/golden/nvfp4.txt), every E4M3
code round-tripping, brute-force nearest rounding with exact rationals,
saturation, on-grid round trips, and the GEMM contract in exact rationals."""
from fractions import Fraction

import numpy as np

import oracle.svdq as O
from golden_io import read_golden


def _e4m3_grid():
    """All finite non-negative E4M3 values by byte, from the format's
    definition written out directly (independent of e4m3_value)."""
    vals = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        vals.append(Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7))
    return vals


def test_e4m3_golden():
    g = read_golden("nvfp4.txt")
    for code, val in g["e4m3_dec"]:
        assert float(O.e4m3_value(int(code, 16))) == float(val), code
    for val, code in g["e4m3_enc"]:
        assert int(O.e4m3_rne(np.array([float(val)], np.float32))[0]) == int(code, 16), val
    assert np.isnan(O.e4m3_value(0x7F)) and np.isnan(O.e4m3_value(0xFF))


def test_e4m3_every_code_round_trips_and_matches_definition():
    grid = _e4m3_grid()
    for c in range(0x7F):
        assert Fraction(float(O.e4m3_value(c))) == grid[c]
        assert float(O.e4m3_value(c | 0x80)) == -float(grid[c])
        assert int(O.e4m3_rne(np.array([float(grid[c])], np.float32))[0]) == c


def test_e4m3_rounding_brute_force():
    grid = _e4m3_grid()
    rng = np.random.default_rng(21)
    mids = [float((grid[i] + grid[i + 1]) / 2) for i in range(len(grid) - 1)]
    a = np.concatenate([rng.uniform(0, 460, 4000), 2.0 ** rng.uniform(-12, 9, 4000), mids,
                        np.nextafter(np.float32(mids), np.float32(0)),
                        np.nextafter(np.float32(mids), np.float32(1000))]).astype(np.float32)
    got = O.e4m3_rne(a)
    for x, c in zip(a.tolist(), got.tolist()):
        fx = Fraction(x)
        if fx >= 448:
            assert c == 0x7E
            continue
        best = min(range(0x7F), key=lambda i: (abs(fx - grid[i]), i % 2))
        assert c == best, (x, c, best)


def test_nvfp4_golden_blocks():
    g = read_golden("nvfp4.txt")
    for b in ("blockA", "blockB"):
        v = np.array([[float(t) for t in g[b + "_v"][0]]], np.float32)
        codes, sc = O.quantize_nvfp4_g16(v, np.float32(float(g[b + "_g"][0][0])))
        assert [int(t) for t in codes[0]] == [int(t) for t in g[b + "_codes"][0]], b
        assert int(sc[0, 0]) == int(g[b + "_scale"][0][0]), b


def test_nvfp4_codes_are_nearest_given_scale():
    rng = np.random.default_rng(22)
    v = (rng.standard_normal((40, 64)) * 2.0 ** rng.integers(-8, 8, (40, 1))).astype(np.float32)
    v[3, :16] = 0
    for gsc in (np.float32(0.37), np.float32(1e-3), O.nvfp4_global_scale(np.max(np.abs(v)))):
        codes, sc = O.quantize_nvfp4_g16(v, gsc)
        d6 = np.float32(np.float32(6.0) * gsc)
        for i in range(v.shape[0]):
            for blk in range(4):
                seg = v[i, 16 * blk:16 * blk + 16]
                sf = np.float32(np.max(np.abs(seg)) / d6)
                assert sc[i, blk] == O.e4m3_rne(np.array([sf]))[0]
                d = np.float32(np.float32(O.e4m3_value(sc[i, blk])) * gsc)
                for j in range(16):
                    c = int(codes[i, 16 * blk + j])
                    if d == 0:
                        assert c == 0
                        continue
                    u = abs(Fraction(float(np.float32(seg[j] / d))))
                    best = min(range(8), key=lambda k: (abs(u - Fraction(float(O.E2M1_VALUES[k]))), k % 2))
                    assert c == (best | (8 if np.signbit(seg[j]) else 0))


def test_nvfp4_on_grid_round_trip_and_zero_block():
    gsc = np.float32(0.25)
    rng = np.random.default_rng(23)
    # a block whose largest magnitude is 6 * E4M3(s) * g reproduces exactly
    for s in (0x01, 0x08, 0x2A, 0x38, 0x45, 0x7E):
        sval = float(O.e4m3_value(s))
        c = rng.integers(0, 16, 16)
        c[0] = 7
        vals = np.where(c & 8, -1, 1) * O.E2M1_VALUES[c & 7] * sval * float(gsc)
        v = vals.astype(np.float32)[None, :]
        assert (v.astype(np.float64) == vals).all()
        codes, sc = O.quantize_nvfp4_g16(v, gsc)
        assert int(sc[0, 0]) == s
        back = O.dequantize(codes, sc, "nvfp4_g16", gsc)
        assert (back == vals).all(), s
    codes, sc = O.quantize_nvfp4_g16(np.zeros((1, 32), np.float32), gsc)
    assert (codes == 0).all() and (sc == 0).all()


def test_nvfp4_global_scale_puts_the_largest_block_on_448():
    x = np.array([[0.1, -5000.0] + [1.0] * 14], np.float32)
    g = O.nvfp4_global_scale(5000.0)
    _, sc = O.quantize_nvfp4_g16(x, g)
    assert sc[0, 0] == 0x7E
    assert O.nvfp4_global_scale(0.0) == 1.0


def test_nvfp4_gemm_rational():
    rng = np.random.default_rng(24)
    M, N, K = 3, 4, 64
    qx, qw = rng.integers(0, 16, (M, K)), rng.integers(0, 16, (N, K))
    sx = rng.integers(0, 0x7F, (M, K // 16)).astype(np.uint8)
    sw = rng.integers(0, 0x7F, (N, K // 16)).astype(np.uint8)
    gx, gw = np.float32(0.013), np.float32(7.5e-4)
    y = O.gemm_ref(qx, sx, np.zeros((M, 0)), qw, sw, np.zeros((N, 0)), None, "nvfp4_g16",
                   act_gscale=gx, w_gscale=gw)
    grid = _e4m3_grid()

    def val(c, s, gsc):
        mag = Fraction(float(O.E2M1_VALUES[int(c) & 7]))
        return (-mag if int(c) & 8 else mag) * grid[int(s)] * Fraction(float(gsc))
    for m in range(M):
        for n in range(N):
            e = sum(val(qx[m, k], sx[m, k // 16], gx) * val(qw[n, k], sw[n, k // 16], gw) for k in range(K))
            assert abs(y[m, n] - float(e)) <= 1e-13 * abs(float(e)) + 1e-300
