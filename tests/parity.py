"""Comparison rules shared by the GPU parity tests.

Two bars for every float output of a kernel against the oracle:

  - relative L2 over the compared values: 2e-3 for layer, GEMM and GEMV
    outputs (the layer's stated tolerance), 1e-3 for lora_act;
  - a bound on every element:
        |y - y_ref| <= ULPS * ulp(|y_ref|) + FLOOR * rms(y_ref)
    with ulp the spacing of the output's own 16-bit type at |y_ref| (fp16:
    2^(e - 10), 2^-24 below the normal range; bf16: 2^(e - 7)) and rms over
    the compared values. A correct kernel is off by its final rounding (half
    an ulp) plus fp32 summation error far below 1e-3 rms; a single wrong value
    (a dropped group, a wrong column block, a tile written to the wrong place)
    is off by a sizeable fraction of rms and fails here even when the global
    relative L2 stays under its bar.

Rows of full-size launches are sampled by `band_rows`: one random row from
every band of 64 rows (so every M-tile of every tile shape has a checked row),
plus the first and the last row, all columns.
"""
import numpy as np

Y_TOL = 2e-3
LORA_TOL = 1e-3
ULPS = 2
FLOOR = 1e-3


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def _kind(y):
    y = np.asarray(y)
    if y.dtype == np.float16:
        return "float16"
    if y.dtype == np.float32 and not (y.view(np.uint32) & 0xFFFF).any():
        return "bfloat16"
    return "float32"


def ulp(ref, kind):
    """Spacing of the 16-bit type `kind` at |ref| (float64 array)."""
    a = np.abs(np.asarray(ref, np.float64))
    mant, emin = {"float16": (10, -14), "bfloat16": (7, -126), "float32": (23, -126)}[kind]
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(ex.astype(np.int64) - 1, emin)
    return np.ldexp(1.0, e - mant)


def assert_close(y, y_ref, tol=Y_TOL, kind=None, ulps=ULPS, floor=FLOOR, what=""):
    """Both bars (see the module docstring); `kind` defaults to the type y
    holds (fp16 array, or float32 holding bf16 values). Returns the relative L2."""
    y = np.asarray(y)
    kind = kind or _kind(y)
    y64 = y.astype(np.float64)
    r64 = np.asarray(y_ref, np.float64)
    assert y64.shape == r64.shape, (y64.shape, r64.shape)
    assert np.isfinite(y64).all(), f"{what}: non-finite outputs"
    rel = rel_l2(y64, r64)
    assert rel <= tol, f"{what}: relative L2 {rel:.3e} > {tol:.1e}"
    rms = np.sqrt(np.mean(r64 ** 2)) if r64.size else 0.0
    bound = ulps * ulp(r64, kind) + floor * rms
    err = np.abs(y64 - r64)
    bad = err > bound
    if bad.any():
        idx = np.unravel_index(int(np.argmax(err - bound)), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements outside {ulps} ulp + {floor:g} rms; "
            f"worst at {tuple(int(i) for i in idx)}: {y64[idx]!r} vs {r64[idx]!r} (bound {bound[idx]:.3e})")
    return rel


def band_rows(M, band=64, seed=0, extra=()):
    """One random row from every band of `band` rows, plus rows 0 and M - 1
    and any `extra` rows below M, sorted and unique."""
    rng = np.random.default_rng(seed)
    starts = np.arange(0, M, band)
    picks = starts + rng.integers(0, band, starts.size)
    picks = np.minimum(picks, M - 1)
    ex = [e for e in extra if 0 <= e < M]
    return np.unique(np.concatenate([picks, [0, M - 1], np.asarray(ex, dtype=np.int64)])).astype(np.int64)
