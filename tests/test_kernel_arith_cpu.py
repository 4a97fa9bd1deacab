"""Arithmetic identities the kernels rely on, proven on the CPU by exhaustive
enumeration (no GPU, no oracle): each replaces an IEEE operation of the
quantizer's rule by a cheaper sequence that must give the same fp32 result for
every input the kernels can see.

fl32(a / 7): the INT4 scale is fp16(fl32(amax / 7)). The kernels form the
quotient as q = RN(a z), z = RN(1/7), r = RN(a - 7 q) (one fma: the residual is
exact), q' = RN(q + r z) (one fma). The emulation below computes each step's
exact value in float64 (a z and 7 q are products of 24-bit and at most 24-bit
significands, 48 bits; a - 7 q is exact by cancellation) and rounds once to
fp32, as the fma does; the last sum q + r z can need more than 53 bits, so a
float64 result that lands exactly on an fp32 rounding midpoint is re-done in
exact rationals. Every significand of a binade is enumerated; the sequence
scales exactly by powers of two wherever its intermediates stay normal, so the
subnormals, the lowest binades and the highest one stand for all of fp32 here
(a slower sweep over the lowest 40 and highest 55 binades also found no
difference).
"""
from fractions import Fraction

import numpy as np
import pytest

Z = np.float32(1.0) / np.float32(7.0)


def div7_sequence(a32):
    a = a32.astype(np.float64)
    z = np.float64(Z)
    q0 = (a * z).astype(np.float32)
    r = (a - q0.astype(np.float64) * 7.0).astype(np.float32)
    s = q0.astype(np.float64) + r.astype(np.float64) * z
    q1 = s.astype(np.float32)
    up = np.nextafter(q1, np.float32(np.inf))
    dn = np.nextafter(q1, np.float32(-np.inf))
    on_mid = (s == (q1.astype(np.float64) + up.astype(np.float64)) / 2) | \
             (s == (q1.astype(np.float64) + dn.astype(np.float64)) / 2)
    for i in np.nonzero(on_mid)[0]:        # exact rational re-rounding of the rare midpoints
        exact = Fraction(float(q0[i])) + Fraction(float(r[i])) * Fraction(float(z))
        cands = [q1[i], up[i], dn[i]]
        q1[i] = min(cands, key=lambda c: (abs(Fraction(float(c)) - exact), int(np.float32(c).view(np.uint32)) & 1))
    return q1


def test_reciprocal_constant():
    assert int(Z.view(np.uint32)) == 0x3E124925


@pytest.mark.parametrize("exp_field", [0, 1, 2, 3, 4, 5, 127, 254])
def test_div7_sequence_equals_ieee_division(exp_field):
    """Every fp32 significand of the binade (exp_field 0: the subnormals)."""
    a = (np.arange(1 << 23, dtype=np.uint32) | np.uint32(exp_field << 23)).view(np.float32)
    ieee = (a.astype(np.float64) / 7.0).astype(np.float32)   # A / 7 is never an fp32 midpoint
    got = div7_sequence(a)
    bad = np.nonzero(got.view(np.uint32) != ieee.view(np.uint32))[0]
    assert bad.size == 0, [(float(a[i]), float(got[i]), float(ieee[i])) for i in bad[:5]]


def test_div7_sequence_zero():
    assert div7_sequence(np.array([0.0], np.float32))[0] == 0.0
