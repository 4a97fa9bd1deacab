"""The shader-clock probe on the GPU: one value per workgroup, inside the
chip's clock range (MI355X: up to 2400 MHz), and consistent across
workgroups run at the same time."""
import numpy as np
import pytest

import bit_diffusion_transformer_act_amd as P

pytestmark = pytest.mark.gpu


def test_clock_probe_range():
    mhz = P.svdq_clock_probe(0, workgroups=256, ticks=100_000)
    assert mhz.shape == (256,)
    assert np.all(mhz > 100.0) and np.all(mhz < 3000.0), (mhz.min(), mhz.max())
    med = np.median(mhz)
    assert np.all(np.abs(mhz - med) < 0.25 * med), (mhz.min(), med, mhz.max())
    print(f"shader clock: median {med:.0f} MHz, range {mhz.min():.0f}..{mhz.max():.0f}")
