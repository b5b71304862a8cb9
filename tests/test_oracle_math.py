"""Pins of the oracle's exp and log: correctly rounded to fp32.

Page "(11) FusedNormalization", section 12 draws the log aspect ratio
uniformly between the logs of the ratio bounds and takes exp of it.  The
oracle's reading is the correctly rounded fp32 exp and log; these tests
check that against 60-digit decimal arithmetic (exact rounding) and, over
every reachable draw of the default ratio range, against numpy's float64 exp.
"""
from __future__ import annotations

import numpy as np
import pytest

import exact


def reachable_log_ratios(orc, rmin=0.3, rmax=3.3) -> np.ndarray:
    """Every log aspect ratio one draw can produce: lmin + u*(lmax - lmin),
    u = k 2^-24, each operation rounded to fp32 (numpy fp32 ops do not fuse)."""
    lmin = np.float32(orc.log_ratio(rmin))
    lmax = np.float32(orc.log_ratio(rmax))
    u = (np.arange(2**24, dtype=np.float64) * 2.0**-24).astype(np.float32)
    span = np.float32(lmax - lmin)
    return (lmin + (u * span).astype(np.float32)).astype(np.float32)


@pytest.mark.parametrize("r", [0.3, 3.3, 1.0, 0.5, 2.0, 1e-20, 1e20, 0.1, 10.0])
def test_log_ratio_correctly_rounded(orc, r):
    assert np.float32(orc.log_ratio(r)) == exact.ln_f32(np.float32(r))


def test_expf_correctly_rounded_sample(orc):
    L = reachable_log_ratios(orc)[::4099]
    grid = np.linspace(-46.0, 46.0, 1501).astype(np.float32)
    special = np.array([0.0, -0.0, 2.0**-30, -2.0**-30, 2.0**-24, -2.0**-25, 1e-7, -1e-7,
                        0.5, -0.5, 1.0, -1.0, np.log(2.0), -np.log(2.0)], np.float32)
    for x in np.concatenate([L, grid, special]):
        assert np.float32(orc.expf(float(x))) == exact.exp_f32(float(x)), x


def test_expf_exhaustive_reachable_matches_float64_exp(orc):
    """All 2^24 draws at ratio [0.3, 3.3]: RN32(expl) == RN32(exp in float64)."""
    L = reachable_log_ratios(orc)
    got = orc.expf_array(L)
    ref = np.exp(L.astype(np.float64)).astype(np.float32)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, (bad[:5], L[bad[:5]])
    # the draws span the log range end to end and stay inside it
    assert L.min() == np.float32(orc.log_ratio(0.3))
    assert L.max() <= np.float32(orc.log_ratio(3.3))
