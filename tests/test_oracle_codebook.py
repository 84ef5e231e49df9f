"""Pins for the oracle's NF4 codebook (CPU only).

The codebook is tied to things outside the oracle: scipy's normal quantile
(Cephes ``ndtri``, a different algorithm from the oracle's bisection), the
equal-probability spacing the pages describe, and the exact zero and +-1 ends.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle

P_TAIL = 1.0 - 1.0 / 32.0


def phi(x):
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def test_shape_order_and_ends():
    cb = oracle.codebook()
    assert cb.dtype == np.float32 and cb.shape == (16,)
    assert np.all(np.diff(cb) > 0), "levels must be strictly increasing"
    assert cb[0] == np.float32(-1.0) and cb[15] == np.float32(1.0)
    assert cb.view(np.uint32)[7] == 0, "level 7 must be +0.0 exactly"
    assert int(np.sum(cb < 0)) == 7 and int(np.sum(cb > 0)) == 8


def test_matches_scipy_quantiles_bit_exact():
    """Each level is float32(Phi^-1(p) / Phi^-1(P)) with p evenly spaced on each
    half; scipy's ndtri gives the same float32 values."""
    z = scipy.special.ndtri(P_TAIL)
    exp = np.zeros(16, dtype=np.float32)
    for j in range(1, 8):
        exp[7 - j] = np.float32(-scipy.special.ndtri(0.5 + (P_TAIL - 0.5) * j / 7.0) / z)
    for j in range(1, 9):
        exp[7 + j] = np.float32(scipy.special.ndtri(0.5 + (P_TAIL - 0.5) * j / 8.0) / z)
    cb = oracle.codebook()
    assert np.array_equal(cb.view(np.uint32), exp.view(np.uint32)), (cb, exp)


@pytest.mark.parametrize("p", [0.5, 0.55, 0.7, 0.9, 0.96875, 0.999, 0.01])
def test_phi_inv_against_scipy(p):
    assert oracle.phi_inv(p) == pytest.approx(scipy.special.ndtri(p), rel=1e-13, abs=1e-15)


def test_equal_probability_share_per_side():
    """Neighbouring levels on each side are one equal probability step apart
    (the equal share of a zero-centred normal)."""
    cb = oracle.codebook().astype(np.float64)
    z = scipy.special.ndtri(P_TAIL)
    probs = np.array([phi(c * z) for c in cb])
    neg = np.diff(probs[:8])          # levels 0..7
    pos = np.diff(probs[7:])          # levels 7..15
    assert np.allclose(neg, (P_TAIL - 0.5) / 7.0, atol=1e-6)
    assert np.allclose(pos, (P_TAIL - 0.5) / 8.0, atol=1e-6)
    assert probs[15] == pytest.approx(P_TAIL, abs=1e-7)
