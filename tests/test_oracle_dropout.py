"""Pins of the oracle's LoRA dropout (the ``lora_dropout`` knob of the LoRA
configuration in "QLoRA: Fine-Tuning a 70B on One GPU", section "Practical
Implementation"): the Philox4x32-10 generator against the known-answer
vectors published with it, the keep rate, and the backward's agreement with
the forward through the same mask (adjoint identity, finite differences)."""
import numpy as np
import pytest

import oracle
from oracle import dropout


# Known-answer vectors of Philox4x32 with 10 rounds, as published with the
# generator (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy
# as 1, 2, 3", SC 2011, and the known-answer file of their Random123
# library): counter, key -> output words.
KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,out", KAT)
def test_philox_known_answers(ctr, key, out):
    got = dropout.philox4x32_10(np.array([ctr], dtype=np.uint32), key)
    assert [int(v) for v in got[0]] == list(out)


def test_mask_layout_is_row_major_element_index():
    a = dropout.keep_mask(7, 36, 0.3, 99)
    b = dropout.keep_mask(1, 7 * 36, 0.3, 99).reshape(7, 36)
    assert np.array_equal(a, b)
    # element e takes word e mod 4 of counter e div 4
    words = dropout.philox4x32_10(np.array([[2, 0, 0, 0]], dtype=np.uint32), (99, 0))[0]
    thr = dropout.threshold(0.3)
    assert [bool(w >= thr) for w in words] == list(a.reshape(-1)[8:12])


@pytest.mark.parametrize("p", [0.05, 0.5])
def test_keep_rate(p):
    m = dropout.keep_mask(1024, 1024, p, 2024)
    n = m.size
    sd = np.sqrt(n * p * (1 - p))
    assert abs((n - m.sum()) - n * p) < 6 * sd
    assert not np.array_equal(m, dropout.keep_mask(1024, 1024, p, 2025))


def _case(seed, M=9, N=11, K=64, r=4):
    rng = np.random.default_rng(seed)
    wd = rng.standard_normal((N, K)) * 0.1
    x = rng.standard_normal((M, K))
    a = rng.standard_normal((r, K)) * 0.2
    b = rng.standard_normal((N, r)) * 0.2
    dy = rng.standard_normal((M, N))
    return wd, x, a, b, dy


def test_zero_probability_is_no_dropout():
    wd, x, a, b, dy = _case(1)
    y0, xa0 = oracle.linear_fwd(wd, x, a, b, 8.0)
    y1, xa1 = oracle.linear_fwd(wd, x, a, b, 8.0, drop=(0.0, 5))
    assert np.array_equal(y0, y1) and np.array_equal(xa0, xa1)
    for u, v in zip(oracle.linear_bwd(wd, x, a, b, 8.0, dy),
                    oracle.linear_bwd(wd, x, a, b, 8.0, dy, drop=(0.0, 5))):
        assert np.array_equal(u, v)


def test_dropped_elements_do_not_reach_the_adapter():
    wd, x, a, b, dy = _case(2)
    drop = (0.5, 77)
    keep = dropout.keep_mask(*x.shape, 0.5, 77)
    x2 = x.copy()
    x2[~keep] += 123.0        # only dropped elements change
    _, xa1 = oracle.linear_fwd(wd, x, a, b, 8.0, drop=drop)
    _, xa2 = oracle.linear_fwd(wd, x2, a, b, 8.0, drop=drop)
    assert np.allclose(xa1, xa2, rtol=0, atol=1e-12)
    _, xa3 = oracle.linear_fwd(wd, x, a, b, 8.0, drop=(0.5, 78))
    assert not np.allclose(xa1, xa3)


def test_adjoint_identity_with_dropout():
    """Y is linear in X for a fixed mask, so <dY, Y(X)> = <dX, X> exactly
    up to float64 rounding."""
    wd, x, a, b, dy = _case(3)
    drop = (0.3, 11)
    y, _ = oracle.linear_fwd(wd, x, a, b, 8.0, drop=drop)
    dx, _, _ = oracle.linear_bwd(wd, x, a, b, 8.0, dy, drop=drop)
    lhs, rhs = float(np.sum(dy * y)), float(np.sum(dx * x))
    assert abs(lhs - rhs) <= 1e-10 * max(abs(lhs), 1.0)


def test_adapter_gradients_by_finite_differences_with_dropout():
    wd, x, a, b, dy = _case(4)
    drop = (0.3, 12)
    _, da, db = oracle.linear_bwd(wd, x, a, b, 8.0, dy, drop=drop)

    def loss(a_, b_):
        return float(np.sum(dy * oracle.linear_fwd(wd, x, a_, b_, 8.0, drop=drop)[0]))

    h = 1e-6
    for (i, j) in [(0, 0), (1, 5), (3, 63)]:
        ap, am = a.copy(), a.copy()
        ap[i, j] += h
        am[i, j] -= h
        assert abs((loss(ap, b) - loss(am, b)) / (2 * h) - da[i, j]) < 1e-6
    for (i, j) in [(0, 0), (7, 2), (10, 3)]:
        bp, bm = b.copy(), b.copy()
        bp[i, j] += h
        bm[i, j] -= h
        assert abs((loss(a, bp) - loss(a, bm)) / (2 * h) - db[i, j]) < 1e-6


def test_sampled_rows_match_full():
    wd, x, a, b, dy = _case(5, M=20)
    drop = (0.25, 31)
    rows = np.array([2, 7, 19])
    y, xa = oracle.linear_fwd(wd, x, a, b, 8.0, drop=drop)
    ys, xas = oracle.linear_fwd(wd, x[rows], a, b, 8.0, drop=(0.25, 31, rows))
    assert np.allclose(ys, y[rows], rtol=0, atol=1e-12)
    assert np.allclose(xas, xa[rows], rtol=0, atol=1e-12)
