"""Pins for three details of the double quantisation that ordinary random
data cannot tell apart (CPU only).

"QLoRA: Fine-Tuning a 70B on One GPU", section "Double Quantization", fixes
that the block constants are themselves quantised and that the weights are
rebuilt from the quantised constants for compute.  The readings of how are:

  * the mean of the constants is one float64 binary tree of adjacent pairs
    (padded with +0.0 to a power of two), divided by the count, rounded once
    to float32;
  * a constant is rebuilt as one correctly rounded fused multiply-add,
    q * S + mean;
  * a weight dequantises with that rebuilt constant, not the exact absmax.

Each test below is built so that the plausible alternative (a left-to-right
or exact sum, two roundings, the exact absmax) gives a different answer, and
the expected value is worked out by hand or in exact rational arithmetic.
"""
from fractions import Fraction

import numpy as np

import oracle


# ------------------------------------------------------------ exact rounding
def round_to_f32(x: Fraction) -> np.float32:
    """The float32 nearest to the rational x, ties to the even significand
    (IEEE round to nearest even), by exact comparison with the neighbours of
    a candidate; x must lie inside float32's normal range."""
    c = np.float32(float(x))
    best = c
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d_best = abs(Fraction(float(best)) - x)
        d_cand = abs(Fraction(float(cand)) - x)
        if d_cand < d_best or (d_cand == d_best and
                               (int(cand.view(np.uint32)) & 1) == 0 and cand != best):
            best = cand
    return best


def test_round_to_f32_helper():
    one = Fraction(1)
    ulp = Fraction(1, 2 ** 23)
    assert round_to_f32(one + ulp / 2) == np.float32(1.0)                  # tie -> even
    assert round_to_f32(one + 3 * ulp / 2) == np.float32(1.0 + 2.0 ** -22)  # tie -> even
    assert round_to_f32(one + ulp / 2 + Fraction(1, 2 ** 60)) == np.float32(1.0 + 2.0 ** -23)
    assert round_to_f32(Fraction(1, 3)) == np.float32(1.0 / 3.0)


# ------------------------------------------------------- (a) fused rebuild
def test_constant_rebuild_is_one_fused_rounding():
    """q * S + mean rounded once.  Random (q, S, mean) where rounding q * S
    first changes the result: the oracle must give the exactly rounded value
    in every case, which the two-rounding form misses in the chosen ones."""
    rng = np.random.default_rng(11)
    n = 20000
    q = rng.integers(-127, 128, size=n).astype(np.int8)
    S = (rng.uniform(0.5, 1.0, size=n) * 2.0 ** rng.integers(-12, -4, size=n)).astype(np.float32)
    mu = rng.uniform(0.01, 0.2, size=n).astype(np.float32)
    two_step = (q.astype(np.float32) * S).astype(np.float32) + mu   # float32 ops: two roundings
    differs = []
    for i in range(n):
        exact = round_to_f32(Fraction(int(q[i])) * Fraction(float(S[i])) + Fraction(float(mu[i])))
        if exact != two_step[i]:
            differs.append((i, exact))
        if len(differs) == 64:
            break
    assert len(differs) == 64, "too few cases where the two forms differ"
    idx = np.array([i for i, _ in differs])
    # one DQ block per case (scale index b // 256), so lay each case out at
    # position 256 k
    qq = np.zeros(256 * len(idx), dtype=np.int8)
    qq[::256] = q[idx]
    for k, i in enumerate(idx):
        got = oracle.dequant_absmax(qq[256 * k:256 * (k + 1)], S[i:i + 1], mu[i])[0]
        assert got == differs[k][1], (k, got, differs[k][1], two_step[i])
        assert got != two_step[i]


# ------------------------------------------------------------ (b) tree order
def test_mean_follows_the_adjacent_pair_tree():
    """Constants c = [4, 2^-22, 2^-51, 2^-51].

    The tree adds (4 + 2^-22) + (2^-51 + 2^-51).  In float64 4 + 2^-22 is
    exact, 2^-51 + 2^-51 = 2^-50 is exact, and 4 + 2^-22 + 2^-50 is exact too
    (2^-50 is one unit in the last place at 4), so the tree sum is
    T = 4 + 2^-22 + 2^-50 and T / 4 = 1 + 2^-24 + 2^-52: above the float32
    midpoint 1 + 2^-24, so the mean is 1 + 2^-23.

    Left to right: (4 + 2^-22) + 2^-51 is half a unit in the last place; the
    tie goes to the even neighbour, 4 + 2^-22, and so does the next 2^-51.
    That sum is 4 + 2^-22, whose quarter 1 + 2^-24 is a float32 tie that goes
    to 1.0.  So a left-to-right sum gives the mean 1.0."""
    c = np.array([4.0, 2.0 ** -22, 2.0 ** -51, 2.0 ** -51], dtype=np.float32)
    _, _, mu = oracle.double_quant(c)
    assert mu == np.float32(1.0 + 2.0 ** -23)
    seq = 0.0
    for v in c.astype(np.float64):
        seq += v
    assert np.float32(seq / 4) == np.float32(1.0)   # the alternative really differs


def test_mean_tree_differs_from_the_exact_mean():
    """Constants c = [4, 2^-51, 2^-22, 2^-51].

    The tree adds (4 + 2^-51) + (2^-22 + 2^-51).  4 + 2^-51 is a tie at half
    a unit in the last place and goes to the even 4; 2^-22 + 2^-51 is exact;
    4 + (2^-22 + 2^-51) is again a tie and goes to the even 4 + 2^-22.  The
    quarter, 1 + 2^-24, is a float32 tie that goes to 1.0.

    The exact mean, (4 + 2^-22 + 2^-50) / 4, lies above that midpoint and
    rounds to 1 + 2^-23: an exact (or compensated) sum gives another mean."""
    c = np.array([4.0, 2.0 ** -51, 2.0 ** -22, 2.0 ** -51], dtype=np.float32)
    _, _, mu = oracle.double_quant(c)
    assert mu == np.float32(1.0)
    exact = sum(Fraction(float(v)) for v in c) / 4
    assert round_to_f32(exact) == np.float32(1.0 + 2.0 ** -23)


def test_mean_tree_pads_with_zeros_and_divides_by_the_count():
    """Five constants c = [5, 5 * 2^-24, 2^-51, 2^-51, 0] pad to eight with
    zeros: ((c0 + c1) + (c2 + c3)) + ((c4 + 0) + (0 + 0)).

    c0 + c1 = 5 + 5 * 2^-24 is exact in float64 and its last bit (2^-50) is
    0; c2 + c3 = 2^-50; their sum 5 + 5 * 2^-24 + 2^-50 is exact (53 bits
    from 2^2 to 2^-50).  Divided by the count 5 it is 1 + 2^-24 + 2^-50 / 5
    rounded to float64, above the float32 midpoint 1 + 2^-24, so the mean is
    1 + 2^-23.  Left to right each 2^-51 is a tie against 5 + 5 * 2^-24 that
    goes to that even value; (5 + 5 * 2^-24) / 5 = 1 + 2^-24 exactly, a
    float32 tie that goes to 1.0.  Dividing by the padded length 8 would give
    about 0.625."""
    c = np.array([5.0, 5.0 * 2.0 ** -24, 2.0 ** -51, 2.0 ** -51, 0.0], dtype=np.float32)
    assert float(c[1]) == 5.0 * 2.0 ** -24
    _, _, mu = oracle.double_quant(c)
    assert mu == np.float32(1.0 + 2.0 ** -23)
    seq = 0.0
    for v in c.astype(np.float64):
        seq += v
    assert np.float32(seq / 5) == np.float32(1.0)


# ---------------------------------------------- (c) dequantise with a-hat
def test_dequantise_uses_the_rebuilt_constant():
    """256 blocks (one second-level block) with absmax a_0 = 1 + 127/128,
    a_1 = 1/128, a_2 = 1 + 2^-9, a_3 = 1 - 2^-9 and a_b = 1 otherwise; every
    block holds each level four times, times its absmax.

    By hand: the deviations from 1 sum to zero and are multiples of 2^-9, so
    the float64 sum is exact and the mean is exactly 1.  The largest |d| is
    127/128, so S = (127/128)/127 = 1/128 exactly.  q_0 = 127, q_1 = -127,
    q_2 = rint(1/4) = 0, q_3 = rint(-1/4) = 0, every other q is 0.  The
    rebuilt constants are 1 + 127/128, 1/128, then 1 for every other block:
    blocks 2 and 3 rebuild to 1, not to their absmax.  Their weights
    therefore dequantise to the levels themselves, where the exact absmax
    would give level * (1 +- 2^-9)."""
    cb = oracle.codebook()
    a = np.ones(256, dtype=np.float64)
    a[0], a[1], a[2], a[3] = 1 + 127 / 128, 1 / 128, 1 + 2.0 ** -9, 1 - 2.0 ** -9
    idx = np.tile(np.arange(16), 4)
    w = np.stack([(cb[idx].astype(np.float64) * a_b).astype(np.float32) for a_b in a])
    qt = oracle.quantize(w)
    codes = oracle.unpack_codes(qt["codes"], w.size).reshape(256, 64)
    assert np.all(codes == idx)
    assert qt["absmax_mean"] == np.float32(1.0)
    assert qt["absmax_scale"][0] == np.float32(1 / 128)
    assert qt["absmax_q"][:5].tolist() == [127, -127, 0, 0, 0]
    d = oracle.dequantize(qt).reshape(256, 64)
    for b in (2, 3):
        assert np.array_equal(d[b], cb[idx]), b            # level * 1
        assert not np.array_equal(d[b], w[b])               # not level * absmax
    assert np.array_equal(d[1], (cb[idx] / np.float32(128)).astype(np.float32))
    assert np.array_equal(d[0], (cb[idx] * np.float32(1 + 127 / 128)).astype(np.float32))
    assert np.array_equal(d[4:], np.tile(cb[idx], (252, 1)))
