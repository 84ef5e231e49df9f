"""Pins for the oracle's blockwise quantisation, double quantisation and
dequantisation (CPU only).

Each pin comes from outside the oracle's own code: hand-built blocks whose
codes follow from the definition (levels map to themselves, exact midpoints
go to the lower level), an equivalent threshold-count characterisation of
"nearest level", exact rational arithmetic for the mean, hand-worked
round-half-to-even cases for the int8 constants, and the round trip.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _cb():
    return oracle.codebook()


def test_levels_round_trip_exactly():
    """Blocks made of every level times a power of two (each block holds -1 and
    +1, so absmax is that power of two): codes are the level indices, every
    constant reconstructs exactly and dequantisation returns the input bits."""
    cb = _cb()
    blocks = []
    for e in range(-8, 3):
        idx = np.tile(np.arange(16), 4)
        blocks.append(cb[idx] * np.float32(2.0 ** e))
    # All blocks share one absmax so the per-tensor mean is exact and every
    # second-level scale is 0; use one exponent per tensor.
    for e, blk in zip(range(-8, 3), blocks):
        w = np.concatenate([blk] * 300)           # 300 blocks -> 2 DQ blocks
        qt = oracle.quantize(w)
        codes = oracle.unpack_codes(qt["codes"], w.size)
        assert np.array_equal(codes, np.tile(np.arange(16), 4 * 300))
        assert np.all(qt["absmax"] == np.float32(2.0 ** e))
        assert qt["absmax_mean"] == np.float32(2.0 ** e)
        assert np.all(qt["absmax_scale"] == 0) and np.all(qt["absmax_q"] == 0)
        back = oracle.dequantize(qt)
        assert np.array_equal(back.view(np.uint32), w.view(np.uint32))


def _single_block(values, absmax=1.0):
    """One 64-block whose absmax is `absmax` (element 63 carries it)."""
    blk = np.zeros(64, dtype=np.float32)
    blk[:len(values)] = values
    blk[63] = absmax
    return blk


def test_exact_midpoints_go_to_lower_level():
    cb = _cb().astype(np.float64)
    vals, expect = [], []
    for j in range(15):
        m = (cb[j] + cb[j + 1]) / 2.0            # exact in double
        f = np.float32(m)
        if float(f) == m:                        # representable midpoint: a tie
            vals += [f, np.nextafter(f, np.float32(2)), np.nextafter(f, np.float32(-2))]
            expect += [j, j + 1, j]
        else:                                    # the floats on either side
            lo = f if float(f) < m else np.nextafter(f, np.float32(-2))
            hi = np.nextafter(lo, np.float32(2))
            vals += [lo, hi]
            expect += [j, j + 1]
    assert len(vals) <= 63
    qt = oracle.quantize(_single_block(vals))
    codes = oracle.unpack_codes(qt["codes"], 64)
    assert codes[:len(vals)].tolist() == expect
    assert codes[63] == 15


def test_threshold_count_equals_nearest_level():
    """'Nearest level, ties to the lower index' equals 'number of midpoints
    strictly below x' -- an independent way to state the same rule."""
    rng = np.random.default_rng(1)
    cb = _cb().astype(np.float64)
    mids = (cb[:-1] + cb[1:]) / 2.0
    x = rng.uniform(-1, 1, size=64 * 2000).astype(np.float32)
    # plus the float neighbourhood (+-8 ulp) of every midpoint
    extra = []
    for m in mids:
        f = np.float32(m)
        for k in range(-8, 9):
            g = f
            step = np.float32(2) if k > 0 else np.float32(-2)
            for _ in range(abs(k)):
                g = np.nextafter(g, step)
            extra.append(g)
    x[:len(extra)] = extra
    x = x.reshape(-1, 64)
    x[:, 63] = 1.0                                # absmax 1 so w/absmax == w
    qt = oracle.quantize(x)
    codes = oracle.unpack_codes(qt["codes"], x.size).reshape(x.shape)
    count = (x.astype(np.float64)[..., None] > mids).sum(-1)
    assert np.array_equal(codes, count)


def test_zero_block_negative_zero_and_nibble_order():
    cb = _cb()
    w = np.zeros(64 * 3 + 5, dtype=np.float32)   # ragged: 5 elements in last block
    w[64:128] = -0.0
    blk = _single_block([cb[3] * 0.5, cb[12] * 0.5, -0.0, 0.0], absmax=0.5)
    w[128:192] = blk
    w[192:] = [cb[1], cb[14], cb[0], cb[15], cb[9]]
    qt = oracle.quantize(w)
    assert qt["codes"].size == (w.size + 1) // 2
    codes = oracle.unpack_codes(qt["codes"], w.size)
    assert np.all(codes[:128] == 7)
    assert qt["absmax"][0] == 0 and qt["absmax"][1] == 0
    # element 2i in the low nibble of byte i
    assert qt["codes"][64] == (3 | (12 << 4))
    assert codes[130] == 7 and codes[131] == 7
    assert codes[192:].tolist() == [1, 14, 0, 15, 9]
    assert qt["codes"][-1] >> 4 == 0, "odd length: last high nibble stays 0"


def test_absmax_is_block_max_abs():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal(64 * 100 + 17) * 0.02).astype(np.float32)
    qt = oracle.quantize(w)
    pad = np.concatenate([w, np.zeros(64 - 17, np.float32)]).reshape(-1, 64)
    assert np.array_equal(qt["absmax"], np.abs(pad).max(1))


def test_mean_is_exact_mean_rounded():
    """With float inputs of similar magnitude the double sum is exact, so the
    mean must be the exact rational mean rounded once to float32."""
    rng = np.random.default_rng(3)
    for nb in (1, 7, 256, 1000, 4099):
        a = np.abs(rng.standard_normal(nb).astype(np.float32)) * np.float32(0.05) + np.float32(1e-3)
        q, s, mu = oracle.double_quant(a)
        exact = sum(Fraction(float(v)) for v in a) / nb
        f = np.float32(float(exact))
        # float(Fraction) is correctly rounded to double; one more rounding to
        # float32 can only differ if the double sits on a float32 tie.
        assert mu == f


def test_int8_constants_round_half_even():
    """Hand-built constants: mean exactly 1, block max deviation 127/128 so the
    scale is exactly 1/128, and deviations at k + 1/2 steps."""
    d_steps = [127, -127, 2.5, -2.5, 3.5, -3.5, 0.5, -0.5, 1.5, -1.5, 126.5, -126.5, 7, -7]
    expect = [127, -127, 2, -2, 4, -4, 0, 0, 2, -2, 126, -126, 7, -7]
    a = np.ones(256, dtype=np.float32)
    a[:len(d_steps)] = 1.0 + np.array(d_steps, dtype=np.float64) / 128.0
    q, s, mu = oracle.double_quant(a)
    assert mu == np.float32(1.0)
    assert s.shape == (1,) and s[0] == np.float32(1.0 / 128.0)
    assert q[:len(expect)].tolist() == expect
    assert np.all(q[len(expect):] == 0)
    ahat = oracle.dequant_absmax(q, s, mu)
    assert np.array_equal(ahat[:len(expect)], (1.0 + np.array(expect) / 128.0).astype(np.float32))


def test_constant_block_and_ragged_dq_tail():
    a = np.full(256 + 40, 0.25, dtype=np.float32)
    a[256:] = 0.5                                 # second DQ block: 40 constants
    q, s, mu = oracle.double_quant(a)
    assert s.shape == (2,)
    exact_mu = np.float32((256 * 0.25 + 40 * 0.5) / 296)
    assert mu == exact_mu
    ahat = oracle.dequant_absmax(q, s, mu)
    # every constant reconstructs within half a step of its own DQ block
    for j, (lo, hi) in enumerate([(0, 256), (256, 296)]):
        assert np.all(np.abs(ahat[lo:hi] - a[lo:hi]) <= s[j] * 0.5 * (1 + 2 ** -16) + 1e-12)
    # all-equal block after centring: scale 0, q 0, ahat == mean
    q2, s2, mu2 = oracle.double_quant(np.full(300, 0.125, np.float32))
    assert np.all(s2 == 0) and np.all(q2 == 0) and mu2 == np.float32(0.125)
    assert np.all(oracle.dequant_absmax(q2, s2, mu2) == np.float32(0.125))


def test_reconstruction_error_bound_random():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((512, 1024)) * 0.02).astype(np.float32)
    qt = oracle.quantize(w)
    ahat = oracle.dequant_absmax(qt["absmax_q"], qt["absmax_scale"], qt["absmax_mean"])
    S = np.repeat(qt["absmax_scale"], 256)[:ahat.size]
    err = np.abs(ahat.astype(np.float64) - qt["absmax"])
    ulp = np.spacing(np.abs(qt["absmax"])).astype(np.float64)
    assert np.all(err <= S * (0.5 + 2 ** -16) + 2 * ulp)
    # and the 4-bit reconstruction of each weight is within half the widest
    # level gap (0.3066, between -1 and the next level) of its block absmax
    wd = oracle.dequantize(qt).reshape(w.shape)
    absmax = np.repeat(qt["absmax"], 64).reshape(w.shape)
    ahat_e = np.repeat(ahat, 64).reshape(w.shape)
    assert np.all(np.abs(wd - w) <= 0.16 * absmax + np.abs(ahat_e - absmax) + 1e-7)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(100000).astype(np.float32)
    # exact ties: low 16 bits == 0x8000 with both parities of bit 16
    u = rng.integers(0, 2 ** 31, size=2000, dtype=np.uint64).astype(np.uint32)
    u = (u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    u &= np.uint32(0x7F7FFFFF)                     # stay finite
    x = np.concatenate([x, u.view(np.float32)])
    mine = oracle.to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
