"""Pins of the oracle's 4-bit type and constant variants: the INT4 table the
NF4 type is set against ("QLoRA: Fine-Tuning a 70B on One GPU", section "NF4
Quantization: Beyond Standard INT4"), and quantisation without double
quantisation (the double-quant switch, "Practical Implementation" section).
Each check ties the oracle to a closed form or to a claim the pages make,
not to a retyped copy of its own code."""
import numpy as np
import pytest

import oracle


def test_int4_table_is_the_integer_grid_over_seven():
    cb = oracle.codebook("int4")
    assert cb.dtype == np.float32 and cb.shape == (16,)
    k = np.arange(-8, 8)
    # every level is the float32 nearest to k / 7 ...
    assert np.all(np.abs(cb.astype(np.float64) * 7 - k) <= 7 * 2.0 ** -24)
    # ... so the ends and the zero are exact, and the spacing is uniform
    assert cb[1] == -1.0 and cb[15] == 1.0
    assert cb[8].view(np.uint32) == 0
    d = np.diff(cb.astype(np.float64))
    assert np.all(np.abs(d - 1 / 7) < 1e-7)


def _int4_code_closed_form(x):
    # nearest integer to 7x with halves going down, shifted to the code range
    y = x.astype(np.float64) * 7.0          # exact: 24 + 3 bits
    return (np.ceil(y - 0.5) + 8).astype(np.int64)


def test_int4_codes_are_rounding_to_sevenths():
    """Brute-force nearest level (the oracle) against arithmetic rounding of
    7 x, away from the midpoints, where the float32 levels' rounding could
    decide either way."""
    rng = np.random.default_rng(41)
    x = rng.uniform(-1, 1, 1 << 18).astype(np.float32)
    frac = np.abs(x.astype(np.float64) * 7 - np.floor(x.astype(np.float64) * 7) - 0.5)
    x = x[frac > 1e-5]
    x[:4] = [-1.0, 1.0, 0.0, -0.0]
    w = np.ones(64 * ((x.size + 63) // 64), dtype=np.float32)
    w[: x.size] = x
    w[63::64] = 1.0   # absmax 1 in every block, so the quantised value is x itself
    keep = np.ones(w.size, dtype=bool)
    keep[63::64] = False
    keep[x.size:] = False
    qt = oracle.quantize(w, kind="int4", dq=False)
    codes = oracle.unpack_codes(qt["codes"], w.size)
    assert np.array_equal(codes[keep], _int4_code_closed_form(w[keep]))
    assert codes.min() >= 1   # level -8/7 is never the nearest


@pytest.mark.parametrize("kind", ["nf4", "int4"])
def test_no_double_quant_round_trip_is_exact(kind):
    """Blocks made of table levels times a power of two, each block holding a
    level of magnitude 1: the absmax is the power of two, every weight divides
    back to its level and the stored float32 constant rebuilds it exactly."""
    cb = oracle.codebook(kind)
    rng = np.random.default_rng(5)
    blocks = []
    for b in range(40):
        lv = cb[rng.integers(1, 16, 64)]
        lv[rng.integers(0, 64)] = 1.0 if b % 2 else -1.0
        blocks.append(lv * np.float32(2.0 ** int(rng.integers(-20, 10))))
    w = np.concatenate(blocks).astype(np.float32)
    qt = oracle.quantize(w, kind=kind, dq=False)
    assert "absmax_q" not in qt
    back = oracle.dequantize(qt)
    assert np.array_equal(back.view(np.uint32), w.view(np.uint32))


def test_double_quant_changes_only_the_constants():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal(64 * 300) * 0.02).astype(np.float32)
    a = oracle.quantize(w, dq=True)
    b = oracle.quantize(w, dq=False)
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(a["absmax"], b["absmax"])
    # without double quantisation the constant is the absmax itself
    assert np.array_equal(oracle.block_constants(b), b["absmax"])


@pytest.mark.parametrize("dq", [True, False])
def test_nf4_error_below_int4_on_normal_weights(dq):
    """The pages' claim that the normal-quantile table keeps normally
    distributed weights more accurately than uniform INT4: mean squared
    reconstruction error on N(0, 0.02) weights, same blocks and constants."""
    rng = np.random.default_rng(17)
    w = (rng.standard_normal(1 << 20) * 0.02).astype(np.float32)
    err = {}
    for kind in ("nf4", "int4"):
        back = oracle.dequantize(oracle.quantize(w, kind=kind, dq=dq))
        err[kind] = float(np.mean((back.astype(np.float64) - w) ** 2))
    assert err["nf4"] < err["int4"]
    # and by a clear margin, not by rounding noise
    assert err["nf4"] < 0.9 * err["int4"]
