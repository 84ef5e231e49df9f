"""Pins of the oracle's AdamW step with 8-bit statistics (CPU only).

The training arguments of the addaly.com lesson "Fitting a fine-tune in 16 GB"
name an 8-bit paged AdamW, and "QLoRA: Fine-Tuning a 70B on One GPU", section
"Paged Optimizers", places its states in paged memory; the pages give no
8-bit format.  The oracle's reading (blockwise 8-bit codes with a float32
scale per 256 statistics: m signed with max|m| / 127, sqrt(v) unsigned with
max sqrt(v) / 255) is pinned here by exact round trips, the half-step error
bound checked in rational arithmetic, hand-worked codes including ties, the
zero state, reductions to the float32 AdamW update (first step, betas of 0)
and agreement with the float64 AdamW over several steps.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle.adamw import (STATE_BLOCK, adamw8_step, adamw_step, dequantize_state,
                          quantize_state)

F32 = np.float32


def test_levels_round_trip_exactly():
    """Values k * 2^-e, with +-127 (signed) or 255 (unsigned) in every block,
    have scale 2^-e exactly, codes k and dequantise to themselves."""
    rng = np.random.default_rng(1)
    for signed, top in ((True, 127), (False, 255)):
        for e in (3, 10, 20):
            n = 3 * STATE_BLOCK + 77
            k = rng.integers(-top if signed else 0, top + 1, size=n)
            k[::STATE_BLOCK] = top                      # every block reaches the top code
            x = (k * 2.0 ** -e).astype(F32)
            codes, scales = quantize_state(x, signed)
            assert np.all(scales == F32(2.0 ** -e))
            assert np.array_equal(codes.astype(np.int64), k)
            assert np.array_equal(dequantize_state(codes, scales), x)


def test_error_is_at_most_half_a_step():
    """|code * scale - x| <= scale * (1/2 + 2^-17) + half an ulp of the
    product, checked exactly (the division x / scale rounds once, so the
    code is within 1/2 + 127 * 2^-24 steps of x / scale)."""
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(5 * STATE_BLOCK) * np.exp(rng.uniform(-8, 2, 5 * STATE_BLOCK))
         ).astype(F32)
    for signed, data in ((True, x), (False, np.abs(x))):
        codes, scales = quantize_state(data, signed)
        back = dequantize_state(codes, scales)
        for i in range(0, data.size, 7):
            s = Fraction(float(scales[i // STATE_BLOCK]))
            err = abs(Fraction(float(back[i])) - Fraction(float(data[i])))
            ulp = Fraction(float(np.spacing(np.abs(back[i])))) / 2
            assert err <= s * (Fraction(1, 2) + Fraction(1, 2 ** 17)) + ulp, (signed, i)


def test_hand_worked_codes_with_ties():
    """One unsigned block with max 255/256: scale = (255/256) / 255 = 1/256
    exactly, so u = j/256 has code j, and the ties 127.5/256 and 126.5/256
    go to the even codes 128 and 126.  One signed block with max 127/64:
    scale 1/64, and -2.5/64, 3.5/64 go to -2 and 4."""
    u = np.zeros(STATE_BLOCK, dtype=F32)
    u[:5] = np.array([255, 127.5, 126.5, 3, 0.25]) / 256
    codes, scales = quantize_state(u, signed=False)
    assert scales[0] == F32(1 / 256)
    assert codes[:5].tolist() == [255, 128, 126, 3, 0]
    m = np.zeros(STATE_BLOCK, dtype=F32)
    m[:4] = np.array([127, -2.5, 3.5, -127]) / 64
    codes, scales = quantize_state(m, signed=True)
    assert scales[0] == F32(1 / 64)
    assert codes[:4].tolist() == [127, -2, 4, -127]


def test_zero_blocks_and_ragged_tail():
    x = np.zeros(2 * STATE_BLOCK + 10, dtype=F32)
    x[STATE_BLOCK + 3] = -0.5                # block 1 only
    x[-1] = 0.25                             # the 10-element tail block
    codes, scales = quantize_state(x, signed=True)
    assert scales.tolist() == [0.0, F32(0.5) / F32(127), F32(0.25) / F32(127)]
    assert not codes[:STATE_BLOCK].any()
    assert codes[STATE_BLOCK + 3] == -127 and codes[-1] == 127


def _zero_state(n):
    return (np.zeros(n, np.int8), np.zeros((n + 255) // 256, F32),
            np.zeros(n, np.uint8), np.zeros((n + 255) // 256, F32))


def test_zero_gradient_from_zero_state_only_decays():
    rng = np.random.default_rng(3)
    p = rng.standard_normal(700).astype(F32)
    mq, ms, vq, vs = _zero_state(700)
    p1, mq1, ms1, vq1, vs1 = adamw8_step(p, np.zeros(700, F32), mq, ms, vq, vs, 1, 1e-3,
                                         wd=0.1)
    assert np.array_equal(p1, p * F32(1.0 - 1e-3 * 0.1))
    assert not mq1.any() and not vq1.any() and not ms1.any() and not vs1.any()


def test_first_step_is_the_float32_adamw_step():
    """From the zero state nothing has been quantised yet, so the first step
    is AdamW's first step in float32: within float32 rounding of the
    float64 oracle's, and the new codes quantise m = (1 - b1) g and
    sqrt(v) = sqrt((1 - b2) g^2) in float32."""
    rng = np.random.default_rng(4)
    n = 1000
    p = (rng.standard_normal(n) * 0.02).astype(F32)
    g = (rng.standard_normal(n) * 1e-3).astype(F32)
    mq, ms, vq, vs = _zero_state(n)
    p1, mq1, ms1, vq1, vs1 = adamw8_step(p, g, mq, ms, vq, vs, 1, 2e-4, 0.9, 0.999, 1e-8, 0.01)
    p64, m64, v64 = adamw_step(p.astype(np.float64), g.astype(np.float64), np.zeros(n),
                               np.zeros(n), 1, 2e-4, 0.9, 0.999, 1e-8, 0.01)
    # a handful of float32 roundings: within a few float32 ulps of the two
    # terms, the decayed weight and the step of size lr / (1 - b1) = 2e-3
    bound = 4 * (np.spacing(np.abs(p)) + np.spacing(F32(2e-3)))
    assert np.all(np.abs(p1 - p64) <= bound)
    m1 = F32(0.1) * g
    assert np.array_equal((mq1, ms1)[0], quantize_state(m1, True)[0])
    u1 = np.sqrt(F32(0.999) * np.zeros(n, F32) + F32(1.0 - 0.999) * (g * g))
    assert np.array_equal(vq1, quantize_state(u1, False)[0])


def test_zero_betas_ignore_the_stored_state():
    """With b1 = b2 = 0 the moments are g and g^2 whatever was stored, so a
    step from a random state equals the step from the zero state bit for
    bit, and the update is lr g / (|g| + eps) after the decay."""
    rng = np.random.default_rng(5)
    n = 600
    p = rng.standard_normal(n).astype(F32)
    g = rng.standard_normal(n).astype(F32)
    rand_state = (rng.integers(-127, 128, n).astype(np.int8), np.full(3, 0.3, F32),
                  rng.integers(0, 256, n).astype(np.uint8), np.full(3, 0.7, F32))
    a = adamw8_step(p, g, *rand_state, 7, 1e-3, 0.0, 0.0, 1e-8, 0.05)
    b = adamw8_step(p, g, *_zero_state(n), 7, 1e-3, 0.0, 0.0, 1e-8, 0.05)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    want = p * F32(1.0 - 1e-3 * 0.05) - F32(1e-3) * (g / (np.abs(g) + F32(1e-8)))
    assert np.array_equal(a[0], want)


@pytest.mark.parametrize("seed", [6, 7])
def test_tracks_float64_adamw_over_ten_steps(seed):
    """Ten steps on fresh N(0, 1e-6) gradients: every statistic is rebuilt
    within half a step of its block's largest value, and the parameters stay
    within 0.1 lr t of the float64 AdamW's (the step of one element is at
    most about 7.3 lr with these betas)."""
    rng = np.random.default_rng(seed)
    n = 4 * STATE_BLOCK + 33
    lr = 2e-4
    p8 = (rng.standard_normal(n) * 0.02).astype(F32)
    state = _zero_state(n)
    p64, m64, v64 = p8.astype(np.float64), np.zeros(n), np.zeros(n)
    for t in range(1, 11):
        g = (rng.standard_normal(n) * 1e-3).astype(F32)
        p8, *state = adamw8_step(p8, g, *state, t, lr, 0.9, 0.999, 1e-8, 0.01)
        p64, m64, v64 = adamw_step(p64, g.astype(np.float64), m64, v64, t, lr, 0.9, 0.999,
                                   1e-8, 0.01)
        assert np.max(np.abs(p8 - p64)) <= 0.1 * lr * t, t
        m_hat = dequantize_state(state[0], state[1])
        u_hat = dequantize_state(state[2], state[3])
        sm = np.repeat(state[1], STATE_BLOCK)[:n].astype(np.float64)
        su = np.repeat(state[3], STATE_BLOCK)[:n].astype(np.float64)
        # against the float64 moments: half a step plus the drift of the
        # earlier steps' rounding, a few per cent of the block's largest
        assert np.all(np.abs(m_hat - m64) <= 0.5 * sm + 0.05 * 127 * sm)
        assert np.all(np.abs(u_hat - np.sqrt(v64)) <= 0.5 * su + 0.05 * 255 * su)


def test_state_bytes_per_parameter():
    """The 8-bit state costs 2 + 8/256 bytes per parameter against 8 for two
    float32 statistics."""
    n = 41_943_040          # every adapter of the 8B model at r = 16
    mq, ms, vq, vs = _zero_state(n)
    total = mq.nbytes + ms.nbytes + vq.nbytes + vs.nbytes
    assert total == n * 2 + 2 * 4 * (n // 256)
    assert total / n == pytest.approx(2.03125)
