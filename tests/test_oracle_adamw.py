"""Pins of the oracle's AdamW step (adapter optimiser; "QLoRA: Fine-Tuning a
70B on One GPU", section "Paged Optimizers", and "Fine-Tuning Memory
Requirements: Full Training vs LoRA vs QLoRA", section "Where training memory
goes"): closed forms of the first step and of a constant gradient, the
moment recurrences against their unrolled sums, and torch.optim.AdamW's own
implementation in float64 over several steps with weight decay."""
import numpy as np
import pytest
import torch

from oracle.adamw import adamw_step


def _rand(seed, n=257):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(n), rng.standard_normal(n) * 1e-3,
            np.abs(rng.standard_normal(n)) * 1e-2, np.abs(rng.standard_normal(n)) * 1e-6)


def test_first_step_is_a_signed_unit_step():
    """From zero moments the bias-corrected moments are g and g^2, so the
    step is lr * g / (|g| + eps) after the decay."""
    p, g, _, _ = _rand(1)
    lr, wd, eps = 1e-3, 0.1, 1e-8
    p1, m1, v1 = adamw_step(p, g, np.zeros_like(p), np.zeros_like(p), 1, lr, 0.9, 0.999, eps, wd)
    assert np.allclose(m1, 0.1 * g, rtol=1e-15, atol=0)
    assert np.allclose(v1, 0.001 * g * g, rtol=1e-14, atol=0)
    ref = p * (1 - lr * wd) - lr * g / (np.abs(g) + eps)
    assert np.allclose(p1, ref, rtol=1e-13, atol=1e-16)


def test_constant_gradient_keeps_the_corrected_moments_exact():
    """With the same gradient every step, m_t = (1 - b1^t) g and
    v_t = (1 - b2^t) g^2, so every bias-corrected step is again
    lr * g / (|g| + eps)."""
    p, g, _, _ = _rand(2)
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    lr, b1, b2, eps = 2e-3, 0.8, 0.95, 1e-10
    for t in range(1, 8):
        pn, m, v = adamw_step(p, g, m, v, t, lr, b1, b2, eps, 0.0)
        assert np.allclose(m, (1 - b1 ** t) * g, rtol=1e-13, atol=0)
        assert np.allclose(v, (1 - b2 ** t) * g * g, rtol=1e-13, atol=0)
        assert np.allclose(pn, p - lr * g / (np.abs(g) + eps), rtol=1e-12, atol=1e-15)
        p = pn


def test_moments_are_the_weighted_gradient_sums():
    """m_t = (1 - b1) sum_i b1^(t-i) g_i and v_t likewise with g_i^2, from
    zero moments."""
    rng = np.random.default_rng(3)
    gs = [rng.standard_normal(31) for _ in range(6)]
    p = rng.standard_normal(31)
    m = np.zeros(31)
    v = np.zeros(31)
    b1, b2 = 0.9, 0.99
    for t, g in enumerate(gs, start=1):
        p, m, v = adamw_step(p, g, m, v, t, 1e-3, b1, b2, 1e-8, 0.01)
    T = len(gs)
    m_ref = sum((1 - b1) * b1 ** (T - i) * g for i, g in enumerate(gs, start=1))
    v_ref = sum((1 - b2) * b2 ** (T - i) * g * g for i, g in enumerate(gs, start=1))
    assert np.allclose(m, m_ref, rtol=1e-13, atol=1e-16)
    assert np.allclose(v, v_ref, rtol=1e-13, atol=1e-16)


def test_zero_learning_rate_moves_only_the_moments():
    p, g, m, v = _rand(4)
    p1, m1, v1 = adamw_step(p, g, m, v, 3, 0.0, 0.9, 0.999, 1e-8, 0.5)
    assert np.array_equal(p1, p)
    assert not np.array_equal(m1, m) and not np.array_equal(v1, v)


@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_matches_torch_adamw_in_float64(wd):
    """torch.optim.AdamW (decoupled weight decay) on float64 tensors, five
    steps with changing gradients and nonzero starting moments excluded (torch
    starts from zero)."""
    rng = np.random.default_rng(5)
    p0 = rng.standard_normal((16, 40))
    grads = [rng.standard_normal((16, 40)) * 1e-2 for _ in range(5)]
    lr, b1, b2, eps = 3e-3, 0.9, 0.999, 1e-8
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    for t, g in enumerate(grads, start=1):
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
        p, m, v = adamw_step(p, g, m, v, t, lr, b1, b2, eps, wd)
        st = opt.state[tp]
        assert np.allclose(st["exp_avg"].numpy(), m, rtol=1e-12, atol=1e-18)
        assert np.allclose(st["exp_avg_sq"].numpy(), v, rtol=1e-12, atol=1e-20)
        assert np.allclose(tp.detach().numpy(), p, rtol=1e-12, atol=1e-15)


def test_step_number_starts_at_one():
    p, g, m, v = _rand(6)
    with pytest.raises(ValueError):
        adamw_step(p, g, m, v, 0, 1e-3)
