"""Pins for the oracle's float64 forward and backward (CPU only).

The forward is tied to special cases with known answers (one-hot rows pick a
column of W', a zero adapter leaves the base product, a zero base leaves the
rank-1 closed form) and to torch's float64 linear; the backward is tied to the
forward by central finite differences of L = <dY, Y> and by the adjoint
identity, so a wrong sign, scale, transpose or operand fails.
"""
import numpy as np
import pytest
import torch

import oracle


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


def test_one_hot_rows_pick_weight_columns():
    rng = np.random.default_rng(10)
    N, K, r = 24, 64, 4
    wd = _rand(rng, N, K)
    x = np.zeros((K, K))
    x[np.arange(K), np.arange(K)] = 1.0
    a = _rand(rng, r, K)
    b = np.zeros((N, r))
    y, xa = oracle.linear_fwd(wd, x, a, b, alpha=8.0)
    assert np.array_equal(y, wd.T)           # row k of Y is column k of W'
    assert np.array_equal(xa, a.T)


def test_zero_adapter_is_torch_linear():
    rng = np.random.default_rng(11)
    N, K, M, r = 40, 96, 7, 8
    wd, x, a = _rand(rng, N, K), _rand(rng, M, K), _rand(rng, r, K)
    y, _ = oracle.linear_fwd(wd, x, a, np.zeros((N, r)), alpha=16.0)
    ref = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(wd)).numpy()
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-12)


def test_zero_base_rank_one_closed_form():
    """W' = 0, r = 1, X = e_k: Y[n] = (alpha / 1) * A[0, k] * B[n, 0]."""
    rng = np.random.default_rng(12)
    N, K = 16, 64
    a = _rand(rng, 1, K)
    b = _rand(rng, N, 1)
    k = 37
    x = np.zeros((1, K))
    x[0, k] = 1.0
    y, _ = oracle.linear_fwd(np.zeros((N, K)), x, a, b, alpha=3.0)
    assert np.allclose(y[0], 3.0 * a[0, k] * b[:, 0], rtol=1e-15, atol=0)


def test_lora_scale_is_alpha_over_r():
    rng = np.random.default_rng(13)
    N, K, M, r = 8, 64, 3, 4
    x, a, b = _rand(rng, M, K), _rand(rng, r, K), _rand(rng, N, r)
    wd = np.zeros((N, K))
    y1, _ = oracle.linear_fwd(wd, x, a, b, alpha=4.0)      # s = 1
    y2, _ = oracle.linear_fwd(wd, x, a, b, alpha=8.0)      # s = 2
    assert np.allclose(y2, 2.0 * y1, rtol=1e-14)
    # with W' = 0 and s = 1 the layer is two chained torch float64 linears
    t = torch.nn.functional.linear
    ref = t(t(torch.from_numpy(x), torch.from_numpy(a)), torch.from_numpy(b)).numpy()
    assert np.allclose(y1, ref, rtol=1e-13, atol=1e-13)


def _loss(wd, x, a, b, alpha, dy):
    y, _ = oracle.linear_fwd(wd, x, a, b, alpha)
    return float(np.sum(y * dy))


@pytest.mark.parametrize("alpha", [16.0, 0.5])
def test_backward_central_differences(alpha):
    rng = np.random.default_rng(14)
    N, K, M, r = 6, 5, 4, 3
    wd, x, a, b = _rand(rng, N, K), _rand(rng, M, K), _rand(rng, r, K), _rand(rng, N, r)
    dy = _rand(rng, M, N)
    dx, da, db = oracle.linear_bwd(wd, x, a, b, alpha, dy)
    h = 1e-5
    for name, t, g in (("X", x, dx), ("A", a, da), ("B", b, db)):
        num = np.zeros_like(t)
        for idx in np.ndindex(t.shape):
            old = t[idx]
            t[idx] = old + h
            lp = _loss(wd, x, a, b, alpha, dy)
            t[idx] = old - h
            lm = _loss(wd, x, a, b, alpha, dy)
            t[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        assert np.allclose(num, g, rtol=1e-7, atol=1e-8), name
    # the gradients-only entry is the same dA, dB, and needs no weight
    da2, db2 = oracle.adapter_grads(x, a, b, alpha, dy)
    assert np.array_equal(da2, da) and np.array_equal(db2, db)


def test_backward_adjoint_identity():
    rng = np.random.default_rng(15)
    N, K, M, r = 33, 64, 9, 2
    wd, x, a, b = _rand(rng, N, K), _rand(rng, M, K), _rand(rng, r, K), _rand(rng, N, r)
    dy = _rand(rng, M, N)
    y, _ = oracle.linear_fwd(wd, x, a, b, 4.0)
    dx, _, _ = oracle.linear_bwd(wd, x, a, b, 4.0, dy)
    # Y is linear in X, so <dY, Y(X)> == <dX, X>
    assert np.sum(dy * y) == pytest.approx(np.sum(dx * x), rel=1e-12)


def test_frozen_weight_has_no_gradient_output():
    rng = np.random.default_rng(16)
    out = oracle.linear_bwd(_rand(rng, 4, 64), _rand(rng, 2, 64), _rand(rng, 1, 64),
                            _rand(rng, 4, 1), 1.0, _rand(rng, 2, 4))
    assert len(out) == 3


def test_merged_weight_reproduces_the_adapted_layer():
    """The merged weight's plain product equals the adapted forward, and its
    input gradient the adapted dX (float64 rounding only)."""
    rng = np.random.default_rng(77)
    N, K, M, r = 24, 128, 9, 5
    wd = rng.standard_normal((N, K)) * 0.05
    a = rng.standard_normal((r, K)) * 0.1
    b = rng.standard_normal((N, r)) * 0.1
    x = rng.standard_normal((M, K))
    dy = rng.standard_normal((M, N))
    wm = oracle.merge_adapter(wd, a, b, 10.0)
    y, _ = oracle.linear_fwd(wd, x, a, b, 10.0)
    assert np.allclose(x @ wm.T, y, rtol=1e-12, atol=1e-12)
    dx, _, _ = oracle.linear_bwd(wd, x, a, b, 10.0, dy)
    assert np.allclose(dy @ wm, dx, rtol=1e-12, atol=1e-12)
    # rank one: the update is the outer product of B's and A's single vectors
    w1 = oracle.merge_adapter(wd, a[:1], b[:, :1], 3.0)
    assert np.allclose(w1 - wd, 3.0 * np.outer(b[:, 0], a[0]), rtol=1e-14, atol=1e-15)
