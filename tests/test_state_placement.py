"""The optimiser-statistics placement policy (host logic, CPU only): under an
HBM budget the largest tensors' statistics stay on the device, the device
share never exceeds the budget, and no tensor left in host memory would have
fit in what the budget has left."""
import numpy as np
import pytest

import bit_quantized_lora_quant_amd as q


def _check(sizes, budget):
    host = q.plan_state_placement(sizes, budget)
    dev = sum(s for s, h in zip(sizes, host) if not h)
    assert dev <= budget
    spare = budget - dev
    assert all(s > spare for s, h in zip(sizes, host) if h)
    return host, dev


def test_state_bytes():
    assert q.adamw8_state_bytes(256) == 2 * 256 + 8
    assert q.adamw8_state_bytes(257) == 2 * 257 + 16
    assert q.adamw8_state_bytes(1) == 2 + 8


@pytest.mark.parametrize("seed", range(5))
def test_budget_invariants(seed):
    rng = np.random.default_rng(seed)
    sizes = [int(s) for s in rng.integers(1, 10 ** 7, size=int(rng.integers(1, 60)))]
    for frac in (0.0, 0.1, 0.5, 0.9, 1.0, 2.0):
        _check(sizes, int(sum(sizes) * frac))


def test_largest_first_and_extremes():
    sizes = [10, 50, 20, 40]
    host, dev = _check(sizes, 60)
    assert host == [False, False, True, True]      # 50 first, then 10 fits the 10 left
    assert q.plan_state_placement(sizes, 0) == [True] * 4
    assert q.plan_state_placement(sizes, 10 ** 9) == [False] * 4
    assert q.plan_state_placement([], 100) == []


def test_8b_adapters_half_budget():
    """All 448 adapters of the 8B model at r = 16 (the bench's AdamW leg) with
    half of their 8-bit statistics' bytes as the budget: about half go to
    host memory."""
    numels = []
    for _ in range(32):
        for K, N in ((4096, 4096), (4096, 1024), (4096, 1024), (4096, 4096),
                     (4096, 14336), (4096, 14336), (14336, 4096)):
            numels += [16 * K, N * 16]
    sizes = [q.adamw8_state_bytes(n) for n in numels]
    host, dev = _check(sizes, sum(sizes) // 2)
    assert len(numels) == 448
    assert 0.49 * sum(sizes) <= dev <= 0.5 * sum(sizes)
