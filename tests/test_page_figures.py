"""The pages' printed figures, reproduced from the oracle's storage accounting
and the workload shapes (CPU only).  Fixture: tests/golden/page_figures.json."""
import json
import os

import pytest

import oracle
import workloads

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def _close(key, got):
    g = GOLD[key]
    if "abs_tol" in g:
        assert abs(got - g["value"]) <= g["abs_tol"], (key, got, g)
    elif "rel_tol" in g:
        assert abs(got - g["value"]) <= g["rel_tol"] * g["value"], (key, got, g)
    else:
        assert got == g["value"], (key, got, g)


# a large tensor, so per-tensor terms vanish; a multiple of 64*256
N_BIG = 4096 * 14336


def _saving_bits_per_param(n):
    return (oracle.storage_bits(n, double_quant=False) - oracle.storage_bits(n, True)) / n


def test_dq_saving_bits():
    s = _saving_bits_per_param(N_BIG)
    assert s == pytest.approx(0.5 - (8 / 64 + 32 / (64 * 256)), abs=1e-6)
    _close("dq_saving_bits_per_param", s)
    _close("dq_saving_bits_per_param_rounded", s)


def test_dq_saving_gb_at_65b():
    g = GOLD["dq_saving_gb_at_65b"]
    _close("dq_saving_gb_at_65b", g["params"] * _saving_bits_per_param(N_BIG) / 8 / 1e9)


def test_constants_memory_reduction():
    n = N_BIG
    const_plain = oracle.storage_bits(n, False) - 4 * n
    const_dq = oracle.storage_bits(n, True) - 4 * n
    _close("constants_memory_reduction", 1 - const_dq / const_plain)


def test_bits_per_param_near_4_127():
    total = sum(oracle.storage_bits(r * c) for _, _, r, c in workloads.llama8b_weight_set())
    params = sum(r * c for _, _, r, c in workloads.llama8b_weight_set())
    assert total / params == pytest.approx(4.127, abs=5e-4)
    # 1024 x 1024: 4 + 8/64 + 32 * 64 / 2^20 + 32 / 2^20
    assert oracle.storage_bits(1024 * 1024) / 2 ** 20 == pytest.approx(4.126984, abs=1e-6)


def test_adapter_counts_pin_llama8b_shapes():
    per_layer = sum(k + n for _, k, n in workloads.LLAMA8B_LINEARS)
    _close("llama31_8b_adapter_dims_per_layer", per_layer)
    _close("llama31_8b_adapter_params_r16", per_layer * 16 * 32)
    _close("llama31_8b_adapter_params_r64", per_layer * 64 * 32)


def test_adapter_count_pins_70b_shapes():
    per_layer = sum(k + n for _, k, n in workloads.LLAMA70B_LINEARS)
    _close("llama_70b_adapter_params_r16", per_layer * 16 * 80)


def test_param_total_pins_full_weight_set():
    params = sum(r * c for _, _, r, c in workloads.llama8b_weight_set())
    assert params == 8_029_995_008
    _close("llama31_8b_params", params)
