"""Helpers shared by the GPU parity tests: device transfer, the oracle side of
a comparison, and the float tolerance."""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

DEV = "cuda:0"


def say(msg):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print("[gpu-case] %s" % msg, flush=True)


def tol(ref: np.ndarray) -> float:
    """Acceptance bound for a bf16 output against its float64 reference:
    max|delta| <= 1e-2 * max|ref| + 1e-3."""
    return 1e-2 * float(np.max(np.abs(ref))) + 1e-3


def assert_close(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    bound = tol(ref) if ref.size else 0.0
    assert err <= bound, "%s: max|delta| %.4g > bound %.4g (max|ref| %.4g)" % (
        name, err, bound, float(np.max(np.abs(ref))))
    return err, bound


def to_dev(x):
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x))
    return x.contiguous().to(DEV)


def host(t):
    return t.detach().to("cpu")


def bf16_np(t) -> np.ndarray:
    """float64 values of a bf16 tensor."""
    return host(t).to(torch.float32).numpy().astype(np.float64)


def oracle_weight(w_np: np.ndarray):
    """Oracle quantisation and float32 dequantised weight [N, K]."""
    qt = oracle.quantize(w_np)
    wd = oracle.dequantize(qt).reshape(w_np.shape)
    return qt, wd


def compare_quant_state(q, ws, qt, n):
    """Bit-exact comparison of the GPU quantised state with the oracle's."""
    nb = qt["absmax"].size
    codes = host(q.codes).numpy()
    assert np.array_equal(codes, qt["codes"]), "codes differ at %s" % (
        np.nonzero(codes != qt["codes"])[0][:8],)
    absmax = host(ws[: nb * 4].view(torch.float32)).numpy()
    assert np.array_equal(absmax.view(np.uint32), qt["absmax"].view(np.uint32)), "absmax differs"
    assert host(q.absmax_mean).numpy().view(np.uint32)[0] == np.float32(qt["absmax_mean"]).view(np.uint32), \
        "mean differs: %r vs %r" % (host(q.absmax_mean).item(), qt["absmax_mean"])
    assert np.array_equal(host(q.absmax_scale).numpy().view(np.uint32),
                          qt["absmax_scale"].view(np.uint32)), "second-level scale differs"
    assert np.array_equal(host(q.absmax_q).numpy(), qt["absmax_q"]), "int8 constants differ"
