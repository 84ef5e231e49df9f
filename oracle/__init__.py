"""CPU oracle for the QLoRA frozen-NF4 linear with a LoRA side path.

TEST INFRASTRUCTURE ONLY: the parity reference for the GPU library.  Only the
tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may
import it.  It shares no code with the GPU library and never calls it.

Four parts:
  * ``nf4_oracle.c`` (wrapped here): codebook, blockwise absmax quantisation,
    double quantisation of the constants, dequantisation, bf16 rounding.
  * ``linear.py``: the forward and backward of
        Y = X . W'^T + (alpha / r) . (X . A^T) . B^T
    written as their float64 definitions with numpy matmul as the only step,
    optionally with dropout on the LoRA input, and the merged weight
    W' + (alpha / r) . B . A.
  * ``dropout.py``: the keep mask of that dropout (Philox4x32-10).
  * ``adamw.py``: the AdamW step on the adapters.

Pins (tests/test_oracle_*.py) tie every function here to something other than
itself: scipy's normal quantile, printed figures from the pages, closed forms,
invariants, hand-built special cases and finite differences.
"""
import ctypes
import os

import numpy as np

from . import build as _build
from .linear import (linear_fwd, linear_bwd, adapter_grads, lora_scale,  # noqa: F401
                     merge_adapter)
from . import dropout  # noqa: F401
from . import adamw  # noqa: F401

NF4_BLOCK = 64
DQ_BLOCK = 256

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_phi_inv.restype = ctypes.c_double
        lib.oracle_phi_inv.argtypes = [ctypes.c_double]
        lib.oracle_codebook.argtypes = [P]
        lib.oracle_quantize.argtypes = [P, I64, P, P, P]
        lib.oracle_double_quant.argtypes = [P, I64, P, P, P, P]
        lib.oracle_dequant_absmax.argtypes = [P, P, ctypes.c_float, I64, P]
        lib.oracle_dequant.argtypes = [P, P, I64, P, P]
        lib.oracle_to_bf16.argtypes = [P, I64, P]
        lib.oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def threads() -> int:
    """OpenMP threads the C oracle runs with."""
    return int(_load().oracle_threads())


def phi_inv(p: float) -> float:
    return float(_load().oracle_phi_inv(float(p)))


QUANT_TYPES = ("nf4", "int4")


def int4_codebook() -> np.ndarray:
    """The uniform 4-bit table the NF4 type is set against ("QLoRA: Fine-Tuning
    a 70B on One GPU", section "NF4 Quantization: Beyond Standard INT4": 16
    integer levels at uniform intervals).  Reading: the sixteen 4-bit
    two's-complement integers k = -8 .. 7 over the block absmax scaled to 7,
    i.e. level k / 7 (computed in double, rounded once to float32).  Level -8/7
    lies below -1, so for |x| <= 1 it is never the nearest: 15 levels are used,
    with an exact zero (code 8) and the ends -1 (code 1) and +1 (code 15)."""
    return (np.arange(-8, 8, dtype=np.float64) / 7.0).astype(np.float32)


def codebook(kind: str = "nf4") -> np.ndarray:
    """The 16 levels of a 4-bit type, ascending (code k holds level k)."""
    if kind == "int4":
        return int4_codebook()
    if kind != "nf4":
        raise ValueError("unknown 4-bit type %r" % (kind,))
    out = np.zeros(16, dtype=np.float32)
    _load().oracle_codebook(_ptr(out))
    return out


def num_blocks(n: int) -> int:
    return (n + NF4_BLOCK - 1) // NF4_BLOCK


def num_dq_blocks(n: int) -> int:
    return (num_blocks(n) + DQ_BLOCK - 1) // DQ_BLOCK


def quantize(w: np.ndarray, kind: str = "nf4", dq: bool = True) -> dict:
    """Blockwise 4-bit quantisation (the NF4 table, or the INT4 table it is set
    against), followed by double quantisation of the constants unless dq is
    False (the double-quant switch of the pages' configuration,
    "Practical Implementation" section).

    Returns codes (packed, uint8[ceil(n/2)]) and the exact first-level absmax
    (float32[nb]), which without double quantisation is the stored constant;
    with it, the stored constants absmax_q (int8[nb]), absmax_scale
    (float32[nd]) and absmax_mean (float32 scalar)."""
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    n = w.size
    if n == 0:
        raise ValueError("empty tensor")
    nb = num_blocks(n)
    cb = codebook(kind)
    codes = np.zeros((n + 1) // 2, dtype=np.uint8)
    absmax = np.zeros(nb, dtype=np.float32)
    lib = _load()
    lib.oracle_quantize(_ptr(w), n, _ptr(cb), _ptr(codes), _ptr(absmax))
    out = {"n": n, "codes": codes, "absmax": absmax, "kind": kind, "dq": dq}
    if dq:
        q, scale, mean = double_quant(absmax)
        out.update({"absmax_q": q, "absmax_scale": scale, "absmax_mean": mean})
    return out


def double_quant(absmax: np.ndarray):
    absmax = np.ascontiguousarray(absmax, dtype=np.float32)
    nb = absmax.size
    nd = (nb + DQ_BLOCK - 1) // DQ_BLOCK
    q = np.zeros(nb, dtype=np.int8)
    scale = np.zeros(nd, dtype=np.float32)
    mean = np.zeros(1, dtype=np.float32)
    pow2 = 1
    while pow2 < nb:
        pow2 <<= 1
    scratch = np.zeros(pow2, dtype=np.float64)
    _load().oracle_double_quant(_ptr(absmax), nb, _ptr(q), _ptr(scale), _ptr(mean),
                                _ptr(scratch))
    return q, scale, np.float32(mean[0])


def dequant_absmax(absmax_q: np.ndarray, absmax_scale: np.ndarray, absmax_mean) -> np.ndarray:
    q = np.ascontiguousarray(absmax_q, dtype=np.int8)
    s = np.ascontiguousarray(absmax_scale, dtype=np.float32)
    out = np.zeros(q.size, dtype=np.float32)
    _load().oracle_dequant_absmax(_ptr(q), _ptr(s), ctypes.c_float(float(absmax_mean)),
                                  q.size, _ptr(out))
    return out


def block_constants(qt: dict) -> np.ndarray:
    """The constant each 64-block dequantises with: the reconstruction from
    the 8-bit state, or the stored float32 absmax without double quantisation."""
    if qt.get("dq", True):
        return dequant_absmax(qt["absmax_q"], qt["absmax_scale"], qt["absmax_mean"])
    return np.ascontiguousarray(qt["absmax"], dtype=np.float32)


def dequantize(qt: dict) -> np.ndarray:
    """float32 dequantised weights (flat), from the stored state only."""
    ahat = block_constants(qt)
    n = qt["n"]
    out = np.zeros(n, dtype=np.float32)
    cb = codebook(qt.get("kind", "nf4"))
    _load().oracle_dequant(_ptr(np.ascontiguousarray(qt["codes"])), _ptr(ahat), n,
                           _ptr(cb), _ptr(out))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    out = np.zeros(x.size, dtype=np.uint16)
    _load().oracle_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def unpack_codes(codes: np.ndarray, n: int) -> np.ndarray:
    """uint8 code per element from the packed buffer (element 2i = low nibble)."""
    c = np.empty(2 * codes.size, dtype=np.uint8)
    c[0::2] = codes & 15
    c[1::2] = codes >> 4
    return c[:n]


def storage_bits(n: int, double_quant: bool = True) -> int:
    """Bits the quantised state of an n-weight tensor occupies: 4-bit codes plus
    either float32 absmax per 64 weights, or (double quantisation) an int8 per
    64 weights, a float32 scale per 256 constants and one float32 mean."""
    nb = num_blocks(n)
    code_bits = 8 * ((n + 1) // 2)
    if not double_quant:
        return code_bits + 32 * nb
    nd = (nb + DQ_BLOCK - 1) // DQ_BLOCK
    return code_bits + 8 * nb + 32 * nd + 32
