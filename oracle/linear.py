"""Float64 forward and backward of the frozen-NF4 linear with a LoRA side path.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The layer (PyTorch ``Linear`` convention, W is [N, K] = out x in):

    Y  = X . W'^T + s . (X . A^T) . B^T,      s = alpha / r

with W' the dequantised frozen weight, A [r, K] the LoRA down-projection and
B [N, r] the up-projection (the low-rank adapter pair beside the frozen base of
the xingyuzhitong guide, section "LoRA: freeze the base, train small adapters";
alpha and r are the ``lora_alpha`` and ``r`` knobs of the PEFT configuration in
"QLoRA: Fine-Tuning a 70B on One GPU", section "Practical Implementation").

W is frozen: the gradient flows through it into the adapters (inquiringlines
note, mechanism paragraph), so the backward yields dX, dA and dB and no dW:

    G  = dY . B                (gradient reaching X . A^T, scaled by s below)
    dX = dY . W' + s . G . A
    dA = s . G^T . X
    dB = s . dY^T . (X . A^T)

Every product is a numpy float64 matmul of the given values; nothing is
blocked, fused or reordered.
"""
import numpy as np


def lora_scale(alpha: float, r: int) -> float:
    return float(alpha) / float(r)


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _dropout_scale(x, drop):
    """keep / (1 - p) per element of x (all ones without dropout).  drop is
    None or (p, seed, row0): row0 is the first row's index in the full X, for
    a comparison on sampled rows."""
    if drop is None or drop[0] == 0.0:
        return None
    from .dropout import keep_mask
    p, seed = drop[0], drop[1]
    row0 = drop[2] if len(drop) > 2 else 0
    rows = np.asarray(row0).reshape(-1)
    M, K = x.shape
    if rows.size == 1:
        keep = keep_mask(int(rows[0]) + M, K, p, seed)[int(rows[0]):]
    else:   # explicit row indices
        keep = keep_mask(int(rows.max()) + 1, K, p, seed)[rows]
    return keep.astype(np.float64) / (1.0 - float(p))


def linear_fwd(wd, x, a, b, alpha, drop=None):
    """Returns (Y, XA) in float64.  wd: [N, K] dequantised weight; x: [M, K];
    a: [r, K]; b: [N, r].  With drop = (p, seed[, rows]) the down-projection
    sees the dropped input D(X) (see dropout.py); the frozen path sees X."""
    wd, x, a, b = _f64(wd), _f64(x), _f64(a), _f64(b)
    s = lora_scale(alpha, a.shape[0])
    d = _dropout_scale(x, drop)
    xa = (x if d is None else x * d) @ a.T
    y = x @ wd.T + s * (xa @ b.T)
    return y, xa


def adapter_grads(x, a, b, alpha, dy, drop=None):
    """(dA, dB) in float64, the adapter gradients alone (they reduce over all
    tokens, so they need every row of X and dY; the frozen W plays no part):
        dA = s . (dY . B)^T . D(X),   dB = s . dY^T . (D(X) . A^T)
    with D(X) = X without dropout."""
    x, a, b, dy = _f64(x), _f64(a), _f64(b), _f64(dy)
    s = lora_scale(alpha, a.shape[0])
    d = _dropout_scale(x, drop)
    xd = x if d is None else x * d
    g = dy @ b
    da = s * (g.T @ xd)
    db = s * (dy.T @ (xd @ a.T))
    return da, db


def linear_bwd(wd, x, a, b, alpha, dy, drop=None):
    """Returns (dX, dA, dB) in float64.  With dropout, dA uses D(X), dB the
    dropped forward's X . A^T, and the LoRA share of dX passes back through
    the same keep / (1 - p) factors."""
    wd, x, a, b, dy = _f64(wd), _f64(x), _f64(a), _f64(b), _f64(dy)
    s = lora_scale(alpha, a.shape[0])
    d = _dropout_scale(x, drop)
    g = dy @ b
    lora_dx = s * (g @ a)
    dx = dy @ wd + (lora_dx if d is None else lora_dx * d)
    da, db = adapter_grads(x, a, b, alpha, dy, drop)
    return dx, da, db


def merge_adapter(wd, a, b, alpha):
    """The merged weight of an adapted layer in float64: W' + s . B . A, whose
    plain product X . W_merged^T is the adapted forward ("Fine-Tuning Memory
    Requirements: Full Training vs LoRA vs QLoRA", section "LoRA: freeze the
    base, train small adapters": the adapters are a low-rank update of W)."""
    wd, a, b = _f64(wd), _f64(a), _f64(b)
    return wd + lora_scale(alpha, a.shape[0]) * (b @ a)
