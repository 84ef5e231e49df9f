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


def linear_fwd(wd, x, a, b, alpha):
    """Returns (Y, XA) in float64.  wd: [N, K] dequantised weight; x: [M, K];
    a: [r, K]; b: [N, r]."""
    wd, x, a, b = _f64(wd), _f64(x), _f64(a), _f64(b)
    s = lora_scale(alpha, a.shape[0])
    xa = x @ a.T
    y = x @ wd.T + s * (xa @ b.T)
    return y, xa


def linear_bwd(wd, x, a, b, alpha, dy):
    """Returns (dX, dA, dB) in float64."""
    wd, x, a, b, dy = _f64(wd), _f64(x), _f64(a), _f64(b), _f64(dy)
    s = lora_scale(alpha, a.shape[0])
    g = dy @ b
    dx = dy @ wd + s * (g @ a)
    da = s * (g.T @ x)
    db = s * (dy.T @ (x @ a.T))
    return dx, da, db
