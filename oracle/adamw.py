"""AdamW step on the LoRA adapters, for the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: AdamW keeps two states per trainable parameter, a running
mean of the gradient and a running mean of its square ("QLoRA: Fine-Tuning a
70B on One GPU", section "Paged Optimizers"; "Fine-Tuning Memory
Requirements: Full Training vs LoRA vs QLoRA", section "Where training memory
goes"), and the adapter training state is float32 weight, float32 gradient
and 8 bytes of Adam statistics per parameter (same page, section "LoRA:
freeze the base, train small adapters").  The update itself is not printed.
Reading (also in the design notes): Adam (Kingma and Ba, ICLR 2015) with
decoupled weight decay (Loshchilov and Hutter, ICLR 2019), in the order
torch.optim.AdamW applies it, at step t = 1, 2, ...:

    p <- p * (1 - lr * wd)
    m <- b1 * m + (1 - b1) * g
    v <- b2 * v + (1 - b2) * g^2
    p <- p - lr / (1 - b1^t) * m / (sqrt(v / (1 - b2^t)) + eps)

Everything here is float64.
"""
import numpy as np


def adamw_step(p, g, m, v, t, lr, b1=0.9, b2=0.999, eps=1e-8, wd=0.0):
    """One AdamW step.  Returns new (p, m, v) as float64 arrays; the inputs are
    not modified.  t is the 1-based step number of this update."""
    if t < 1:
        raise ValueError("the step number starts at 1")
    p = np.asarray(p, dtype=np.float64) * (1.0 - lr * wd)
    g = np.asarray(g, dtype=np.float64)
    m = b1 * np.asarray(m, dtype=np.float64) + (1.0 - b1) * g
    v = b2 * np.asarray(v, dtype=np.float64) + (1.0 - b2) * g * g
    m_hat = m / (1.0 - b1 ** t)
    v_hat = v / (1.0 - b2 ** t)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v
