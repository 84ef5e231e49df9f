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


# ------------------------------------------------------------ 8-bit state
# "paged_adamw_8bit" (the optimiser named in the training arguments of the
# addaly.com lesson "Fitting a fine-tune in 16 GB"; the paged optimiser
# states of "QLoRA: Fine-Tuning a 70B on One GPU", section "Paged
# Optimizers") keeps the two statistics in 8 bits.  The pages give no format.
# Reading: the blockwise 8-bit scheme this method already applies to its
# block constants ("Double Quantization": constants quantised to INT8 with a
# float32 scale per block), on blocks of 256 statistics:
#   m   signed:   scale = max|m| / 127,   code = clamp(rint(m / scale), -127, 127)
#   v   as u = sqrt(v) >= 0, unsigned:
#                 scale = max u / 255,    code = clamp(rint(u / scale), 0, 255)
# (code 0 and scale 0 for an all-zero block; rint rounds half to even).
# One step dequantises (m = code * scale, v = (code * scale)^2), applies the
# AdamW update of adamw_step in float32 -- one IEEE rounding per operation,
# in the order written below -- and quantises the new statistics again.
# The codes are decided in float32, so this part of the oracle works in
# float32 too: the float32 coefficients are formed in double and rounded once,
# as adamw_coefficients states.

STATE_BLOCK = 256
F32 = np.float32


def adamw_coefficients(t, lr, b1, b2, eps, wd):
    """The float32 coefficients of step t: each formed in double from the
    double hyperparameters and rounded once."""
    return dict(decay=F32(1.0 - lr * wd), b1=F32(b1), omb1=F32(1.0 - b1), b2=F32(b2),
                omb2=F32(1.0 - b2), inv_sqrt_bc2=F32(1.0 / np.sqrt(1.0 - b2 ** t)),
                eps=F32(eps), step_size=F32(lr / (1.0 - b1 ** t)))


def quantize_state(x, signed):
    """Blockwise 8-bit codes and float32 scales of a float32 vector x (x >= 0
    when not signed).  Returns (codes int8 or uint8 [n], scales float32
    [ceil(n / 256)])."""
    x = np.asarray(x, dtype=F32)
    n = x.size
    nb = (n + STATE_BLOCK - 1) // STATE_BLOCK
    top = F32(127.0) if signed else F32(255.0)
    codes = np.zeros(n, dtype=np.int8 if signed else np.uint8)
    scales = np.zeros(nb, dtype=F32)
    for b in range(nb):
        blk = x[b * STATE_BLOCK:(b + 1) * STATE_BLOCK]
        s = F32(np.max(np.abs(blk))) / top           # one float32 division
        scales[b] = s
        if s == 0:
            continue
        q = np.rint(blk / s)                         # float32 division, half to even
        q = np.clip(q, -top if signed else F32(0.0), top)
        codes[b * STATE_BLOCK:(b + 1) * STATE_BLOCK] = q.astype(np.int32)
    return codes, scales


def dequantize_state(codes, scales):
    """float32 values code * scale of the block the element lies in."""
    codes = np.asarray(codes)
    s = np.repeat(np.asarray(scales, dtype=F32), STATE_BLOCK)[:codes.size]
    return codes.astype(F32) * s


def adamw8_step(p, g, m_codes, m_scales, v_codes, v_scales, t, lr, b1=0.9, b2=0.999,
                eps=1e-8, wd=0.0):
    """One AdamW step with 8-bit statistics.  p, g float32 [n]; the state as
    quantize_state gives it (m signed, v in the square-root domain).  Returns
    (p, m_codes, m_scales, v_codes, v_scales); inputs are not modified."""
    if t < 1:
        raise ValueError("the step number starts at 1")
    c = adamw_coefficients(t, lr, b1, b2, eps, wd)
    p = np.asarray(p, dtype=F32)
    g = np.asarray(g, dtype=F32)
    m = dequantize_state(m_codes, m_scales)
    u = dequantize_state(v_codes, v_scales)
    v = u * u
    p = p * c["decay"]
    m = c["b1"] * m + c["omb1"] * g
    v = c["b2"] * v + c["omb2"] * (g * g)
    u = np.sqrt(v)
    p = p - c["step_size"] * (m / (u * c["inv_sqrt_bc2"] + c["eps"]))
    mq, ms = quantize_state(m, signed=True)
    vq, vs = quantize_state(u, signed=False)
    return p, mq, ms, vq, vs
