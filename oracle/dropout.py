"""Dropout mask of the LoRA input, for the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

PEFT's LoRA applies dropout to the layer input before the down-projection
(``lora_dropout`` of the LoraConfig in "QLoRA: Fine-Tuning a 70B on One GPU",
section "Practical Implementation", 0.05 there):

    Y = X . W'^T + s . (D(X) . A^T) . B^T,   D(X) = X * keep / (1 - p)

The keep decision of element (m, k) must be the same in the forward and the
backward and on both sides of a comparison, so it comes from a counter-based
generator: Philox4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011), written here from
that definition.  Readings (also in the design notes):
  * element e = m * K + k of X (row-major); counter (e div 4 as a 64-bit value
    in words 0 and 1, words 2 and 3 zero), key = the 64-bit seed (low word
    first); the element takes output word e mod 4;
  * keep when that word >= floor(p * 2^32) (so p = 0 keeps everything).
"""
import numpy as np

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = np.uint64(0x9E3779B9), np.uint64(0xBB67AE85)
_LO = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """Philox4x32-10 of counters ctr (uint32 [n, 4]) under key (k0, k1);
    returns uint32 [n, 4].  Each round multiplies words 0 and 2 by the two
    round constants into high and low halves, mixes the high halves with
    words 1 and 3 and the key, and the key advances by the two Weyl
    constants between rounds."""
    c = np.asarray(ctr, dtype=np.uint64).reshape(-1, 4)
    c0, c1, c2, c3 = c[:, 0], c[:, 1], c[:, 2], c[:, 3]
    k0, k1 = np.uint64(key[0]), np.uint64(key[1])
    for _ in range(10):
        p0 = _M0 * c0
        p1 = _M1 * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & _LO,
                          (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & _LO)
        k0 = (k0 + _W0) & _LO
        k1 = (k1 + _W1) & _LO
    return np.stack([c0, c1, c2, c3], axis=1).astype(np.uint32)


def threshold(p: float) -> int:
    """Drop when the element's word is below this (floor(p * 2^32))."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return min(int(np.floor(float(p) * 4294967296.0)), 0xFFFFFFFF)


def keep_mask(M: int, K: int, p: float, seed: int) -> np.ndarray:
    """bool [M, K]: which elements of X the dropout keeps."""
    n = M * K
    blocks = np.arange((n + 3) // 4, dtype=np.uint64)
    ctr = np.zeros((blocks.size, 4), dtype=np.uint64)
    ctr[:, 0] = blocks & _LO
    ctr[:, 1] = blocks >> np.uint64(32)
    words = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)).reshape(-1)[:n]
    return (words >= np.uint32(threshold(p)) if threshold(p) > 0
            else np.ones(n, dtype=bool)).reshape(M, K)
