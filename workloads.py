"""Seeded synthetic inputs and the workload shapes they are drawn for.

This module holds no step of the method: it only names shapes and draws random
numbers, and it serves the tests, the smoke check and the benchmark alike (both
the GPU library and the CPU oracle receive the same bytes from here).

Random streams: numpy ``Generator(PCG64(SeedSequence([workload, layer, tensor,
role])))`` on the host.  Roles: W=0, A=1, B=2, X=3, dY=4.  Weights are float32
~N(0, 0.02); A ~U(-1/sqrt(K), 1/sqrt(K)); B ~N(0, 0.01) (non-zero so the LoRA
path is exercised); X and dY ~N(0, 1).  X, dY, A and B are rounded once to
bfloat16 (round to nearest even) and those bf16 values are the inputs.

Very large weight sets (the full 8.03B-parameter set, 80-layer stacks) are
drawn on the device with torch's seeded CUDA generator instead (see
``device_weight``); a host copy of those exact values is what the oracle sees.

The Llama-3.1-8B projection widths are the pages' (xingyuzhitong guide,
section "LoRA: freeze the base, train small adapters": model width 4,096, KV
width 1,024, feed-forward width 14,336, seven adapted projections per layer).
The LLaMA-65B layer (width 8,192, 64 heads x 128, feed-forward 22,016) and the
70B decode shapes (width 8,192, KV 1,024, feed-forward 28,672) follow the public
model configurations; the pages give only those models' parameter totals.
"""
from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

ROLE_W, ROLE_A, ROLE_B, ROLE_X, ROLE_DY = 0, 1, 2, 3, 4

# (name, K = in_features, N = out_features)
LLAMA8B_LINEARS: List[Tuple[str, int, int]] = [
    ("q_proj", 4096, 4096), ("k_proj", 4096, 1024), ("v_proj", 4096, 1024),
    ("o_proj", 4096, 4096), ("gate_proj", 4096, 14336), ("up_proj", 4096, 14336),
    ("down_proj", 14336, 4096),
]
LLAMA65B_LINEARS = [
    ("q_proj", 8192, 8192), ("k_proj", 8192, 8192), ("v_proj", 8192, 8192),
    ("o_proj", 8192, 8192), ("gate_proj", 8192, 22016), ("up_proj", 8192, 22016),
    ("down_proj", 22016, 8192),
]
LLAMA70B_LINEARS = [
    ("q_proj", 8192, 8192), ("k_proj", 8192, 1024), ("v_proj", 8192, 1024),
    ("o_proj", 8192, 8192), ("gate_proj", 8192, 28672), ("up_proj", 8192, 28672),
    ("down_proj", 28672, 8192),
]
# Vocabulary of the public Llama-3.1 tokenizer (not printed on the pages); only
# the embedding and LM-head shapes of the full weight set use it.
LLAMA3_VOCAB = 128256


@dataclass
class Workload:
    key: int                      # first word of every seed
    name: str
    linears: List[Tuple[str, int, int]]
    r: int
    alpha: float
    m: int                        # tokens per step (rows of X)
    layers: int = 1
    notes: str = ""
    decode_m: List[int] = field(default_factory=list)


SINGLE_1024 = Workload(0, "single linear 1024->1024, r=8, alpha=16, 128 tokens",
                       [("linear", 1024, 1024)], r=8, alpha=16.0, m=128)
LLAMA8B_LAYER = Workload(1, "Llama-3.1-8B layer linears, r=16, alpha=32, 1x2048 tokens",
                         LLAMA8B_LINEARS, r=16, alpha=32.0, m=2048, layers=32)
LLAMA8B_WEIGHTS = Workload(2, "Llama-3.1-8B full weight set (8.03B params) quantise+dequantise",
                           LLAMA8B_LINEARS, r=16, alpha=32.0, m=0, layers=32)
LLAMA65B_LAYER = Workload(3, "LLaMA-65B layer linears, r=64, alpha=16, 4x1024 tokens, 80 layers",
                          LLAMA65B_LINEARS, r=64, alpha=16.0, m=4096, layers=80)
LLAMA70B_DECODE = Workload(4, "70B-shaped decode GEMV, r=64, alpha=16, M in {1,4,16}",
                           LLAMA70B_LINEARS, r=64, alpha=16.0, m=1, layers=80,
                           decode_m=[1, 4, 16])

WORKLOADS = [SINGLE_1024, LLAMA8B_LAYER, LLAMA8B_WEIGHTS, LLAMA65B_LAYER, LLAMA70B_DECODE]


def llama8b_weight_set() -> List[Tuple[str, int, int, int]]:
    """(name, layer, rows, cols) of every 2-D weight of the 8.03B model: 32
    layers x 7 projections, plus the embedding and the LM head."""
    out = [("embed_tokens", -1, LLAMA3_VOCAB, 4096)]
    for layer in range(32):
        for name, k, n in LLAMA8B_LINEARS:
            out.append((name, layer, n, k))
    out.append(("lm_head", -1, LLAMA3_VOCAB, 4096))
    return out


def _rng(*words: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(w) & 0x7FFFFFFF for w in words])))


def weight(key: int, layer: int, tensor: int, n: int, k: int, std: float = 0.02) -> np.ndarray:
    """float32 [n, k] ~N(0, std)."""
    g = _rng(key, layer, tensor, ROLE_W)
    return g.standard_normal((n, k), dtype=np.float32) * np.float32(std)


def _bf16(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def lora_a(key: int, layer: int, tensor: int, r: int, k: int):
    g = _rng(key, layer, tensor, ROLE_A)
    lim = 1.0 / np.sqrt(k)
    return _bf16(g.uniform(-lim, lim, size=(r, k)).astype(np.float32))


def lora_b(key: int, layer: int, tensor: int, n: int, r: int, std: float = 0.01):
    g = _rng(key, layer, tensor, ROLE_B)
    return _bf16(g.standard_normal((n, r), dtype=np.float32) * np.float32(std))


def activations(key: int, layer: int, tensor: int, m: int, k: int, role: int = ROLE_X):
    g = _rng(key, layer, tensor, role)
    return _bf16(g.standard_normal((m, k), dtype=np.float32))


def device_weight(key: int, layer: int, tensor: int, n: int, k: int, std: float = 0.02,
                  device="cuda"):
    """float32 [n, k] ~N(0, std) drawn on the device (torch Philox stream)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(((key & 0xFFFF) << 32) | ((layer & 0xFFFF) << 16) | (tensor & 0xFFFF))
    w = torch.empty((n, k), dtype=torch.float32, device=device)
    w.normal_(0.0, std, generator=g)
    return w


def bf16_to_f64(t) -> np.ndarray:
    """Exact float64 values of a bf16 torch tensor."""
    import torch
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)


def linear_inputs(wl: Workload, layer: int, tensor: int, m: int = None):
    """(W fp32 numpy [N,K], X, A, B, dY bf16 torch CPU) for one linear."""
    name, k, n = wl.linears[tensor]
    m = wl.m if m is None else m
    w = weight(wl.key, layer, tensor, n, k)
    x = activations(wl.key, layer, tensor, m, k, ROLE_X)
    a = lora_a(wl.key, layer, tensor, wl.r, k)
    b = lora_b(wl.key, layer, tensor, n, wl.r)
    dy = activations(wl.key, layer, tensor, m, n, ROLE_DY)
    return w, x, a, b, dy
