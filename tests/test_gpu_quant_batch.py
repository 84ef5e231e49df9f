"""GPU parity of the batched quantiser and dequantiser (qlora_quantize_nf4_batch,
qlora_dequantize_nf4_batch): every tensor of a batch that spans several
launches, mixes both 4-bit tables, tensors with and without double
quantisation and sizes from one weight to several tiles, must equal the oracle
bit for bit (codes, constants, mean, scales, dequantised float32 and bf16),
and equal what the single-tensor calls give."""
import numpy as np
import pytest
import torch

from gpu_common import DEV, host, oracle, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import bit_quantized_lora_quant_amd as q
    q.lib()
    assert torch.cuda.is_available()
    return q


def _u32(t):
    return host(t).numpy().view(np.uint32)


def _cases(seed, count):
    rng = np.random.default_rng(seed)
    shapes = [(1, 1), (1, 65), (3, 5), (7, 64 * 5 + 3), (64, 64), (257, 255), (1024, 1024),
              (333, 4096), (2, 100), (1, 2049 * 64)]
    out = []
    for i in range(count):
        rows, cols = shapes[i % len(shapes)] if i < len(shapes) else \
            (int(rng.integers(1, 300)), int(rng.integers(1, 3000)))
        w = (rng.standard_normal((rows, cols)) * 10.0 ** rng.uniform(-3, 0)).astype(np.float32)
        kind = "int4" if i % 3 == 2 else "nf4"
        dq = i % 4 != 3
        out.append((w, kind, dq))
    return out


def _check_state(qq, qt, label):
    assert np.array_equal(host(qq.codes).numpy(), qt["codes"]), label + ": codes"
    if qq.double_quant:
        assert _u32(qq.absmax_mean)[0] == np.float32(qt["absmax_mean"]).view(np.uint32), \
            label + ": mean"
        assert np.array_equal(_u32(qq.absmax_scale), qt["absmax_scale"].view(np.uint32)), \
            label + ": scales"
        assert np.array_equal(host(qq.absmax_q).numpy(), qt["absmax_q"]), label + ": int8 constants"
    else:
        assert np.array_equal(_u32(qq.absmax), qt["absmax"].view(np.uint32)), label + ": absmax"


@pytest.mark.parametrize("count", [1, 41, 70])
def test_batch_quantise_matches_the_oracle_and_single_calls(q, count):
    cases = _cases(count, count)
    say("quant batch of %d tensors" % count)
    Ws = [to_dev(w) for w, _, _ in cases]
    batch = [q.NF4Tensor(w.shape[0], w.shape[1], DEV, kind, dq) for w, kind, dq in cases]
    q.qlora_quantize_nf4_batch(Ws, batch)
    singles = [q.qlora_quantize_nf4(W, quant_type=kind, double_quant=dq)[0]
               for W, (_, kind, dq) in zip(Ws, cases)]
    torch.cuda.synchronize()
    for i, ((w, kind, dq), qq, qs) in enumerate(zip(cases, batch, singles)):
        label = "tensor %d %s %s dq=%s" % (i, w.shape, kind, dq)
        qt = oracle.quantize(w, kind, dq)
        _check_state(qq, qt, label)
        for name in ("codes", "absmax_q", "absmax_scale", "absmax_mean", "absmax"):
            a, b = getattr(qq, name), getattr(qs, name)
            assert (a is None) == (b is None) and (a is None or torch.equal(a, b)), \
                label + ": batch and single call differ in " + name
    # batched dequantisation, both output types, against the oracle
    wd = [oracle.dequantize(oracle.quantize(w, kind, dq)) for w, kind, dq in cases]
    for dt in (torch.float32, torch.bfloat16):
        outs = [torch.full((w.shape[0], w.shape[1]), float("nan"), dtype=dt, device=DEV)
                for w, _, _ in cases]
        q.qlora_dequantize_nf4_batch(batch, outs)
        torch.cuda.synchronize()
        for i, (o, ref) in enumerate(zip(outs, wd)):
            if dt == torch.float32:
                got = host(o).numpy().reshape(-1)
                assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), \
                    "fp32 dequant of tensor %d" % i
            else:
                got = host(o).view(torch.int16).numpy().view(np.uint16).reshape(-1)
                assert np.array_equal(got, oracle.to_bf16_bits(ref)), "bf16 dequant of tensor %d" % i


def test_batch_repeat_is_deterministic_and_reuses_the_workspace(q):
    """The same batch twice through one workspace (left holding the first
    call's partials) gives the same state."""
    cases = _cases(5, 36)
    Ws = [to_dev(w) for w, _, _ in cases]
    a = [q.NF4Tensor(w.shape[0], w.shape[1], DEV, kind, dq) for w, kind, dq in cases]
    b = [q.NF4Tensor(w.shape[0], w.shape[1], DEV, kind, dq) for w, kind, dq in cases]
    ws = q.qlora_quantize_nf4_batch(Ws, a)
    q.qlora_quantize_nf4_batch(Ws, b, ws)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        for name in ("codes", "absmax_q", "absmax_scale", "absmax_mean", "absmax"):
            u, v = getattr(x, name), getattr(y, name)
            assert u is None or torch.equal(u, v)


def test_batch_of_model_tensors(q):
    """One decoder layer's seven projections at the 8B model's shapes in one
    call: every state against the oracle."""
    shapes = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (14336, 4096),
              (14336, 4096), (4096, 14336)]
    rng = np.random.default_rng(9)
    ws_np = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in shapes]
    say("quant batch: 8B layer")
    Ws = [to_dev(w) for w in ws_np]
    qs = [q.NF4Tensor(r, c, DEV) for r, c in shapes]
    q.qlora_quantize_nf4_batch(Ws, qs)
    torch.cuda.synchronize()
    del Ws
    for i, (w, qq) in enumerate(zip(ws_np, qs)):
        _check_state(qq, oracle.quantize(w), "projection %d" % i)
