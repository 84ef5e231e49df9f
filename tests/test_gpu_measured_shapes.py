"""GPU parity at the exact shapes and launch configurations the benchmark
times, against the float64 oracle (max|delta| <= 1e-2 * max|ref| + 1e-3 per
output tensor):

  * the Llama-3.1-8B layer step as the layer driver runs it: q/k/v as one
    grouped weight (N = 6144, three adapter pairs), o (4096 x 4096, split-K),
    gate/up as one grouped weight (N = 28672, two pairs), down (14336 ->
    4096); 2048 tokens, r = 16.  Y and dX on sampled rows, XA on the same
    rows, dA and dB in full, every projection against the oracle applied to
    that projection alone;
  * the LLaMA-65B gate projection (8192 -> 22016) at 4096 tokens, r = 64;
  * the 70B decode q/o (8192 -> 8192) and gate/up (8192 -> 28672) shapes at
    1, 4 and 16 tokens, r = 64, every output element.
"""
import numpy as np
import pytest
import torch

from gpu_common import DEV, assert_close, bf16_np, host, oracle, oracle_weight, say, to_dev, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import bit_quantized_lora_quant_amd as q
    q.lib()
    assert torch.cuda.is_available()
    return q


# the layer driver's units: projections that read one input share a weight
UNITS = [("qkv", [0, 1, 2]), ("o", [3]), ("gate_up", [4, 5]), ("down", [6])]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("unit", UNITS, ids=[u[0] for u in UNITS])
def test_llama8b_layer_driver_unit(q, unit):
    name, idx = unit
    wl = workloads.LLAMA8B_LAYER
    M, r, alpha = wl.m, wl.r, wl.alpha
    ins = [workloads.linear_inputs(wl, 0, t) for t in idx]
    K = wl.linears[idx[0]][1]
    rows = [wl.linears[t][2] for t in idx]
    N, G = sum(rows), len(idx)
    say("8B layer unit %s M=%d N=%d K=%d G=%d r=%d" % (name, M, N, K, G, r))
    w = np.concatenate([i[0] for i in ins], 0)
    x = ins[0][1]                                   # the shared layer input
    X = to_dev(x)
    if G == 1:
        A, B, dY = to_dev(ins[0][2]), to_dev(ins[0][3]), to_dev(ins[0][4])
    else:
        A = to_dev(torch.cat([i[2] for i in ins], 0))
        Bh = torch.zeros((N, G * r), dtype=torch.bfloat16)
        e = 0
        for g, i in enumerate(ins):
            Bh[e:e + rows[g], g * r:(g + 1) * r] = i[3]
            e += rows[g]
        B = to_dev(Bh)
        dY = to_dev(torch.cat([i[4] for i in ins], 1))
    qq, _ = q.qlora_quantize_nf4(to_dev(w))
    if G == 1:
        Y, XA = q.qlora_linear_fwd(qq, X, A, B, alpha, return_xa=True)
        dX, dA, dB = q.qlora_linear_bwd(qq, X, A, B, alpha, dY, XA_in=XA)
    else:
        Y, XA = q.qlora_grouped_fwd(qq, X, A, B, r, rows, alpha, return_xa=True)
        dX, dA, dB = q.qlora_grouped_bwd(qq, X, A, B, r, rows, alpha, dY, XA_in=XA)
    torch.cuda.synchronize()
    Yh, XAh, dXh = bf16_np(Y), bf16_np(XA), bf16_np(dX)
    dAh, dBh = host(dA).numpy(), host(dB).numpy()
    del Y, XA, dX, dA, dB
    _, wd = oracle_weight(w)
    xf = bf16_np(x)
    sample = np.sort(np.random.default_rng(len(name)).choice(M, size=128, replace=False))
    dx_ref = 0.0
    e = 0
    for g, (_, _, a, b, dy) in enumerate(ins):
        sl, cs = slice(e, e + rows[g]), slice(g * r, (g + 1) * r)
        af, bfl, dyf = bf16_np(a), bf16_np(b), bf16_np(dy)
        y_ref, xa_ref = oracle.linear_fwd(wd[sl], xf[sample], af, bfl, alpha)
        assert_close("Y[%d]" % g, Yh[sample][:, sl], y_ref)
        assert_close("XA[%d]" % g, XAh[sample][:, cs], xa_ref)
        dx_g, _, _ = oracle.linear_bwd(wd[sl], xf[sample], af, bfl, alpha, dyf[sample])
        dx_ref = dx_ref + dx_g
        da_ref, db_ref = oracle.adapter_grads(xf, af, bfl, alpha, dyf)
        assert_close("dA[%d]" % g, dAh[cs], da_ref)
        assert_close("dB[%d]" % g, dBh[sl, cs], db_ref)
        if G > 1:
            off = dBh[sl].copy()
            off[:, cs] = 0.0
            assert not off.any(), "dB off the diagonal block of group %d" % g
        e += rows[g]
    assert_close("dX", dXh[sample], dx_ref)


@pytest.mark.timeout(300)
def test_llama65b_gate_sampled(q):
    """LLaMA-65B gate projection 8192 -> 22016 at 4096 tokens, r = 64: 128
    sampled rows of Y / XA / dX, dA and dB in full."""
    wl = workloads.LLAMA65B_LAYER
    w, x, a, b, dy = workloads.linear_inputs(wl, 0, 4)
    say("65B gate M=%d N=%d K=%d r=%d" % (wl.m, w.shape[0], w.shape[1], wl.r))
    qq, _ = q.qlora_quantize_nf4(to_dev(w))
    X, A, B, dY = to_dev(x), to_dev(a), to_dev(b), to_dev(dy)
    Y, XA = q.qlora_linear_fwd(qq, X, A, B, wl.alpha, return_xa=True)
    dX, dA, dB = q.qlora_linear_bwd(qq, X, A, B, wl.alpha, dY, XA_in=XA)
    torch.cuda.synchronize()
    _, wd = oracle_weight(w)
    xf, af, bfl, dyf = bf16_np(x), bf16_np(a), bf16_np(b), bf16_np(dy)
    rows = np.sort(np.random.default_rng(4).choice(wl.m, size=128, replace=False))
    y_ref, xa_ref = oracle.linear_fwd(wd, xf[rows], af, bfl, wl.alpha)
    assert_close("Y", bf16_np(Y)[rows], y_ref)
    assert_close("XA", bf16_np(XA)[rows], xa_ref)
    dx_ref, _, _ = oracle.linear_bwd(wd, xf[rows], af, bfl, wl.alpha, dyf[rows])
    assert_close("dX", bf16_np(dX)[rows], dx_ref)
    da_ref, db_ref = oracle.adapter_grads(xf, af, bfl, wl.alpha, dyf)
    assert_close("dA", host(dA).numpy(), da_ref)
    assert_close("dB", host(dB).numpy(), db_ref)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("tensor", [0, 4], ids=["q_proj", "gate_proj"])
def test_decode_70b_wide_shapes(q, tensor):
    """70B decode q (8192 -> 8192) and gate (8192 -> 28672) at 1, 4 and 16
    tokens: every element of Y and XA (one quantisation, three token counts)."""
    wl = workloads.LLAMA70B_DECODE
    w, _, a, b, _ = workloads.linear_inputs(wl, 0, tensor, m=1)
    qq, _ = q.qlora_quantize_nf4(to_dev(w))
    _, wd = oracle_weight(w)
    af, bfl = bf16_np(a), bf16_np(b)
    A, B = to_dev(a), to_dev(b)
    for M in wl.decode_m:
        x = workloads.activations(wl.key, 0, tensor, M, w.shape[1])
        say("decode M=%d %s N=%d K=%d" % (M, wl.linears[tensor][0], w.shape[0], w.shape[1]))
        Y, XA = q.qlora_linear_fwd(qq, to_dev(x), A, B, wl.alpha, return_xa=True)
        torch.cuda.synchronize()
        y_ref, xa_ref = oracle.linear_fwd(wd, bf16_np(x), af, bfl, wl.alpha)
        assert_close("Y M=%d" % M, bf16_np(Y), y_ref)
        assert_close("XA M=%d" % M, bf16_np(XA), xa_ref)
