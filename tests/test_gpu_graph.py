"""HIP graph capture of the library's calls (the benchmark replays its
quantise/dequantise passes and decode steps from graphs): every replay must
reproduce the eager results bit for bit, with eager work and synchronisation
between replays.  The calls record only kernel launches (no memset nodes)."""
import numpy as np
import pytest
import torch

from gpu_common import DEV, say

import bit_quantized_lora_quant_amd as q

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _scribble(ts):
    # eager work between replays: overwrite the outputs so a replay that
    # writes nothing cannot pass
    for t in ts:
        t.view(torch.uint8).fill_(0xA5)
    x = torch.randn(1 << 20, device=DEV)
    (x * 2.0).sum().item()
    torch.cuda.synchronize()


def test_quantize_dequantize_graph_replays():
    say("graph: quantize + dequantize 384x1088")
    g0 = torch.Generator(device=DEV)
    g0.manual_seed(11)
    W = torch.randn((384, 1088), generator=g0, device=DEV) * 0.02
    Q = q.NF4Tensor(384, 1088, DEV)
    ws = q.workspace(q.qlora_quantize_workspace_bytes(384, 1088), DEV)
    out = torch.empty((384, 1088), dtype=torch.bfloat16, device=DEV)

    def run():
        q.qlora_quantize_nf4(W, Q, ws)
        q.qlora_dequantize_nf4(Q, out=out)

    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (Q.codes, Q.absmax_q, Q.absmax_scale, Q.absmax_mean, out)]
    g = _capture(run)
    for i in range(REPLAYS):
        _scribble([Q.codes, Q.absmax_q, Q.absmax_scale, Q.absmax_mean, out])
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("codes", "absmax_q", "scale", "mean", "dequant"),
                              (Q.codes, Q.absmax_q, Q.absmax_scale, Q.absmax_mean, out), ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (i, name)


@pytest.mark.parametrize("M,N,K,r", [(4, 1024, 2048, 64), (300, 512, 4160, 16)],
                         ids=["decode_M4", "gemm_split"])
def test_linear_graph_replays(M, N, K, r):
    say("graph: linear fwd+bwd M=%d N=%d K=%d r=%d" % (M, N, K, r))
    g0 = torch.Generator(device=DEV)
    g0.manual_seed(M + N)
    W = torch.randn((N, K), generator=g0, device=DEV) * 0.02
    Qw, _ = q.qlora_quantize_nf4(W)
    X = torch.randn((M, K), generator=g0, device=DEV).to(torch.bfloat16)
    A = (torch.rand((r, K), generator=g0, device=DEV) * 2 - 1).mul_(K ** -0.5).to(torch.bfloat16)
    B = (torch.randn((N, r), generator=g0, device=DEV) * 0.01).to(torch.bfloat16)
    dY = torch.randn((M, N), generator=g0, device=DEV).to(torch.bfloat16)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    XA = torch.empty((M, r), dtype=torch.bfloat16, device=DEV)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    dA = torch.empty((r, K), dtype=torch.float32, device=DEV)
    dB = torch.empty((N, r), dtype=torch.float32, device=DEV)
    ws = q.workspace(q.qlora_linear_workspace_bytes(M, N, K, r), DEV)

    def run():
        q.qlora_linear_fwd(Qw, X, A, B, 2.0, Y=Y, XA_out=XA, ws=ws, return_xa=True)
        q.qlora_linear_bwd(Qw, X, A, B, 2.0, dY, XA_in=XA, dX=dX, dA=dA, dB=dB, ws=ws)

    run()
    torch.cuda.synchronize()
    outs = [Y, XA, dX, dA, dB]
    ref = [t.clone() for t in outs]
    g = _capture(run)
    for i in range(REPLAYS):
        _scribble(outs)
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("Y", "XA", "dX", "dA", "dB"), outs, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (i, name)
    assert np.isfinite(Y.float().cpu().numpy()).all()


def test_grouped_and_dropout_graph_replays():
    """The grouped layer-driver calls and the dropout calls (with stored keep
    bits) replayed from one graph."""
    M, K, r = 300, 512, 16
    rows = [256, 64, 64]
    N = sum(rows)
    say("graph: grouped + dropout M=%d N=%d K=%d" % (M, N, K))
    g0 = torch.Generator(device=DEV)
    g0.manual_seed(5)
    Qw, _ = q.qlora_quantize_nf4(torch.randn((N, K), generator=g0, device=DEV) * 0.02)
    X = torch.randn((M, K), generator=g0, device=DEV).to(torch.bfloat16)
    A = (torch.rand((3 * r, K), generator=g0, device=DEV) * 2 - 1).mul_(K ** -0.5).to(torch.bfloat16)
    B = torch.zeros((N, 3 * r), dtype=torch.bfloat16, device=DEV)
    e = 0
    for g, n in enumerate(rows):
        B[e:e + n, g * r:(g + 1) * r] = (torch.randn((n, r), generator=g0, device=DEV) * 0.01)
        e += n
    A1, B1 = A[:r].contiguous(), (torch.randn((N, r), generator=g0, device=DEV) * 0.01).to(torch.bfloat16)
    dY = torch.randn((M, N), generator=g0, device=DEV).to(torch.bfloat16)
    outs = dict(Y=torch.empty((M, N), dtype=torch.bfloat16, device=DEV),
                XA=torch.empty((M, 3 * r), dtype=torch.bfloat16, device=DEV),
                dX=torch.empty((M, K), dtype=torch.bfloat16, device=DEV),
                dA=torch.empty((3 * r, K), dtype=torch.float32, device=DEV),
                dB=torch.empty((N, 3 * r), dtype=torch.float32, device=DEV),
                Yd=torch.empty((M, N), dtype=torch.bfloat16, device=DEV),
                XAd=torch.empty((M, r), dtype=torch.bfloat16, device=DEV),
                bits=q.keep_bits_buffer(M, K, DEV),
                dXd=torch.empty((M, K), dtype=torch.bfloat16, device=DEV),
                dAd=torch.empty((r, K), dtype=torch.float32, device=DEV),
                dBd=torch.empty((N, r), dtype=torch.float32, device=DEV))
    ws = q.workspace(q.qlora_grouped_workspace_bytes(M, N, K, r, 3), DEV)
    o = outs

    def run():
        q.qlora_grouped_fwd(Qw, X, A, B, r, rows, 32.0, Y=o["Y"], XA_out=o["XA"], ws=ws,
                            return_xa=True)
        q.qlora_grouped_bwd(Qw, X, A, B, r, rows, 32.0, dY, XA_in=o["XA"], dX=o["dX"],
                            dA=o["dA"], dB=o["dB"], ws=ws)
        q.qlora_linear_fwd(Qw, X, A1, B1, 32.0, Y=o["Yd"], XA_out=o["XAd"], ws=ws,
                           return_xa=True, dropout=(0.1, 77), keep_bits=o["bits"])
        q.qlora_linear_bwd(Qw, X, A1, B1, 32.0, dY, XA_in=o["XAd"], dX=o["dXd"], dA=o["dAd"],
                           dB=o["dBd"], ws=ws, dropout=(0.1, 77), keep_bits=o["bits"])

    run()
    torch.cuda.synchronize()
    ref = {k: t.clone() for k, t in outs.items()}
    g = _capture(run)
    for i in range(REPLAYS):
        _scribble(list(outs.values()))
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k].view(torch.uint8), ref[k].view(torch.uint8)), (i, k)


def test_merge_and_adamw_graph_replays():
    """The merge + re-quantise call and one optimiser step replayed from a
    graph; each replay starts from the same restored inputs."""
    N, K, r = 256, 512, 8
    say("graph: merge + adamw")
    g0 = torch.Generator(device=DEV)
    g0.manual_seed(9)
    W = torch.randn((N, K), generator=g0, device=DEV) * 0.02
    Qw, _ = q.qlora_quantize_nf4(W)
    A = (torch.randn((r, K), generator=g0, device=DEV) * 0.05).to(torch.bfloat16)
    B = (torch.randn((N, r), generator=g0, device=DEV) * 0.05).to(torch.bfloat16)
    out = q.NF4Tensor(N, K, DEV)
    merged = torch.empty((N, K), dtype=torch.float32, device=DEV)
    mws = q.workspace(q.qlora_merge_workspace_bytes(N, K), DEV)
    P0 = torch.randn(5000, generator=g0, device=DEV)
    G = torch.randn(5000, generator=g0, device=DEV) * 1e-3
    P, Mo, V = P0.clone(), torch.zeros(5000, device=DEV), torch.zeros(5000, device=DEV)
    PB = torch.empty(5000, dtype=torch.bfloat16, device=DEV)

    def run():
        q.qlora_merge_requantize(Qw, A, B, 16.0, out=out, merged=merged, ws=mws)
        q.qlora_adamw_step([(P, G, Mo, V, PB)], 1, 1e-3, weight_decay=0.01)

    def restore():
        P.copy_(P0)
        Mo.zero_()
        V.zero_()

    run()
    torch.cuda.synchronize()
    outs = [out.codes, out.absmax_q, out.absmax_scale, out.absmax_mean, merged, P, Mo, V, PB]
    ref = [t.clone() for t in outs]
    restore()
    g = _capture(run)
    for i in range(REPLAYS):
        _scribble([out.codes, out.absmax_q, out.absmax_scale, out.absmax_mean, merged, PB])
        restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (i, j)
