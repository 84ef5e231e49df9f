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
