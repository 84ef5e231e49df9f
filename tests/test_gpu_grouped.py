"""GPU parity of the grouped linear (projections of one input fused into one
weight, each with its own adapter pair) against the oracle applied to every
projection on its own: Y and XA per group, dX as the sum of the groups' input
gradients, dA and dB per group, all within max|delta| <= 1e-2 * max|ref| +
1e-3, and dB exactly zero off the diagonal blocks."""
import numpy as np
import pytest
import torch

from gpu_common import DEV, assert_close, bf16_np, host, oracle, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import bit_quantized_lora_quant_amd as q
    q.lib()
    assert torch.cuda.is_available()
    return q


def _inputs(seed, M, rows, K, r):
    rng = np.random.default_rng(seed)
    N = sum(rows)
    G = len(rows)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    lim = 1.0 / np.sqrt(K)
    a = torch.from_numpy(rng.uniform(-lim, lim, (G * r, K)).astype(np.float32)).to(torch.bfloat16)
    b = torch.zeros((N, G * r), dtype=torch.bfloat16)
    e = 0
    for g, n in enumerate(rows):
        blk = (rng.standard_normal((n, r)) * 0.05).astype(np.float32)
        b[e:e + n, g * r:(g + 1) * r] = torch.from_numpy(blk).to(torch.bfloat16)
        e += n
    dy = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(torch.bfloat16)
    return w, x, a, b, dy


CASES = [  # M, group rows, K, r
    (300, (256, 64, 64), 512, 16),        # q/k/v-like, ragged M
    (512, (1024, 256, 256), 1024, 16),
    (130, (640, 640), 384, 32),           # gate/up-like
    (2048, (4096, 1024, 1024), 4096, 16),  # the 8B q/k/v shape (sampled rows)
    (4, (256, 64, 64), 512, 16),          # decode path
]


@pytest.mark.parametrize("M,rows,K,r", CASES, ids=lambda v: str(v))
def test_grouped_matches_separate_projections(q, M, rows, K, r):
    say("grouped M=%d rows=%s K=%d r=%d" % (M, rows, K, r))
    w, x, a, b, dy = _inputs(M + K + r, M, rows, K, r)
    alpha = 2.0 * r
    G = len(rows)
    qq, _ = q.qlora_quantize_nf4(to_dev(w))
    X, A, B, dY = to_dev(x), to_dev(a), to_dev(b), to_dev(dy)
    Y, XA = q.qlora_grouped_fwd(qq, X, A, B, r, rows, alpha, return_xa=True)
    res = {}
    if M > 16:
        res["dX"], res["dA"], res["dB"] = q.qlora_grouped_bwd(qq, X, A, B, r, rows, alpha, dY,
                                                              XA_in=XA)
    torch.cuda.synchronize()
    wd = oracle.dequantize(oracle.quantize(w)).reshape(w.shape)
    xf, af, bfl, dyf = bf16_np(x), bf16_np(a), bf16_np(b), bf16_np(dy)
    sample = np.arange(M) if M <= 512 else np.sort(
        np.random.default_rng(1).choice(M, size=128, replace=False))
    Yh, XAh = bf16_np(Y), bf16_np(XA)
    dx_ref = 0.0
    e = 0
    for g, n in enumerate(rows):
        sl = slice(e, e + n)
        cs = slice(g * r, (g + 1) * r)
        a_g, b_g = af[cs], bfl[sl, cs]
        y_ref, xa_ref = oracle.linear_fwd(wd[sl], xf[sample], a_g, b_g, alpha)
        assert_close("Y[%d]" % g, Yh[sample][:, sl], y_ref)
        assert_close("XA[%d]" % g, XAh[sample][:, cs], xa_ref)
        if M > 16:
            dx_g, _, _ = oracle.linear_bwd(wd[sl], xf[sample], a_g, b_g, alpha, dyf[sample][:, sl])
            dx_ref = dx_ref + dx_g
            da_g, db_g = oracle.adapter_grads(xf, a_g, b_g, alpha, dyf[:, sl])
            assert_close("dA[%d]" % g, host(res["dA"]).numpy()[cs], da_g)
            assert_close("dB[%d]" % g, host(res["dB"]).numpy()[sl, cs], db_g)
            off = host(res["dB"]).numpy()[sl].copy()
            off[:, cs] = 0.0
            assert not off.any(), "dB off the diagonal block of group %d" % g
        e += n
    if M > 16:
        assert_close("dX", bf16_np(res["dX"])[sample], dx_ref)
