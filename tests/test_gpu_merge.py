"""GPU parity of the adapter merge and re-quantisation against the oracle.

The merged float32 weight W' + s.B.A is compared element by element with the
oracle's float64 merge under the bound the float32 arithmetic gives,
|delta| <= (r + 3) * 2^-24 * (|W'| + s * sum_j |B_nj A_jk|)
(r fused multiply-adds, the scaling and the final add, each one rounding);
the re-quantised state is bit-exact against the oracle quantising the
device's own merged weights (the codes are decided in float32 on both
sides); in-place and workspace-only merges give the same bits."""
import numpy as np
import pytest
import torch

from gpu_common import DEV, bf16_np, host, oracle, say, to_dev

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module")
def q():
    import bit_quantized_lora_quant_amd as q
    q.lib()
    assert torch.cuda.is_available()
    return q


def _inputs(seed, N, K, r):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    lim = 1.0 / np.sqrt(K)
    a = torch.from_numpy(rng.uniform(-lim, lim, (r, K)).astype(np.float32)).to(torch.bfloat16)
    b = torch.from_numpy((rng.standard_normal((N, r)) * 0.05).astype(np.float32)).to(torch.bfloat16)
    return w, a, b


def _state(q, qq):
    """Host copies of a 4-bit tensor's buffers (int views for bitwise checks)."""
    out = {"codes": host(qq.codes).numpy()}
    if qq.double_quant:
        out["absmax_q"] = host(qq.absmax_q).numpy()
        out["absmax_scale"] = host(qq.absmax_scale).numpy().view(np.uint32)
        out["absmax_mean"] = host(qq.absmax_mean).numpy().view(np.uint32)
    else:
        out["absmax"] = host(qq.absmax).numpy().view(np.uint32)
    return out


CASES = [  # N, K, r, kind, dq
    (1024, 4096, 16, "nf4", True),
    (300, 1088, 128, "nf4", True),
    (77, 64, 1, "nf4", False),
    (257, 640, 33, "int4", True),
    (130, 192, 64, "int4", False),
]


@pytest.mark.parametrize("N,K,r,kind,dq", CASES, ids=lambda v: str(v))
def test_merge_then_requantize(q, N, K, r, kind, dq):
    say("merge N=%d K=%d r=%d %s dq=%s" % (N, K, r, kind, dq))
    w, a, b = _inputs(N * 7 + K + r, N, K, r)
    alpha = 2.0 * r
    qt = oracle.quantize(w, kind=kind, dq=dq)
    qq, _ = q.qlora_quantize_nf4(to_dev(w), quant_type=kind, double_quant=dq)
    A, B = to_dev(a), to_dev(b)
    out, merged = q.qlora_merge_requantize(qq, A, B, alpha, return_merged=True)
    torch.cuda.synchronize()
    wd = oracle.dequantize(qt).reshape(N, K).astype(np.float64)
    af, bfl = bf16_np(a), bf16_np(b)
    ref = oracle.merge_adapter(wd, af, bfl, alpha)
    got = host(merged).numpy().astype(np.float64)
    s = alpha / r
    bound = (r + 3) * U * (np.abs(wd) + s * (np.abs(bfl) @ np.abs(af)))
    bad = np.abs(got - ref) > bound
    assert not bad.any(), "merged off at %s: %s vs %s" % (
        np.argwhere(bad)[:4], got[bad][:4], ref[bad][:4])
    # the quantiser decides codes in float32: feed the oracle the device's
    # merged weights
    qm = oracle.quantize(host(merged).numpy(), kind=kind, dq=dq)
    st = _state(q, out)
    assert np.array_equal(st["codes"], qm["codes"])
    if dq:
        assert np.array_equal(st["absmax_q"], qm["absmax_q"])
        assert np.array_equal(st["absmax_scale"], qm["absmax_scale"].view(np.uint32))
        assert st["absmax_mean"][0] == np.float32(qm["absmax_mean"]).view(np.uint32)
    else:
        assert np.array_equal(st["absmax"], qm["absmax"].view(np.uint32))


def test_in_place_and_workspace_merge_agree(q):
    N, K, r = 512, 1024, 16
    say("merge in place")
    w, a, b = _inputs(5, N, K, r)
    A, B = to_dev(a), to_dev(b)
    q1, _ = q.qlora_quantize_nf4(to_dev(w))
    out = q.qlora_merge_requantize(q1, A, B, 32.0)           # merged in the workspace
    q2, _ = q.qlora_quantize_nf4(to_dev(w))
    q.qlora_merge_requantize(q2, A, B, 32.0, out=q2)          # in place
    torch.cuda.synchronize()
    s1, s2 = _state(q, out), _state(q, q2)
    for k in s1:
        assert np.array_equal(s1[k], s2[k]), k


def test_zero_adapter_requantizes_to_the_same_state(q):
    """B = 0 merges to W' itself; quantising the dequantised weight again
    gives back the same codes (every W' element is a level times its block's
    constant, and that constant's block max is reached again)."""
    N, K, r = 256, 512, 8
    say("merge zero adapter")
    w, a, _ = _inputs(9, N, K, r)
    for dq in (False,):
        qq, _ = q.qlora_quantize_nf4(to_dev(w), double_quant=dq)
        out = q.qlora_merge_requantize(qq, to_dev(a), torch.zeros((N, r), dtype=torch.bfloat16,
                                                                     device=DEV), 16.0)
        torch.cuda.synchronize()
        assert np.array_equal(host(out.codes).numpy(), host(qq.codes).numpy())
        assert np.array_equal(host(out.absmax).numpy(), host(qq.absmax).numpy())
