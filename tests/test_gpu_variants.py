"""GPU parity of the 4-bit type and constant variants against the oracle: the
INT4 table, and float32 block constants without double quantisation.  Codes,
constants and dequantised weights bit for bit; the fused forward and backward
and the decode path within max|delta| <= 1e-2 * max|ref| + 1e-3; and the
NF4-vs-INT4 reconstruction error on normal weights, measured on the device."""
import numpy as np
import pytest
import torch

from gpu_common import DEV, assert_close, bf16_np, host, oracle, say, to_dev

pytestmark = pytest.mark.gpu

VARIANTS = [("int4", True), ("int4", False), ("nf4", False)]


@pytest.fixture(scope="module")
def q():
    import bit_quantized_lora_quant_amd as q
    q.lib()
    assert torch.cuda.is_available()
    return q


def _quant_both(q, w_np, kind, dq):
    qt = oracle.quantize(w_np, kind=kind, dq=dq)
    qq, ws = q.qlora_quantize_nf4(to_dev(w_np), quant_type=kind, double_quant=dq)
    torch.cuda.synchronize()
    return qt, qq, ws


def _check_state(q, qt, qq, ws):
    codes = host(qq.codes).numpy()
    assert np.array_equal(codes, qt["codes"]), "codes differ at %s" % (
        np.nonzero(codes != qt["codes"])[0][:8],)
    if qt["dq"]:
        nb = qt["absmax"].size
        absmax = host(ws[: nb * 4].view(torch.float32)).numpy()
        assert np.array_equal(absmax.view(np.uint32), qt["absmax"].view(np.uint32))
        assert np.array_equal(host(qq.absmax_q).numpy(), qt["absmax_q"])
        assert np.array_equal(host(qq.absmax_scale).numpy().view(np.uint32),
                              qt["absmax_scale"].view(np.uint32))
        assert host(qq.absmax_mean).numpy().view(np.uint32)[0] == \
            np.float32(qt["absmax_mean"]).view(np.uint32)
    else:
        assert qq.absmax_q is None
        assert np.array_equal(host(qq.absmax).numpy().view(np.uint32),
                              qt["absmax"].view(np.uint32))
    consts = host(q.qlora_dequantize_absmax(qq)).numpy()
    assert np.array_equal(consts.view(np.uint32), oracle.block_constants(qt).view(np.uint32))
    wd = oracle.dequantize(qt)
    f32 = host(q.qlora_dequantize_nf4(qq, torch.float32)).numpy().reshape(-1)
    assert np.array_equal(f32.view(np.uint32), wd.view(np.uint32)), "fp32 dequant at %s" % (
        np.nonzero(f32.view(np.uint32) != wd.view(np.uint32))[0][:8],)
    b16 = host(q.qlora_dequantize_nf4(qq, torch.bfloat16)).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b16.reshape(-1), oracle.to_bf16_bits(wd)), "bf16 dequant"
    return wd


@pytest.mark.parametrize("kind,dq", VARIANTS, ids=lambda v: str(v))
@pytest.mark.parametrize("shape", [(1, 7), (3, 65), (257, 255), (1024, 1024), (333, 4096)],
                         ids=lambda s: "%dx%d" % s)
def test_quantize_dequant_bit_exact(q, kind, dq, shape):
    say("variant quant %s dq=%s %s" % (kind, dq, shape))
    rng = np.random.default_rng(shape[0] * 31 + shape[1])
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    w.reshape(-1)[:64] = 0.0   # an all-zero block
    qt, qq, ws = _quant_both(q, w, kind, dq)
    _check_state(q, qt, qq, ws)


@pytest.mark.parametrize("kind", ["nf4", "int4"])
def test_table_levels_and_midpoints(q, kind):
    """Every level, and the floats on both sides of every decision threshold,
    times powers of two: codes and float32 constants bit for bit."""
    say("variant levels %s" % kind)
    cb = oracle.codebook(kind).astype(np.float64)
    vals = [cb[1:]]
    for j in range(15):
        m = np.float32(0.5 * (cb[j] + cb[j + 1]))
        vals.append(np.array([np.nextafter(m, np.float32(-2)), m, np.nextafter(m, np.float32(2))]))
    v = np.concatenate(vals).astype(np.float32)
    v = v[np.abs(v) <= 1.0]
    blocks = []
    for e in (-7, 0, 3):
        for i in range(0, v.size, 63):
            blk = np.zeros(64, dtype=np.float32)
            chunk = v[i:i + 63]
            blk[: chunk.size] = chunk
            blk[63] = 1.0   # absmax 1 before scaling: the weight / absmax is the value itself
            blocks.append(blk * np.float32(2.0 ** e))
    w = np.concatenate(blocks).reshape(-1, 64)
    for dq in (True, False):
        qt, qq, ws = _quant_both(q, w, kind, dq)
        _check_state(q, qt, qq, ws)


@pytest.mark.parametrize("kind,dq", VARIANTS, ids=lambda v: str(v))
def test_linear_fwd_bwd(q, kind, dq):
    """Fused forward and backward on a ragged shape and a split-K shape."""
    for M, N, K, r in [(300, 1216, 1088, 24), (2048, 1024, 4096, 16)]:
        say("variant linear %s dq=%s M=%d N=%d K=%d r=%d" % (kind, dq, M, N, K, r))
        rng = np.random.default_rng(M + N + K + r)
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
        lim = 1.0 / np.sqrt(K)
        a = torch.from_numpy(rng.uniform(-lim, lim, (r, K)).astype(np.float32)).to(torch.bfloat16)
        b = torch.from_numpy((rng.standard_normal((N, r)) * 0.01).astype(np.float32)).to(torch.bfloat16)
        dy = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(torch.bfloat16)
        alpha = 2.0 * r
        qt, qq, _ = _quant_both(q, w, kind, dq)
        X, A, B, dY = to_dev(x), to_dev(a), to_dev(b), to_dev(dy)
        Y, XA = q.qlora_linear_fwd(qq, X, A, B, alpha, return_xa=True)
        dX, dA, dB = q.qlora_linear_bwd(qq, X, A, B, alpha, dY, XA_in=XA)
        torch.cuda.synchronize()
        wd = oracle.dequantize(qt).reshape(N, K)
        xf, af, bfl, dyf = bf16_np(x), bf16_np(a), bf16_np(b), bf16_np(dy)
        rows = np.sort(np.random.default_rng(1).choice(M, size=min(M, 128), replace=False))
        y_ref, xa_ref = oracle.linear_fwd(wd, xf[rows], af, bfl, alpha)
        dx_ref, _, _ = oracle.linear_bwd(wd, xf[rows], af, bfl, alpha, dyf[rows])
        assert_close("Y", bf16_np(Y)[rows], y_ref)
        assert_close("XA", bf16_np(XA)[rows], xa_ref)
        assert_close("dX", bf16_np(dX)[rows], dx_ref)
        da_ref, db_ref = oracle.adapter_grads(xf, af, bfl, alpha, dyf)
        assert_close("dA", host(dA).numpy(), da_ref)
        assert_close("dB", host(dB).numpy(), db_ref)


@pytest.mark.parametrize("kind,dq", VARIANTS, ids=lambda v: str(v))
@pytest.mark.parametrize("M", [1, 16])
def test_decode(q, kind, dq, M):
    N, K, r = 1024, 8192, 64
    say("variant decode %s dq=%s M=%d" % (kind, dq, M))
    rng = np.random.default_rng(M * 3 + len(kind))
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    lim = 1.0 / np.sqrt(K)
    a = torch.from_numpy(rng.uniform(-lim, lim, (r, K)).astype(np.float32)).to(torch.bfloat16)
    b = torch.from_numpy((rng.standard_normal((N, r)) * 0.01).astype(np.float32)).to(torch.bfloat16)
    qt, qq, _ = _quant_both(q, w, kind, dq)
    Y, XA = q.qlora_linear_fwd(qq, to_dev(x), to_dev(a), to_dev(b), 16.0, return_xa=True)
    torch.cuda.synchronize()
    wd = oracle.dequantize(qt).reshape(N, K)
    y_ref, xa_ref = oracle.linear_fwd(wd, bf16_np(x), bf16_np(a), bf16_np(b), 16.0)
    assert_close("Y", bf16_np(Y), y_ref)
    assert_close("XA", bf16_np(XA), xa_ref)


def test_nf4_error_below_int4_on_device(q):
    """The pages' NF4-vs-INT4 claim on the device's own quantise/dequantise:
    mean squared error on N(0, 0.02) weights, equal to the oracle's."""
    say("variant error comparison")
    rng = np.random.default_rng(17)
    w = (rng.standard_normal((1024, 1024)) * 0.02).astype(np.float32)
    W = to_dev(w)
    err = {}
    for kind in ("nf4", "int4"):
        qq, _ = q.qlora_quantize_nf4(W, quant_type=kind)
        back = q.qlora_dequantize_nf4(qq, torch.float32)
        err[kind] = float(((back.double() - W.double()) ** 2).mean().item())
        ref = oracle.dequantize(oracle.quantize(w, kind=kind)).reshape(w.shape)
        assert abs(err[kind] - float(np.mean((ref.astype(np.float64) - w) ** 2))) <= 1e-12
    assert err["nf4"] < 0.9 * err["int4"]
