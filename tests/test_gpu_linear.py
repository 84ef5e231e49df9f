"""GPU parity of the fused forward and backward against the float64 oracle:
max|delta| <= 1e-2 * max|ref| + 1e-3 per output tensor, plus exact special
cases (one-hot rows pick bf16 columns of W'), ragged shapes, the decode path
and run-to-run determinism."""
import numpy as np
import pytest
import torch

from gpu_common import (DEV, assert_close, bf16_np, host, oracle, oracle_weight, say, to_dev,
                        workloads)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import bit_quantized_lora_quant_amd as q
    q.lib()
    return q


def _inputs(seed, M, N, K, r):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    lim = 1.0 / np.sqrt(K)
    a = torch.from_numpy(rng.uniform(-lim, lim, (r, K)).astype(np.float32)).to(torch.bfloat16)
    b = torch.from_numpy((rng.standard_normal((N, r)) * 0.01).astype(np.float32)).to(torch.bfloat16)
    dy = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(torch.bfloat16)
    return w, x, a, b, dy


def _check_layer(q, w, x, a, b, dy, alpha, label, use_xa=True, rows=None):
    """Runs fwd + bwd on the GPU and compares with the oracle (all rows, or
    the sampled `rows` of Y and dX; dA and dB always in full)."""
    say("linear %s M=%d N=%d K=%d r=%d" % (label, x.shape[0], w.shape[0], w.shape[1], a.shape[0]))
    qq, _ = q.qlora_quantize_nf4(to_dev(w))
    X, A, B, dY = to_dev(x), to_dev(a), to_dev(b), to_dev(dy)
    Y, XA = q.qlora_linear_fwd(qq, X, A, B, alpha, return_xa=True)
    dX, dA, dB = q.qlora_linear_bwd(qq, X, A, B, alpha, dY, XA_in=XA if use_xa else None)
    torch.cuda.synchronize()
    _, wd = oracle_weight(w)
    xf, af, bfl, dyf = bf16_np(x), bf16_np(a), bf16_np(b), bf16_np(dy)
    if rows is not None:
        y_ref, xa_ref = oracle.linear_fwd(wd, xf[rows], af, bfl, alpha)
        dx_ref, _, _ = oracle.linear_bwd(wd, xf[rows], af, bfl, alpha, dyf[rows])
        assert_close("Y", bf16_np(Y)[rows], y_ref)
        assert_close("XA", bf16_np(XA)[rows], xa_ref)
        assert_close("dX", bf16_np(dX)[rows], dx_ref)
        da_ref, db_ref = oracle.adapter_grads(xf, af, bfl, alpha, dyf)
    else:
        y_ref, xa_ref = oracle.linear_fwd(wd, xf, af, bfl, alpha)
        dx_ref, da_ref, db_ref = oracle.linear_bwd(wd, xf, af, bfl, alpha, dyf)
        assert_close("Y", bf16_np(Y), y_ref)
        assert_close("XA", bf16_np(XA), xa_ref)
        assert_close("dX", bf16_np(dX), dx_ref)
    assert_close("dA", host(dA).numpy(), da_ref)
    assert_close("dB", host(dB).numpy(), db_ref)
    return qq


def test_single_linear_1024(q):
    wl = workloads.SINGLE_1024
    w, x, a, b, dy = workloads.linear_inputs(wl, 0, 0)
    _check_layer(q, w, x, a, b, dy, wl.alpha, "single1024")
    _check_layer(q, w, x, a, b, dy, wl.alpha, "single1024-recompute-xa", use_xa=False)


RAGGED = [  # M, N, K, r
    (17, 64, 64, 1), (33, 100, 128, 8), (300, 192, 192, 16), (257, 300, 320, 64),
    (513, 520, 256, 5), (64, 1000, 640, 100), (40, 72, 128, 128), (2, 130, 192, 8),
    (16, 4096, 512, 64), (1, 77, 64, 3), (5, 640, 1024, 16), (600, 264, 64, 33),
    # few output tiles: the inner loop is split across workgroups, with uneven
    # slices (17 = 9 + 8, 65 = 7 x 9 + 2, 19 = 10 + 9 steps of 64)
    (300, 1216, 1088, 24), (70, 512, 4160, 16), (40, 4096, 256, 8),
    # decode path: partial last row tiles of the 4-wave (up to 4 tokens) and
    # 8-wave (5..16 tokens) streamers, ragged last inner ranges, block
    # counts that do not group by four (the per-block constant path)
    (7, 200, 320, 8), (16, 1000, 576, 64), (12, 129, 64, 3), (3, 65, 1088, 16),
    (16, 8, 4160, 32),
]


@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "M%d_N%d_K%d_r%d" % s)
def test_ragged_shapes(q, shape):
    M, N, K, r = shape
    w, x, a, b, dy = _inputs(hash(shape) & 0xFFFF, M, N, K, r)
    _check_layer(q, w, x, a, b, dy, 2.0 * r, "ragged")


@pytest.mark.parametrize("M", [1, 5, 16, 20, 300])
def test_one_hot_rows_pick_bf16_weight_columns(q, M):
    """B = 0 and X = one-hot rows: Y[m, :] must equal bf16(W'[:, k_m]) exactly
    (pins layouts, nibble order and the dequant inside the GEMM); with one-hot
    dY rows, dX[m, :] must equal bf16(W'[n_m, :]) exactly.

    The decode path (M <= 16) scales each block's dot products by the block
    constant after the MFMA, so its weights enter as float32(a * bf16(level)):
    there Y[m, n] must equal bf16(float32(a_(n, k_m) * bf16(level[code])))."""
    say("one-hot M=%d" % M)
    N, K, r = 320, 384, 8
    rng = np.random.default_rng(M)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    kk = rng.integers(0, K, size=M)
    nn = rng.integers(0, N, size=M)
    x = np.zeros((M, K), np.float32)
    x[np.arange(M), kk] = 1.0
    dy = np.zeros((M, N), np.float32)
    dy[np.arange(M), nn] = 1.0
    x = torch.from_numpy(x).to(torch.bfloat16)
    dy = torch.from_numpy(dy).to(torch.bfloat16)
    a = torch.from_numpy(rng.standard_normal((r, K)).astype(np.float32)).to(torch.bfloat16)
    b = torch.zeros((N, r), dtype=torch.bfloat16)
    qq, _ = q.qlora_quantize_nf4(to_dev(w))
    Y = q.qlora_linear_fwd(qq, to_dev(x), to_dev(a), to_dev(b), 16.0)
    dX, _, _ = q.qlora_linear_bwd(qq, to_dev(x), to_dev(a), to_dev(b), 16.0, to_dev(dy))
    torch.cuda.synchronize()
    qt, wd = oracle_weight(w)
    wb = oracle.to_bf16_bits(wd).reshape(N, K)
    y = host(Y).view(torch.int16).numpy().view(np.uint16)
    if M <= 16:
        lv = np.asarray(oracle.codebook(), dtype=np.float32)
        lvb = oracle.bf16_bits_to_f32(oracle.to_bf16_bits(lv)).astype(np.float32)
        codes = oracle.unpack_codes(qt["codes"], N * K).reshape(N, K)
        ahat = oracle.dequant_absmax(qt["absmax_q"], qt["absmax_scale"],
                                     qt["absmax_mean"]).astype(np.float32).reshape(N, K // 64)
        ycol = (ahat[:, kk // 64] * lvb[codes[:, kk]]).astype(np.float32)   # one fp32 rounding
        want = oracle.to_bf16_bits(ycol).reshape(ycol.shape).T
        assert np.array_equal(y, want), "Y rows are not a * bf16(level) of the weight columns"
    else:
        assert np.array_equal(y, wb.T[kk]), "Y rows are not the bf16 weight columns"
    dx = host(dX).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(dx, wb[nn]), "dX rows are not the bf16 weight rows"


def test_zero_weight_is_pure_lora(q):
    M, N, K, r = 70, 200, 256, 16
    w, x, a, b, dy = _inputs(77, M, N, K, r)
    w[:] = 0.0
    _check_layer(q, w, x, a, b, dy, 32.0, "zero-W")


def test_backward_deterministic(q):
    say("bwd determinism")
    M, N, K, r = 700, 1024, 1024, 16
    w, x, a, b, dy = _inputs(5, M, N, K, r)
    qq, _ = q.qlora_quantize_nf4(to_dev(w))
    X, A, B, dY = to_dev(x), to_dev(a), to_dev(b), to_dev(dy)
    r1 = q.qlora_linear_bwd(qq, X, A, B, 32.0, dY)
    r2 = q.qlora_linear_bwd(qq, X, A, B, 32.0, dY)
    y1 = q.qlora_linear_fwd(qq, X, A, B, 32.0)
    y2 = q.qlora_linear_fwd(qq, X, A, B, 32.0)
    torch.cuda.synchronize()
    for t1, t2 in zip(r1 + (y1,), r2 + (y2,)):
        assert torch.equal(t1, t2)


@pytest.mark.parametrize("tensor", [1, 6])
def test_llama8b_layer_linears_full(q, tensor):
    """Llama-3.1-8B linears (k_proj 4096->1024, down_proj 14336->4096) at the
    full 2048 tokens, r = 16, every output element compared."""
    wl = workloads.LLAMA8B_LAYER
    w, x, a, b, dy = workloads.linear_inputs(wl, 0, tensor)
    _check_layer(q, w, x, a, b, dy, wl.alpha, wl.linears[tensor][0])


@pytest.mark.parametrize("tensor", [0, 6])
def test_llama65b_linears_sampled(q, tensor):
    """LLaMA-65B linears (q_proj 8192->8192, down_proj 22016->8192) at 4096
    tokens, r = 64: 256 sampled rows of Y / XA / dX, dA and dB in full."""
    wl = workloads.LLAMA65B_LAYER
    w, x, a, b, dy = workloads.linear_inputs(wl, 0, tensor)
    rows = np.sort(np.random.default_rng(tensor).choice(wl.m, size=256, replace=False))
    _check_layer(q, w, x, a, b, dy, wl.alpha, wl.linears[tensor][0], rows=rows)


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("tensor", [1, 6])
def test_decode_gemv_70b(q, M, tensor):
    """70B-shaped decode forward (k_proj 8192->1024, down_proj 28672->8192)."""
    wl = workloads.LLAMA70B_DECODE
    w, x, a, b, _ = workloads.linear_inputs(wl, 0, tensor, m=M)
    say("decode M=%d %s" % (M, wl.linears[tensor][0]))
    qq, _ = q.qlora_quantize_nf4(to_dev(w))
    Y, XA = q.qlora_linear_fwd(qq, to_dev(x), to_dev(a), to_dev(b), wl.alpha, return_xa=True)
    torch.cuda.synchronize()
    _, wd = oracle_weight(w)
    y_ref, xa_ref = oracle.linear_fwd(wd, bf16_np(x), bf16_np(a), bf16_np(b), wl.alpha)
    assert_close("Y", bf16_np(Y), y_ref)
    assert_close("XA", bf16_np(XA), xa_ref)


def test_autograd_wrapper(q):
    say("autograd")
    M, N, K, r = 96, 256, 512, 8
    w, x, a, b, dy = _inputs(11, M, N, K, r)
    qq, _ = q.qlora_quantize_nf4(to_dev(w))
    X = to_dev(x).requires_grad_(True)
    A = to_dev(a).requires_grad_(True)
    B = to_dev(b).requires_grad_(True)
    Y = q.QLoRALinearFn.apply(X, A, B, qq, 16.0)
    Y.backward(to_dev(dy))
    torch.cuda.synchronize()
    _, wd = oracle_weight(w)
    dx_ref, da_ref, db_ref = oracle.linear_bwd(wd, bf16_np(x), bf16_np(a), bf16_np(b), 16.0,
                                               bf16_np(dy))
    assert_close("dX", bf16_np(X.grad), dx_ref)
    assert_close("dA", bf16_np(A.grad), da_ref)
    assert_close("dB", bf16_np(B.grad), db_ref)


def test_autograd_wrapper_with_dropout(q):
    """The autograd wrapper with dropout: the forward stores the keep bits and
    the backward reads them; gradients equal the oracle's under that mask."""
    say("autograd dropout")
    M, N, K, r = 96, 256, 512, 8
    w, x, a, b, dy = _inputs(12, M, N, K, r)
    qq, _ = q.qlora_quantize_nf4(to_dev(w))
    X = to_dev(x).requires_grad_(True)
    A = to_dev(a).requires_grad_(True)
    B = to_dev(b).requires_grad_(True)
    drop = (0.2, 31337)
    Y = q.QLoRALinearFn.apply(X, A, B, qq, 16.0, drop)
    Y.backward(to_dev(dy))
    torch.cuda.synchronize()
    _, wd = oracle_weight(w)
    y_ref, _ = oracle.linear_fwd(wd, bf16_np(x), bf16_np(a), bf16_np(b), 16.0, drop=drop)
    dx_ref, da_ref, db_ref = oracle.linear_bwd(wd, bf16_np(x), bf16_np(a), bf16_np(b), 16.0,
                                               bf16_np(dy), drop=drop)
    assert_close("Y", bf16_np(Y), y_ref)
    assert_close("dX", bf16_np(X.grad), dx_ref)
    assert_close("dA", bf16_np(A.grad), da_ref)
    assert_close("dB", bf16_np(B.grad), db_ref)
