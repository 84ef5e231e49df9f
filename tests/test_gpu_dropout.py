"""GPU parity of the LoRA dropout against the oracle: the keep mask bit for bit
(the device's Philox4x32-10 against the oracle's own), the dropped forward
and backward within max|delta| <= 1e-2 * max|ref| + 1e-3 on ragged, split-K,
wide-rank and decode shapes, and two exact properties of the fused kernels:
elements the mask drops never reach the adapters, and p = 0 is the plain
layer bit for bit."""
import numpy as np
import pytest
import torch

from gpu_common import DEV, assert_close, bf16_np, host, oracle, oracle_weight, say, to_dev
from oracle import dropout as odrop

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import bit_quantized_lora_quant_amd as q
    q.lib()
    assert torch.cuda.is_available()
    return q


MASKS = [  # M, K, p, seed
    (1, 64, 0.5, 0), (3, 5, 0.3, 1), (7, 36, 0.3, 99), (300, 1088, 0.05, 2024),
    (2048, 4096, 0.1, 0x123456789ABCDEF0), (17, 4096, 0.9, 0xFFFFFFFF), (64, 640, 0.0, 5),
    (5, 1024, 1.0 - 2.0 ** -20, 77),
]


@pytest.mark.parametrize("M,K,p,seed", MASKS)
def test_mask_bit_exact(q, M, K, p, seed):
    say("dropout mask M=%d K=%d p=%r seed=%d" % (M, K, p, seed))
    got = host(q.qlora_dropout_mask(M, K, (p, seed), DEV)).numpy().astype(bool)
    ref = odrop.keep_mask(M, K, p, seed)
    assert np.array_equal(got, ref), "first differences at %s" % (np.argwhere(got != ref)[:8],)


def test_mask_at_an_odd_offset(q):
    """The tail of a mask whose length is not a multiple of 4, written at an
    address that is not 4-byte aligned."""
    say("dropout mask odd offset")
    buf = torch.zeros(1 + 7 * 37, dtype=torch.uint8, device=DEV)
    q.qlora_dropout_mask(7, 37, (0.4, 3), DEV, out=buf[1:].view(7, 37))
    got = host(buf).numpy()
    assert got[0] == 0
    assert np.array_equal(got[1:].reshape(7, 37).astype(bool), odrop.keep_mask(7, 37, 0.4, 3))


def _inputs(seed, M, N, K, r):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    lim = 1.0 / np.sqrt(K)
    a = torch.from_numpy(rng.uniform(-lim, lim, (r, K)).astype(np.float32)).to(torch.bfloat16)
    b = torch.from_numpy((rng.standard_normal((N, r)) * 0.05).astype(np.float32)).to(torch.bfloat16)
    dy = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).to(torch.bfloat16)
    return w, x, a, b, dy


LINEAR = [  # M, N, K, r, p
    (300, 1216, 1088, 24, 0.1),    # ragged M, split-K dX, r32 = 32
    (2048, 1024, 4096, 16, 0.05),  # split-K both ways, rank 16
    (257, 1000, 640, 100, 0.3),    # N % 64 != 0: the single-slice dX kernel; rank > 64
    (130, 1003, 192, 8, 0.5),      # N odd: element-wise dY tiles
    (600, 264, 64, 128, 0.2),      # widest rank
    (40, 4096, 256, 64, 0.1),      # few rows, many columns
    (8, 512, 1024, 16, 0.2),       # decode-path forward (keep bits from its slices), GEMM backward
]


@pytest.mark.parametrize("M,N,K,r,p", LINEAR, ids=lambda v: str(v))
def test_linear_fwd_bwd_with_dropout(q, M, N, K, r, p):
    seed = (M * 1000003 + N * 101 + K + r) & 0xFFFFFFFFFFFF
    say("dropout linear M=%d N=%d K=%d r=%d p=%r seed=%d" % (M, N, K, r, p, seed))
    w, x, a, b, dy = _inputs(seed & 0xFFFF, M, N, K, r)
    alpha = 2.0 * r
    qq, _ = q.qlora_quantize_nf4(to_dev(w))
    X, A, B, dY = to_dev(x), to_dev(a), to_dev(b), to_dev(dy)
    drop = (p, seed)
    bits = q.keep_bits_buffer(M, K, DEV)
    Y, XA = q.qlora_linear_fwd(qq, X, A, B, alpha, return_xa=True, dropout=drop, keep_bits=bits)
    dX, dA, dB = q.qlora_linear_bwd(qq, X, A, B, alpha, dY, XA_in=XA, dropout=drop)
    # the backward without the forward's XA regenerates the mask for it
    dX2, dA2, dB2 = q.qlora_linear_bwd(qq, X, A, B, alpha, dY, XA_in=None, dropout=drop)
    # reading the forward's stored bits instead gives the same bits
    dX3, dA3, dB3 = q.qlora_linear_bwd(qq, X, A, B, alpha, dY, XA_in=XA, dropout=drop,
                                       keep_bits=bits)
    dX4, dA4, dB4 = q.qlora_linear_bwd(qq, X, A, B, alpha, dY, XA_in=None, dropout=drop,
                                       keep_bits=bits)
    torch.cuda.synchronize()
    assert np.array_equal(host(bits).numpy(),
                          np.packbits(odrop.keep_mask(M, K, p, seed).reshape(-1),
                                      bitorder="little")), "stored keep bits"
    for u, v in ((dX, dX3), (dA, dA3), (dB, dB3), (dX2, dX4), (dA2, dA4), (dB2, dB4)):
        assert torch.equal(host(u), host(v))
    _, wd = oracle_weight(w)
    xf, af, bfl, dyf = bf16_np(x), bf16_np(a), bf16_np(b), bf16_np(dy)
    y_ref, xa_ref = oracle.linear_fwd(wd, xf, af, bfl, alpha, drop=drop)
    dx_ref, da_ref, db_ref = oracle.linear_bwd(wd, xf, af, bfl, alpha, dyf, drop=drop)
    assert_close("Y", bf16_np(Y), y_ref)
    assert_close("XA", bf16_np(XA), xa_ref)
    assert_close("dX", bf16_np(dX), dx_ref)
    assert_close("dA", host(dA).numpy(), da_ref)
    assert_close("dB", host(dB).numpy(), db_ref)
    assert_close("dX(recomputed XA)", bf16_np(dX2), dx_ref)
    assert_close("dA(recomputed XA)", host(dA2).numpy(), da_ref)
    assert_close("dB(recomputed XA)", host(dB2).numpy(), db_ref)
    # the LoRA share of dX carries the mask: where an element is dropped, dX
    # is the frozen product alone
    keep = odrop.keep_mask(M, K, p, seed)
    frozen = dyf @ wd.astype(np.float64)
    assert_close("dX at dropped elements", bf16_np(dX)[~keep], frozen[~keep])


@pytest.mark.parametrize("M", [1, 16])
def test_decode_with_dropout(q, M):
    N, K, r, p = 1024, 8192, 64, 0.1
    seed = 4242 + M
    say("dropout decode M=%d" % M)
    w, x, a, b, _ = _inputs(M, M, N, K, r)
    qq, _ = q.qlora_quantize_nf4(to_dev(w))
    bits = q.keep_bits_buffer(M, K, DEV)
    Y, XA = q.qlora_linear_fwd(qq, to_dev(x), to_dev(a), to_dev(b), 16.0, return_xa=True,
                               dropout=(p, seed), keep_bits=bits)
    torch.cuda.synchronize()
    assert np.array_equal(host(bits).numpy(),
                          np.packbits(odrop.keep_mask(M, K, p, seed).reshape(-1),
                                      bitorder="little")), "stored keep bits (decode)"
    _, wd = oracle_weight(w)
    y_ref, xa_ref = oracle.linear_fwd(wd, bf16_np(x), bf16_np(a), bf16_np(b), 16.0,
                                      drop=(p, seed))
    assert_close("Y", bf16_np(Y), y_ref)
    assert_close("XA", bf16_np(XA), xa_ref)


@pytest.mark.parametrize("M,N,K,r", [(300, 1216, 1088, 24), (8, 512, 1024, 16),
                                     (257, 1000, 640, 100)])
def test_dropped_elements_never_reach_the_adapters(q, M, N, K, r):
    """Changing X only where the device mask drops leaves XA, dA and dB bit
    for bit unchanged, and moves dX only through the frozen product."""
    p, seed = 0.3, 99 + M
    say("dropout invariance M=%d N=%d K=%d r=%d" % (M, N, K, r))
    w, x, a, b, dy = _inputs(M + K, M, N, K, r)
    qq, _ = q.qlora_quantize_nf4(to_dev(w))
    A, B, dY = to_dev(a), to_dev(b), to_dev(dy)
    keep = q.qlora_dropout_mask(M, K, (p, seed), DEV).bool()
    X1 = to_dev(x)
    X2 = torch.where(keep, X1, X1 * 3.0 + 1.0)
    out = []
    for X in (X1, X2):
        Y, XA = q.qlora_linear_fwd(qq, X, A, B, 8.0, return_xa=True, dropout=(p, seed))
        res = [XA]
        if M > 16:
            _, dA, dB = q.qlora_linear_bwd(qq, X, A, B, 8.0, dY, XA_in=None, need_dx=False,
                                           dropout=(p, seed))
            res += [dA, dB]
        out.append([host(t) for t in res])
    torch.cuda.synchronize()
    for u, v in zip(*out):
        assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u.view(torch.int32),
                           v.view(torch.int16) if v.dtype == torch.bfloat16 else v.view(torch.int32))


@pytest.mark.parametrize("M", [8, 300])
def test_zero_probability_is_the_plain_layer(q, M):
    N, K, r = 1216, 1088, 24
    say("dropout p=0 M=%d" % M)
    w, x, a, b, dy = _inputs(M, M, N, K, r)
    qq, _ = q.qlora_quantize_nf4(to_dev(w))
    X, A, B, dY = to_dev(x), to_dev(a), to_dev(b), to_dev(dy)
    plain = list(q.qlora_linear_fwd(qq, X, A, B, 48.0, return_xa=True))
    dropped = list(q.qlora_linear_fwd(qq, X, A, B, 48.0, return_xa=True, dropout=(0.0, 1)))
    if M > 16:
        plain += list(q.qlora_linear_bwd(qq, X, A, B, 48.0, dY))
        dropped += list(q.qlora_linear_bwd(qq, X, A, B, 48.0, dY, dropout=(0.0, 1)))
    torch.cuda.synchronize()
    for u, v in zip(plain, dropped):
        assert torch.equal(host(u), host(v))


def test_probability_below_the_generator_resolution_is_no_dropout(q):
    """p below 2^-32 gives threshold 0 (every word keeps): the plain layer bit
    for bit."""
    M, N, K, r = 64, 256, 512, 8
    say("dropout p=1e-12")
    w, x, a, b, dy = _inputs(3, M, N, K, r)
    qq, _ = q.qlora_quantize_nf4(to_dev(w))
    X, A, B, dY = to_dev(x), to_dev(a), to_dev(b), to_dev(dy)
    plain = list(q.qlora_linear_fwd(qq, X, A, B, 16.0, return_xa=True))
    plain += list(q.qlora_linear_bwd(qq, X, A, B, 16.0, dY))
    tiny = list(q.qlora_linear_fwd(qq, X, A, B, 16.0, return_xa=True, dropout=(1e-12, 5)))
    tiny += list(q.qlora_linear_bwd(qq, X, A, B, 16.0, dY, dropout=(1e-12, 5)))
    torch.cuda.synchronize()
    for u, v in zip(plain, tiny):
        assert torch.equal(host(u), host(v))
