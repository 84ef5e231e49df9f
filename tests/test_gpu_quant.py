"""GPU parity: NF4 quantisation, double quantisation and dequantisation must
match the oracle bit for bit (codes, exact absmax, int8 constants, scales,
mean, reconstructed constants, float32 and bf16 dequantised weights)."""
import numpy as np
import pytest
import torch

from gpu_common import (DEV, compare_quant_state, host, oracle, say, to_dev, workloads)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import bit_quantized_lora_quant_amd as q
    q.lib()
    assert torch.cuda.is_available()
    return q


def _roundtrip(q, w_np, check_dequant=True):
    n = w_np.size
    qt = oracle.quantize(w_np)
    qq, ws = q.qlora_quantize_nf4(to_dev(w_np))
    torch.cuda.synchronize()
    compare_quant_state(qq, ws, qt, n)
    if check_dequant:
        ahat = oracle.dequant_absmax(qt["absmax_q"], qt["absmax_scale"], qt["absmax_mean"])
        got_a = host(q.qlora_dequantize_absmax(qq)).numpy()
        assert np.array_equal(got_a.view(np.uint32), ahat.view(np.uint32)), "reconstructed absmax"
        wd = oracle.dequantize(qt)
        f32 = host(q.qlora_dequantize_nf4(qq, torch.float32)).numpy().reshape(-1)
        assert np.array_equal(f32.view(np.uint32), wd.view(np.uint32)), "fp32 dequant at %s" % (
            np.nonzero(f32.view(np.uint32) != wd.view(np.uint32))[0][:8],)
        b16 = host(q.qlora_dequantize_nf4(qq, torch.bfloat16)).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(b16.reshape(-1), oracle.to_bf16_bits(wd)), "bf16 dequant"
    return qq


SHAPES = [(1, 1), (1, 7), (3, 5), (1, 64), (1, 65), (2, 100), (7, 64 * 5 + 3), (64, 64),
          (100, 1000), (257, 255), (1024, 1024), (333, 4096)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%dx%d" % s)
def test_quantize_dequant_bit_exact(q, shape):
    say("quant %s" % (shape,))
    rng = np.random.default_rng(shape[0] * 7919 + shape[1])
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    _roundtrip(q, w)


def test_levels_round_trip(q):
    say("quant level round trip")
    cb = oracle.codebook()
    idx = np.tile(np.arange(16), 4 * 600)
    for e in (-6, -1, 0, 2):
        w = (cb[idx] * np.float32(2.0 ** e)).reshape(600, 64)
        qq = _roundtrip(q, w)
        back = host(q.qlora_dequantize_nf4(qq, torch.float32)).numpy()
        assert np.array_equal(back.view(np.uint32), w.view(np.uint32))


def test_zero_and_midpoint_blocks(q):
    say("quant zero + midpoints")
    cb = oracle.codebook().astype(np.float64)
    w = np.zeros((40, 64), dtype=np.float32)
    w[5:7] = -0.0
    row = 10
    for j in range(15):
        m = (cb[j] + cb[j + 1]) / 2.0
        f = np.float32(m)
        lo = f if float(f) <= m else np.nextafter(f, np.float32(-2))
        w[row, 2 * j] = lo
        w[row, 2 * j + 1] = np.nextafter(lo, np.float32(2))
    w[row, 63] = 1.0
    w[20:] = np.random.default_rng(5).uniform(-1, 1, size=(20, 64)).astype(np.float32)
    _roundtrip(q, w)


def test_heavy_tailed_and_wide_range(q):
    """Constants spanning many magnitudes exercise the int8 clamp, negative
    reconstructed constants and the float64 tree sum."""
    say("quant wide range")
    rng = np.random.default_rng(9)
    w = (rng.standard_cauchy((512, 512)) * 0.01).astype(np.float32)
    w[:10] *= np.float32(1e6)
    w[10:20] *= np.float32(1e-6)
    _roundtrip(q, w)


@pytest.mark.parametrize("consts,mean", [
    ([4.0, 2.0 ** -22, 2.0 ** -51, 2.0 ** -51], 1.0 + 2.0 ** -23),   # tree != left to right
    ([4.0, 2.0 ** -51, 2.0 ** -22, 2.0 ** -51], 1.0),                # tree != exact mean
    ([5.0, 5.0 * 2.0 ** -24, 2.0 ** -51, 2.0 ** -51, 0.0], 1.0 + 2.0 ** -23),   # padded tree
], ids=["left-to-right", "exact", "padded"])
def test_mean_tree_order_constants(q, consts, mean):
    """Blocks whose absmax are constants at which the adjacent-pair float64
    tree, a left-to-right sum and the exact mean round to different float32
    means (worked out by hand in the oracle's pins): the device's mean is
    the tree's, and the whole state matches the oracle."""
    say("quant tree-order constants %s" % (consts,))
    w = np.zeros((len(consts), 64), dtype=np.float32)
    w[:, 0] = consts
    w[:, 1] = -np.float32(0.5) * np.asarray(consts, dtype=np.float32)
    _roundtrip(q, w)
    assert oracle.quantize(w)["absmax_mean"] == np.float32(mean)


def test_blocks_dequantise_with_the_rebuilt_constant(q):
    """The oracle pin's double-quantisation block on the device: absmax 1 +-
    2^-9 rebuild to exactly 1, so those blocks dequantise to the bare levels."""
    say("quant rebuilt-constant blocks")
    cb = oracle.codebook()
    a = np.ones(256, dtype=np.float64)
    a[0], a[1], a[2], a[3] = 1 + 127 / 128, 1 / 128, 1 + 2.0 ** -9, 1 - 2.0 ** -9
    idx = np.tile(np.arange(16), 4)
    w = np.stack([(cb[idx].astype(np.float64) * a_b).astype(np.float32) for a_b in a])
    qq = _roundtrip(q, w)
    back = host(q.qlora_dequantize_nf4(qq, torch.float32)).numpy().reshape(256, 64)
    assert np.array_equal(back[2], cb[idx]) and np.array_equal(back[3], cb[idx])


def test_deterministic_repeat(q):
    say("quant determinism")
    w = to_dev((np.random.default_rng(3).standard_normal((512, 2048)) * 0.02).astype(np.float32))
    a, _ = q.qlora_quantize_nf4(w)
    b, _ = q.qlora_quantize_nf4(w)
    torch.cuda.synchronize()
    for t1, t2 in ((a.codes, b.codes), (a.absmax_q, b.absmax_q), (a.absmax_scale, b.absmax_scale),
                   (a.absmax_mean, b.absmax_mean)):
        assert torch.equal(t1, t2)


@pytest.mark.parametrize("which", ["embed_tokens", "down_proj"])
def test_full_weight_set_tensors(q, which):
    """Full-size tensors of the 8.03B-parameter weight set (drawn on the
    device), every output compared: the embedding (525M weights, three tree
    passes for the mean) and one down projection."""
    spec = [s for s in workloads.llama8b_weight_set() if s[0] == which][0]
    name, layer, rows, cols = spec
    say("full tensor %s %dx%d" % (name, rows, cols))
    w = workloads.device_weight(2, layer, 0 if name == "embed_tokens" else 6, rows, cols)
    qq, ws = q.qlora_quantize_nf4(w)
    torch.cuda.synchronize()
    w_np = host(w).numpy()
    del w
    qt = oracle.quantize(w_np)
    compare_quant_state(qq, ws, qt, w_np.size)
    del ws
    wd = oracle.dequantize(qt)
    out = q.qlora_dequantize_nf4(qq, torch.bfloat16)
    b16 = host(out).view(torch.int16).numpy().view(np.uint16).reshape(-1)
    assert np.array_equal(b16, oracle.to_bf16_bits(wd))
    del out
    f32 = host(q.qlora_dequantize_nf4(qq, torch.float32)).numpy().reshape(-1)
    assert np.array_equal(f32.view(np.uint32), wd.view(np.uint32))
    bits = 8.0 * qq.nbytes() / (rows * cols)
    assert abs(bits - 4.127) < 1e-3


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kind", ["nf4", "int4"])
def test_every_float_in_the_unit_interval(q, kind):
    """Exhaustive: every float32 in [-1, 1] (all 2 x 1,065,353,217 bit patterns
    from +-0 to +-1) quantised on the device inside blocks whose absmax is
    exactly 1, so the quantiser's input is the value itself; the codes (NF4
    and INT4 tables) equal the oracle's nearest-level codes (ties to the lower
    level) for every one of them."""
    total = 0x3F800001                      # patterns 0x00000000 .. 0x3F800000
    per_block = 63                          # the 64th element of a block is 1.0
    nb = 1 << 22                            # blocks per chunk (264M values)
    chunk = per_block * nb
    Q = q.NF4Tensor(nb, 64, DEV, kind, False)
    ws = q.workspace(q.qlora_quantize_workspace_bytes(nb, 64), DEV)
    host_w = np.ones((nb, 64), dtype=np.float32)
    for sign in (0, 0x80000000):
        for start in range(0, total, chunk):
            n = min(chunk, total - start)
            say("exhaustive %s sign=%x start=%d n=%d" % (kind, sign, start, n))
            buf = np.zeros(chunk, dtype=np.uint32)
            buf[:n] = np.arange(start, start + n, dtype=np.uint32) | np.uint32(sign)
            host_w[:, :per_block] = buf.view(np.float32).reshape(nb, per_block)
            W = torch.from_numpy(host_w).to(DEV)
            q.qlora_quantize_nf4(W, Q, ws)
            codes = host(Q.codes).numpy()
            ref = oracle.quantize(host_w.reshape(-1), kind=kind, dq=False)["codes"]
            assert np.array_equal(codes, ref), "codes differ in chunk at %d (sign %x)" % (start, sign)
            del W


@pytest.mark.parametrize("kind", ["nf4", "int4"])
def test_quotients_next_to_thresholds(q, kind):
    """Weights within two ulps of threshold x absmax, in blocks whose absmax
    (first element, either sign) is drawn log-uniformly over 2^-70 .. 2^70:
    the code decision w / absmax > threshold, taken on the device through a
    per-block reciprocal with a residual correction (or the division, for
    absmax outside 2^+-60), equals the oracle's IEEE division for every one."""
    rng = np.random.default_rng(17 if kind == "nf4" else 18)
    cb = oracle.codebook(kind).astype(np.float64)
    thr = (cb[:-1] + cb[1:]) / 2.0
    thr = thr[np.abs(thr) < 1.0]
    nb = 1 << 16
    a = np.exp2(rng.uniform(-70, 70, nb)).astype(np.float32)
    a *= np.where(rng.random(nb) < 0.5, -1, 1).astype(np.float32)
    w = np.empty((nb, 64), dtype=np.float32)
    w[:, 0] = a
    t = rng.choice(thr, size=(nb, 63))
    x = (t * np.abs(a)[:, None].astype(np.float64)).astype(np.float32)
    bits = x.view(np.int32) + rng.integers(-2, 3, size=x.shape).astype(np.int32)
    x = bits.view(np.float32)
    x = np.where(np.abs(x) <= np.abs(a)[:, None], x, np.float32(0))
    w[:, 1:] = x
    say("quotients next to thresholds %s" % kind)
    qq, _ = q.qlora_quantize_nf4(to_dev(w), quant_type=kind, double_quant=False)
    torch.cuda.synchronize()
    ref = oracle.quantize(w.reshape(-1), kind=kind, dq=False)["codes"]
    got = host(qq.codes).numpy()
    assert np.array_equal(got, ref), "codes differ at bytes %s" % (np.nonzero(got != ref)[0][:8],)
