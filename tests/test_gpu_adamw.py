"""GPU parity of the adapter optimiser step against the oracle's AdamW:
master weights and both statistics within a float32 bound over three steps
(max|delta| <= 2e-6 * max|ref| + 1e-12, six roundings a step in float32
against float64), the bf16 copy bit for bit against the device's own float32
result, and exact agreements between the kernel's own paths: unaligned
tensors (element-wise) against aligned ones (vector), several launches
(more than 64 tensors), and statistics in mapped host memory against
statistics in device memory."""
import numpy as np
import pytest
import torch

from gpu_common import DEV, host, say
from oracle.adamw import adamw_step

pytestmark = pytest.mark.gpu

HP = dict(lr=2e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.fixture(scope="module")
def q():
    import bit_quantized_lora_quant_amd as q
    q.lib()
    assert torch.cuda.is_available()
    return q


def _bound(ref):
    return 2e-6 * float(np.max(np.abs(ref))) + 1e-12 if ref.size else 0.0


def _close(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert err <= _bound(ref), "%s: max|delta| %.3g > %.3g" % (name, err, _bound(ref))


def _tensors(sizes, seed):
    rng = np.random.default_rng(seed)
    out = []
    for n in sizes:
        p = (rng.standard_normal(n) * 0.05).astype(np.float32)
        m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        v = (np.abs(rng.standard_normal(n)) * 1e-6).astype(np.float32)
        grads = [(rng.standard_normal(n) * 1e-2).astype(np.float32) for _ in range(3)]
        out.append((p, m, v, grads))
    return out


def _run(q, host_tensors, steps, host_states=False, offset=0):
    """Runs `steps` AdamW steps on the device; returns per tensor (p, m, v,
    bf16 copy) after the last step.  offset > 0 places every tensor that many
    floats past an aligned address (the element-wise path)."""
    keep = []
    dev = []
    for p, m, v, grads in host_tensors:
        n = p.size

        def place(a, dtype=torch.float32, on_host=False):
            if on_host:
                hs = q.qlora_host_state_alloc(n + offset)
                keep.append(hs)
                t = hs.tensor[offset:]
                t.copy_(torch.from_numpy(a))
                return t
            buf = torch.empty(n + offset, dtype=dtype, device=DEV)
            t = buf[offset:]
            t.copy_(torch.from_numpy(a).to(DEV))
            return t

        P = place(p)
        M = place(m, on_host=host_states)
        V = place(v, on_host=host_states)
        G = [place(g) for g in grads]
        PB = torch.empty(n + offset, dtype=torch.bfloat16, device=DEV)[offset:]
        dev.append((P, M, V, G, PB))
    for t in range(1, steps + 1):
        q.qlora_adamw_step([(P, G[t - 1], M, V, PB) for P, M, V, G, PB in dev], t, **HP)
    torch.cuda.synchronize()
    res = [(host(P).numpy().copy(), host(M).numpy().copy(), host(V).numpy().copy(),
            host(PB.view(torch.int16)).numpy().copy()) for P, M, V, G, PB in dev]
    del keep
    return res


def _oracle(host_tensors, steps):
    out = []
    for p, m, v, grads in host_tensors:
        P, M, V = p.astype(np.float64), m.astype(np.float64), v.astype(np.float64)
        for t in range(1, steps + 1):
            P, M, V = adamw_step(P, grads[t - 1], M, V, t, HP["lr"], HP["beta1"], HP["beta2"],
                                 HP["eps"], HP["weight_decay"])
        out.append((P, M, V))
    return out


SIZES = [1, 3, 4095, 4096, 4097, 65536 + 5, 0, 16 * 4096]


def test_step_matches_oracle(q):
    say("adamw oracle parity sizes=%s" % SIZES)
    ht = _tensors(SIZES, 1)
    got = _run(q, ht, 3)
    for i, ((p, m, v, pb), (P, M, V)) in enumerate(zip(got, _oracle(ht, 3))):
        _close("p[%d]" % i, p, P)
        _close("m[%d]" % i, m, M)
        _close("v[%d]" % i, v, V)
        # the bf16 copy is the device's own float32 result rounded to nearest even
        ref16 = torch.from_numpy(p).to(torch.bfloat16).view(torch.int16).numpy()
        assert np.array_equal(pb, ref16), "bf16 copy of tensor %d" % i


def test_one_llama8b_layer_of_adapters(q):
    """The 14 adapter tensors of one Llama-3.1-8B layer at r = 16 (1.31M
    parameters)."""
    say("adamw 8B layer adapters")
    shapes = [(16, 4096), (4096, 16), (16, 4096), (1024, 16), (16, 4096), (1024, 16),
              (16, 4096), (4096, 16), (16, 4096), (14336, 16), (16, 4096), (14336, 16),
              (16, 14336), (4096, 16)]
    ht = _tensors([a * b for a, b in shapes], 2)
    assert sum(p.size for p, _, _, _ in ht) == 1310720
    got = _run(q, ht, 2)
    for i, ((p, m, v, _), (P, M, V)) in enumerate(zip(got, _oracle(ht, 2))):
        _close("p[%d]" % i, p, P)
        _close("m[%d]" % i, m, M)
        _close("v[%d]" % i, v, V)


def test_many_tensors_take_several_launches(q):
    sizes = [int(s) for s in np.random.default_rng(3).integers(0, 9000, 113)]
    say("adamw 113 tensors")
    ht = _tensors(sizes, 3)
    got = _run(q, ht, 2)
    for i, ((p, m, v, _), (P, M, V)) in enumerate(zip(got, _oracle(ht, 2))):
        _close("p[%d]" % i, p, P)
        _close("m[%d]" % i, m, M)
        _close("v[%d]" % i, v, V)


def test_unaligned_tensors_equal_aligned(q):
    """The element-wise path (pointers off 16-byte alignment) gives the same
    bits as the vector path."""
    say("adamw unaligned")
    ht = _tensors([4096 * 3, 5000], 4)
    a = _run(q, ht, 2)
    b = _run(q, ht, 2, offset=1)
    for x, y in zip(a, b):
        for u, w in zip(x, y):
            assert np.array_equal(u.view(np.int32) if u.dtype == np.float32 else u,
                                  w.view(np.int32) if w.dtype == np.float32 else w)


def test_host_resident_statistics_equal_device_resident(q):
    """Statistics in mapped host memory: same kernel, same bits."""
    say("adamw host-resident statistics")
    ht = _tensors([4096 * 5, 777, 65536], 5)
    a = _run(q, ht, 3)
    b = _run(q, ht, 3, host_states=True)
    for x, y in zip(a, b):
        for u, w in zip(x, y):
            assert np.array_equal(u, w)


def test_argument_errors(q):
    say("adamw argument errors")
    import ctypes
    P = torch.zeros(8, device=DEV)
    arr = (q.AdamWTensor * 1)(q.AdamWTensor(P.data_ptr(), P.data_ptr(), P.data_ptr(),
                                            P.data_ptr(), None, 8))
    lib = q.lib()
    for h in (q.AdamWHparams(-1.0, 0.9, 0.999, 1e-8, 0.0), q.AdamWHparams(1e-3, 1.0, 0.999, 1e-8, 0.0),
              q.AdamWHparams(1e-3, 0.9, 0.999, 0.0, 0.0), q.AdamWHparams(1e-3, 0.9, 0.999, 1e-8, -1.0)):
        assert lib.qlora_adamw_step(ctypes.byref(h), 1, arr, 1, None) == q.QLORA_ERR_INVALID_ARG
    ok = q.AdamWHparams(1e-3, 0.9, 0.999, 1e-8, 0.0)
    assert lib.qlora_adamw_step(ctypes.byref(ok), 0, arr, 1, None) == q.QLORA_ERR_INVALID_ARG
    bad = (q.AdamWTensor * 1)(q.AdamWTensor(P.data_ptr() + 2, P.data_ptr(), P.data_ptr(),
                                            P.data_ptr(), None, 4))
    assert lib.qlora_adamw_step(ctypes.byref(ok), 1, bad, 1, None) == q.QLORA_ERR_INVALID_ARG


def test_zero_learning_rate_keeps_the_weights(q):
    """lr = 0: the weights (and their bf16 copy) stay bit for bit while both
    statistics move as the oracle's."""
    say("adamw lr=0")
    rng = np.random.default_rng(21)
    n = 9000
    p = (rng.standard_normal(n) * 0.05).astype(np.float32)
    g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
    P, G = torch.from_numpy(p).to(DEV), torch.from_numpy(g).to(DEV)
    M, V = torch.zeros(n, device=DEV), torch.zeros(n, device=DEV)
    PB = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    q.qlora_adamw_step([(P, G, M, V, PB)], 1, 0.0, weight_decay=0.1)
    torch.cuda.synchronize()
    assert np.array_equal(host(P).numpy().view(np.int32), p.view(np.int32))
    assert torch.equal(host(PB), torch.from_numpy(p).to(torch.bfloat16))
    _, m_ref, v_ref = adamw_step(p, g, np.zeros(n), np.zeros(n), 1, 0.0, 0.9, 0.999, 1e-8, 0.1)
    _close("m", host(M).numpy(), m_ref)
    _close("v", host(V).numpy(), v_ref)
