"""GPU parity of the AdamW step with 8-bit statistics against the oracle
(oracle/adamw.py, adamw8_step).  The codes are decided in float32 on both
sides, with one IEEE rounding per operation in the same order, so every
output is compared bit for bit: the float32 weights, the int8 / uint8 codes,
the float32 block scales and the bf16 copy, over several steps, for the
state in device memory and in mapped host memory, for more tensors than one
launch carries, and on the element-wise path (unaligned tensors)."""
import numpy as np
import pytest
import torch

from gpu_common import DEV, host, oracle, say
from oracle.adamw import adamw8_step

pytestmark = pytest.mark.gpu

HP = dict(lr=2e-4, b1=0.9, b2=0.999, eps=1e-8, wd=0.01)


@pytest.fixture(scope="module")
def q():
    import bit_quantized_lora_quant_amd as q
    q.lib()
    assert torch.cuda.is_available()
    return q


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def _run(q, sizes, steps, host_state=False, offset=0, seed=0):
    """`steps` steps over tensors of `sizes` on the device and in the oracle;
    asserts bit equality after every step.  offset > 0 starts every device
    tensor `offset` elements into its buffer (the element-wise path)."""
    rng = np.random.default_rng(seed)
    dev_t, ora = [], []
    for i, n in enumerate(sizes):
        p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
        pbuf = torch.zeros(n + offset, dtype=torch.float32, device=DEV)
        p = pbuf[offset:]
        p.copy_(torch.from_numpy(p0))
        gbuf = torch.zeros(n + offset, dtype=torch.float32, device=DEV)
        pbb = torch.zeros(n + offset, dtype=torch.bfloat16, device=DEV)
        on_host = host_state[i] if isinstance(host_state, (list, tuple)) else host_state
        st = q.AdamW8State(n, DEV, host=on_host)
        dev_t.append((p, gbuf, st, pbb[offset:], offset))
        z = (n + 255) // 256
        ora.append([p0, np.zeros(n, np.int8), np.zeros(z, np.float32), np.zeros(n, np.uint8),
                    np.zeros(z, np.float32)])
    for t in range(1, steps + 1):
        say("adamw8 sizes=%s step=%d host=%s offset=%d" % (sizes[:6], t, host_state, offset))
        gs = [(rng.standard_normal(n) * 10.0 ** rng.uniform(-5, -2)).astype(np.float32)
              for n in sizes]
        for (p, gbuf, st, pb, off), g in zip(dev_t, gs):
            gbuf[off:].copy_(torch.from_numpy(g))
        q.qlora_adamw8_step([(p, gbuf[off:], st, pb) for p, gbuf, st, pb, off in dev_t], t,
                            HP["lr"], HP["b1"], HP["b2"], HP["eps"], HP["wd"])
        torch.cuda.synchronize()
        for i, g in enumerate(gs):
            ora[i] = list(adamw8_step(*ora[i][:1], g, *ora[i][1:], t, HP["lr"], HP["b1"],
                                      HP["b2"], HP["eps"], HP["wd"]))
            p, _, st, pb, _ = dev_t[i]
            got = [host(p).numpy(), host(st.m_q).numpy(), host(st.m_scale).numpy(),
                   host(st.v_q).numpy(), host(st.v_scale).numpy()]
            for name, a, b in zip(("param", "m codes", "m scales", "v codes", "v scales"),
                                  got, ora[i]):
                assert np.array_equal(_bits(a), _bits(b)), \
                    "%s differs (tensor %d, n=%d, step %d) at %s" % (
                        name, i, sizes[i], t, np.nonzero(_bits(a) != _bits(b))[0][:8])
            pbh = host(pb).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(pbh, oracle.to_bf16_bits(ora[i][0])), "bf16 copy"


SIZES = [1, 3, 255, 256, 257, 1000, 1024, 4099, 65536 + 17]


def test_bit_exact_over_steps(q):
    _run(q, SIZES, steps=4)


def test_host_resident_state(q):
    _run(q, [256, 1000, 70001], steps=3, host_state=True, seed=1)


def test_statistics_split_by_an_hbm_budget(q):
    """Half the statistics' bytes in HBM, the rest mapped from host memory, in
    one launch: the placement changes no bit."""
    sizes = [70001, 256, 4099, 1000, 65536 + 17, 3, 30000]
    need = sum(q.adamw8_state_bytes(n) for n in sizes)
    flags = q.plan_state_placement([q.adamw8_state_bytes(n) for n in sizes], need // 2)
    assert any(flags) and not all(flags)
    states = q.adamw8_states(sizes, DEV, hbm_budget=need // 2)
    assert [st.on_host for st in states] == flags
    for st in states:
        st.free()
    _run(q, sizes, steps=3, host_state=flags, seed=4)


def test_more_tensors_than_one_launch(q):
    sizes = [int(s) for s in np.random.default_rng(2).integers(1, 3000, size=60)]
    _run(q, sizes, steps=2, seed=2)


def test_unaligned_tensors_take_the_elementwise_path(q):
    _run(q, [300, 1024, 5000], steps=3, offset=1, seed=3)


def test_zero_learning_rate_keeps_the_weights(q):
    say("adamw8 lr=0")
    n = 5000
    p = torch.randn(n, device=DEV)
    p0 = p.clone()
    g = torch.randn(n, device=DEV)
    st = q.AdamW8State(n, DEV)
    for t in (1, 2):
        q.qlora_adamw8_step([(p, g, st, None)], t, 0.0, 0.9, 0.999, 1e-8, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(p, p0)
    assert int(st.m_q.abs().max()) == 127 and int(st.v_q.max()) == 255


def test_argument_errors(q):
    n = 10
    p = torch.zeros(n, device=DEV)
    st = q.AdamW8State(n, DEV)
    with pytest.raises(q.QloraError):
        q.qlora_adamw8_step([(p, p, st, None)], 0, 1e-3)          # step starts at 1
    with pytest.raises(q.QloraError):
        q.qlora_adamw8_step([(p, p, st, None)], 1, 1e-3, beta1=1.0)
