"""The allocation-free quantiser entry point (qlora_quantize_nf4_noalloc,
scratch in the library's own device array) against the workspace entry point
(qlora_quantize_nf4), through the C ABI: the quantised state is identical bit
for bit on two calls in a row, the second with a smaller tensor (the array
keeps the first call's contents), the first also against the oracle; the
call allocates no device memory; and a tensor past the array's size is
refused with nothing launched."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_common import DEV, host, oracle, say, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import bit_quantized_lora_quant_amd as q
    q.lib()
    assert torch.cuda.is_available()
    return q


def _state(Q):
    return [host(t).numpy().view(np.uint8) for t in (Q.codes, Q.absmax_q, Q.absmax_scale,
                                                      Q.absmax_mean)]


def test_noalloc_equals_the_workspace_entry_point(q):
    lib = q.lib()
    stream = torch.cuda.current_stream().cuda_stream
    shapes = [(4096, 3072, 1), (300, 777, 2)]          # the second call is smaller
    Ws = [workloads.device_weight(9, 0, s, r, c) for r, c, s in shapes]
    ref = [q.qlora_quantize_nf4(W)[0] for W in Ws]
    got = [q.NF4Tensor(W.shape[0], W.shape[1], DEV) for W in Ws]
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for (rows, cols, _), W, Q in zip(shapes, Ws, got):
        say("noalloc quantise %dx%d" % (rows, cols))
        d = Q.descriptor()
        st = lib.qlora_quantize_nf4_noalloc(ctypes.c_void_p(W.data_ptr()), ctypes.byref(d),
                                            ctypes.c_void_p(stream))
        assert st == q.QLORA_OK, q.status_string(st)
        torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0, "the call allocated device memory"
    for (rows, cols, _), R, Q in zip(shapes, ref, got):
        for name, a, b in zip(("codes", "int8 constants", "scales", "mean"), _state(Q),
                              _state(R)):
            assert np.array_equal(a, b), "%s differ for %dx%d" % (name, rows, cols)
    qt = oracle.quantize(host(Ws[0]).numpy())
    assert np.array_equal(host(got[0].codes).numpy(), qt["codes"])
    assert np.array_equal(host(got[0].absmax_q).numpy(), qt["absmax_q"])


def test_noalloc_refuses_tensors_past_its_scratch(q):
    """2^29 + 64 weights need more than the fixed array: refused on the host
    (the fake buffers are never touched)."""
    lib = q.lib()
    fake = 0x100000
    d = q.NF4Descriptor((1 << 23) + 1, 64, 64, 256, fake, fake, fake, fake, 0, 0, 0)
    assert lib.qlora_quantize_nf4_noalloc(ctypes.c_void_p(fake), ctypes.byref(d), None) == \
        q.QLORA_ERR_UNSUPPORTED
