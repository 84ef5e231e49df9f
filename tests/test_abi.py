"""The C-ABI library on the host (no GPU needed): it loads, exports every
function include/qlora_nf4.h declares, its codebook equals the oracle's bit for
bit, and argument errors come back as status codes before anything is
launched."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora_nf4.h")


@pytest.fixture(scope="module")
def q():
    import bit_quantized_lora_quant_amd as q
    if not os.path.exists(q.LIB_PATH):
        from bit_quantized_lora_quant_amd import build
        build.build()
    return q


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("qlora_quantize_nf4", "qlora_dequantize_nf4", "qlora_linear_fwd", "qlora_linear_bwd"):
        assert n in names


def test_library_exports_every_declared_symbol(q):
    lib = q.lib()
    names = declared_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(q.EXPORTS) == names


def test_codebook_matches_oracle_bit_exact(q):
    lib_cb = np.array(q.qlora_nf4_codebook(), dtype=np.float32)
    assert np.array_equal(lib_cb.view(np.uint32), oracle.codebook().view(np.uint32))


def test_int4_codebook_matches_oracle_bit_exact(q):
    lib_cb = np.array(q.qlora_codebook("int4"), dtype=np.float32)
    assert np.array_equal(lib_cb.view(np.uint32), oracle.codebook("int4").view(np.uint32))
    nf4 = np.array(q.qlora_codebook("nf4"), dtype=np.float32)
    assert np.array_equal(nf4.view(np.uint32), oracle.codebook().view(np.uint32))
    buf = (ctypes.c_float * 16)()
    assert q.lib().qlora_codebook(2, buf) == q.QLORA_ERR_INVALID_ARG
    assert q.lib().qlora_codebook(0, None) == q.QLORA_ERR_INVALID_ARG


def test_descriptor_type_and_constant_fields(q):
    """dq_block 0 needs the float32 absmax buffer (and then not the 8-bit
    state); the type must be NF4 or INT4 and the reserved field zero.  A
    descriptor that passes validation gets as far as the workspace check."""
    lib = q.lib()
    P = ctypes.c_void_p
    fake = 0x100000

    def quant(d):
        return lib.qlora_quantize_nf4(P(0x200000), ctypes.byref(d), P(0x300000), 16, None)

    ok = q.NF4Descriptor(64, 64, 64, 0, fake, 0, 0, 0, fake, 1, 0)
    assert quant(ok) == q.QLORA_ERR_WORKSPACE
    for bad in (q.NF4Descriptor(64, 64, 64, 0, fake, fake, fake, fake, 0, 0, 0),
                q.NF4Descriptor(64, 64, 64, 256, fake, fake, fake, fake, 0, 2, 0),
                q.NF4Descriptor(64, 64, 64, 256, fake, fake, fake, fake, 0, 0, 1),
                q.NF4Descriptor(64, 64, 64, 256, fake, 0, fake, fake, fake, 0, 0)):
        assert quant(bad) == q.QLORA_ERR_INVALID_ARG


def test_status_strings(q):
    for s in range(5):
        assert q.status_string(s)
    assert q.status_string(0) == "ok"


def test_workspace_queries(q):
    assert q.qlora_quantize_workspace_bytes(0, 5) == 0
    assert q.qlora_quantize_workspace_bytes(1024, 1024) >= (1024 * 1024 // 64) * 4
    assert q.qlora_linear_workspace_bytes(128, 1024, 1024, 0) == 0
    assert q.qlora_linear_workspace_bytes(128, 1024, 1024, 129) == 0
    a = q.qlora_linear_workspace_bytes(128, 1024, 1024, 8)
    b = q.qlora_linear_workspace_bytes(2048, 4096, 14336, 16)
    assert 0 < a < b


def _desc(q, rows=64, cols=64, block=64, dq=256, null_codes=False):
    fake = 0x100000  # never dereferenced: validation fails first or shapes are checked
    return q.NF4Descriptor(rows, cols, block, dq, 0 if null_codes else fake, fake, fake, fake)


def test_argument_errors_return_status(q):
    lib = q.lib()
    P = ctypes.c_void_p
    # bad descriptors
    for d in (_desc(q, block=32), _desc(q, dq=128), _desc(q, rows=0), _desc(q, null_codes=True)):
        assert lib.qlora_dequantize_nf4(ctypes.byref(d), q.QLORA_F32, P(0x200000), None) == \
            q.QLORA_ERR_INVALID_ARG
    d = _desc(q)
    # null weight / null output
    assert lib.qlora_quantize_nf4(None, ctypes.byref(d), P(0x200000), 1 << 20, None) == \
        q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_dequantize_nf4(ctypes.byref(d), q.QLORA_F32, None, None) == \
        q.QLORA_ERR_INVALID_ARG
    # workspace too small
    assert lib.qlora_quantize_nf4(P(0x200000), ctypes.byref(d), P(0x300000), 16, None) == \
        q.QLORA_ERR_WORKSPACE
    # K not a multiple of 64 on the linear path
    d2 = _desc(q, rows=64, cols=96)
    X = P(0x400000)
    st = lib.qlora_linear_fwd(ctypes.byref(d2), X, 4, X, X, 8, ctypes.c_float(16.0), X, None,
                              X, 1 << 30, None)
    assert st == q.QLORA_ERR_UNSUPPORTED
    # rank out of range, M < 1, misaligned activation
    assert lib.qlora_linear_fwd(ctypes.byref(d), X, 4, X, X, 0, ctypes.c_float(1.0), X, None, X,
                                1 << 30, None) == q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_linear_fwd(ctypes.byref(d), X, 0, X, X, 8, ctypes.c_float(1.0), X, None, X,
                                1 << 30, None) == q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_linear_fwd(ctypes.byref(d), P(0x400002), 4, X, X, 8, ctypes.c_float(1.0), X,
                                None, X, 1 << 30, None) == q.QLORA_ERR_INVALID_ARG
    # backward: missing dA, workspace too small
    assert lib.qlora_linear_bwd(ctypes.byref(d), X, 4, X, X, 8, ctypes.c_float(1.0), X, None, X,
                                None, X, X, 1 << 30, None) == q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_linear_bwd(ctypes.byref(d), X, 4, X, X, 8, ctypes.c_float(1.0), X, None, X,
                                X, X, X, 64, None) == q.QLORA_ERR_WORKSPACE


def test_no_cpu_fallback(q, monkeypatch):
    """The binding raises when the library is absent instead of computing on
    the host."""
    monkeypatch.setattr(q, "_lib", None)
    monkeypatch.setattr(q, "LIB_PATH", "/nonexistent/libqlora_nf4.so")
    with pytest.raises(RuntimeError):
        q.lib()


def test_dropout_argument_errors(q):
    """Drop probabilities outside [0, 1) (and NaN) are rejected on the host
    by all three dropout calls; an empty mask is a no-op."""
    lib = q.lib()
    P = ctypes.c_void_p
    d = _desc(q)
    X = P(0x400000)
    for p in (1.0, -0.1, 2.0, float("nan")):
        dr = q.QloraDropout(p, 7)
        assert lib.qlora_linear_fwd_dropout(ctypes.byref(d), X, 4, X, X, 8, ctypes.c_float(1.0),
                                            ctypes.byref(dr), None, X, None, X, 1 << 30,
                                            None) == q.QLORA_ERR_INVALID_ARG
        assert lib.qlora_linear_bwd_dropout(ctypes.byref(d), X, 4, X, X, 8, ctypes.c_float(1.0),
                                            ctypes.byref(dr), None, X, None, X, X, X, X, 1 << 30,
                                            None) == q.QLORA_ERR_INVALID_ARG
        assert lib.qlora_dropout_mask(4, 64, ctypes.byref(dr), X, None) == q.QLORA_ERR_INVALID_ARG
    ok = q.QloraDropout(0.1, 7)
    assert lib.qlora_dropout_mask(4, 64, None, X, None) == q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_dropout_mask(-1, 64, ctypes.byref(ok), X, None) == q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_dropout_mask(4, 64, ctypes.byref(ok), None, None) == q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_dropout_mask(0, 64, ctypes.byref(ok), None, None) == q.QLORA_OK
    # the shape checks of the plain calls come first
    assert lib.qlora_linear_fwd_dropout(ctypes.byref(d), X, 0, X, X, 8, ctypes.c_float(1.0),
                                        ctypes.byref(ok), None, X, None, X, 1 << 30, None) == \
        q.QLORA_ERR_INVALID_ARG


def test_adamw_argument_errors(q):
    """Bad hyperparameters, step numbers and tensors come back as status
    codes on the host; an empty tensor list is a no-op."""
    lib = q.lib()
    fake = 0x100000
    arr = (q.AdamWTensor * 1)(q.AdamWTensor(fake, fake, fake, fake, None, 8))
    ok = q.AdamWHparams(1e-3, 0.9, 0.999, 1e-8, 0.0)
    for h in (q.AdamWHparams(-1.0, 0.9, 0.999, 1e-8, 0.0),
              q.AdamWHparams(float("nan"), 0.9, 0.999, 1e-8, 0.0),
              q.AdamWHparams(1e-3, 1.0, 0.999, 1e-8, 0.0),
              q.AdamWHparams(1e-3, 0.9, -0.1, 1e-8, 0.0),
              q.AdamWHparams(1e-3, 0.9, 0.999, 0.0, 0.0),
              q.AdamWHparams(1e-3, 0.9, 0.999, 1e-8, -1.0)):
        assert lib.qlora_adamw_step(ctypes.byref(h), 1, arr, 1, None) == q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_adamw_step(ctypes.byref(ok), 0, arr, 1, None) == q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_adamw_step(None, 1, arr, 1, None) == q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_adamw_step(ctypes.byref(ok), 1, None, 1, None) == q.QLORA_ERR_INVALID_ARG
    for t in (q.AdamWTensor(fake + 2, fake, fake, fake, None, 8),
              q.AdamWTensor(fake, 0, fake, fake, None, 8),
              q.AdamWTensor(fake, fake, fake, fake, fake + 1, 8),
              q.AdamWTensor(fake, fake, fake, fake, None, -1)):
        one = (q.AdamWTensor * 1)(t)
        assert lib.qlora_adamw_step(ctypes.byref(ok), 1, one, 1, None) == q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_adamw_step(ctypes.byref(ok), 1, arr, 0, None) == q.QLORA_OK
    ptr = ctypes.c_void_p()
    assert lib.qlora_host_state_alloc(0, ctypes.byref(ptr)) == q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_host_state_alloc(64, None) == q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_host_state_free(None) == q.QLORA_OK


def test_grouped_argument_errors(q):
    """Groupings that do not cover W's rows, more than 8 groups, an empty
    group or a total rank above 128 are rejected on the host."""
    lib = q.lib()
    P = ctypes.c_void_p
    d = _desc(q, rows=128, cols=128)
    X = P(0x400000)
    for rows, r in (((64, 63), 8), ((16,) * 9, 8), ((64, 0, 64), 8), ((64, 64), 65)):
        arr = (ctypes.c_int64 * len(rows))(*rows)
        assert lib.qlora_grouped_fwd(ctypes.byref(d), X, 32, X, X, r, len(rows), arr,
                                     ctypes.c_float(16.0), X, None, X, 1 << 30, None) == \
            q.QLORA_ERR_INVALID_ARG
        assert lib.qlora_grouped_bwd(ctypes.byref(d), X, 32, X, X, r, len(rows), arr,
                                     ctypes.c_float(16.0), X, None, X, X, X, X, 1 << 30,
                                     None) == q.QLORA_ERR_INVALID_ARG
    assert q.qlora_grouped_workspace_bytes(32, 128, 128, 65, 2) == 0
    assert q.qlora_grouped_workspace_bytes(32, 128, 128, 16, 2) == \
        q.qlora_linear_workspace_bytes(32, 128, 128, 32)


def test_shapes_past_32_bit_offsets_are_unsupported(q):
    """The GEMMs address X, Y, dY, dX and the codes with 32-bit offsets, so
    M*K, M*N or N*K/2 at 2^32 must be refused before anything launches (the
    buffers are never touched: the shape check comes before the workspace
    check), and the workspace query returns 0 for them."""
    lib = q.lib()
    P = ctypes.c_void_p
    fake = P(0x100000)
    cases = [  # (M, N, K): refused
        (1 << 20, 64, 1 << 12),        # M*K = 2^32
        (1 << 20, 1 << 12, 64),        # M*N = 2^32
        (32, 1 << 20, 1 << 13),        # N*K/2 = 2^32
    ]
    for M, N, K in cases:
        d = _desc(q, rows=N, cols=K)
        assert q.qlora_linear_workspace_bytes(M, N, K, 8) == 0, (M, N, K)
        st = lib.qlora_linear_fwd(ctypes.byref(d), fake, M, fake, fake, 8,
                                  ctypes.c_float(16.0), fake, None, None, 0, None)
        assert st == q.QLORA_ERR_UNSUPPORTED, (M, N, K, st)
        st = lib.qlora_linear_bwd(ctypes.byref(d), fake, M, fake, fake, 8,
                                  ctypes.c_float(16.0), fake, None, fake, fake, fake, None, 0,
                                  None)
        assert st == q.QLORA_ERR_UNSUPPORTED, (M, N, K, st)
    # just below every limit: the shape passes and the missing workspace is
    # what is reported
    M, N, K = (1 << 20) - 1, 64, 1 << 12
    d = _desc(q, rows=N, cols=K)
    assert lib.qlora_linear_fwd(ctypes.byref(d), fake, M, fake, fake, 8, ctypes.c_float(16.0),
                                fake, None, None, 0, None) == q.QLORA_ERR_WORKSPACE
    M, N, K = 32, (1 << 19), (1 << 14) - 64
    d = _desc(q, rows=N, cols=K)
    assert q.qlora_linear_workspace_bytes(M, N, K, 8) > 0
    assert lib.qlora_linear_fwd(ctypes.byref(d), fake, M, fake, fake, 8, ctypes.c_float(16.0),
                                fake, None, None, 0, None) == q.QLORA_ERR_WORKSPACE


def test_oversized_tensors_and_masks_are_unsupported(q):
    lib = q.lib()
    P = ctypes.c_void_p
    fake = P(0x100000)
    big = _desc(q, rows=1 << 20, cols=(1 << 17) + 64)      # just over 2^37 weights
    assert q.qlora_quantize_workspace_bytes(1 << 20, (1 << 17) + 64) == 0
    assert lib.qlora_quantize_nf4(fake, ctypes.byref(big), fake, 1 << 30, None) == \
        q.QLORA_ERR_UNSUPPORTED
    assert lib.qlora_dequantize_nf4(ctypes.byref(big), q.QLORA_BF16, fake, None) == \
        q.QLORA_ERR_UNSUPPORTED
    assert lib.qlora_dequantize_absmax(ctypes.byref(big), fake, None) == q.QLORA_ERR_UNSUPPORTED
    assert q.qlora_merge_workspace_bytes(1 << 20, (1 << 17) + 64) == 0
    drop = q.QloraDropout(0.1, 5)
    # M * K would overflow int64: invalid, checked before the product is formed
    assert lib.qlora_dropout_mask(ctypes.c_int64((1 << 62)), 8, ctypes.byref(drop), fake,
                                  None) == q.QLORA_ERR_INVALID_ARG
    # 2^35 elements: more threads than one grid dimension holds
    assert lib.qlora_dropout_mask(ctypes.c_int64(1 << 23), 1 << 12, ctypes.byref(drop), fake,
                                  None) == q.QLORA_ERR_UNSUPPORTED


def test_noalloc_quantise_refuses_past_its_fixed_scratch(q):
    """The allocation-free quantiser takes at most 2^29 weights: one block
    more is refused on the host before any device call (fake buffers)."""
    lib = q.lib()
    fake = 0x100000
    for rows, cols in (((1 << 23) + 1, 64), (1 << 20, (1 << 9) + 64), (1 << 30, 64)):
        d = q.NF4Descriptor(rows, cols, 64, 256, fake, fake, fake, fake, 0, 0, 0)
        assert lib.qlora_quantize_nf4_noalloc(ctypes.c_void_p(fake), ctypes.byref(d), None) == \
            q.QLORA_ERR_UNSUPPORTED, (rows, cols)
    d = _desc(q)
    assert lib.qlora_quantize_nf4_noalloc(None, ctypes.byref(d), None) == q.QLORA_ERR_INVALID_ARG


def test_batch_argument_errors(q):
    """The batched quantiser and dequantiser check every tensor before any
    launch (fake buffers, never dereferenced), take count 0 as nothing to do,
    and need the sum of the single-tensor workspaces."""
    lib = q.lib()
    P = ctypes.c_void_p
    fake = 0x100000
    D2 = q.NF4Descriptor * 2
    ptrs = (P * 2)(P(fake), P(fake))
    bad = D2(_desc(q), _desc(q, rows=0))
    assert lib.qlora_quantize_nf4_batch(ptrs, bad, 2, P(fake), 1 << 30, None) == \
        q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_dequantize_nf4_batch(bad, 2, q.QLORA_F32, ptrs, None) == \
        q.QLORA_ERR_INVALID_ARG
    good = D2(_desc(q), _desc(q, rows=100, cols=1000))
    assert lib.qlora_quantize_nf4_batch(ptrs, good, -1, P(fake), 1 << 30, None) == \
        q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_quantize_nf4_batch(None, good, 2, P(fake), 1 << 30, None) == \
        q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_dequantize_nf4_batch(good, 2, 7, ptrs, None) == q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_dequantize_nf4_batch(good, 2, q.QLORA_F32, (P * 2)(P(fake), P(fake + 8)),
                                          None) == q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_quantize_nf4_batch(None, None, 0, None, 0, None) == q.QLORA_OK
    assert lib.qlora_dequantize_nf4_batch(None, 0, q.QLORA_BF16, None, None) == q.QLORA_OK
    need = q.qlora_quantize_batch_workspace_bytes([(64, 64), (100, 1000)])
    assert need == q.qlora_quantize_workspace_bytes(64, 64) + \
        q.qlora_quantize_workspace_bytes(100, 1000)
    assert lib.qlora_quantize_nf4_batch(ptrs, good, 2, P(fake), need - 1, None) == \
        q.QLORA_ERR_WORKSPACE
    big = D2(_desc(q), q.NF4Descriptor(1 << 31, 1 << 7, 64, 256, fake, fake, fake, fake, 0, 0, 0))
    assert lib.qlora_quantize_nf4_batch(ptrs, big, 2, P(fake), 1 << 40, None) == \
        q.QLORA_ERR_UNSUPPORTED
    assert q.qlora_quantize_batch_workspace_bytes([(0, 5)]) == 0
    assert q.qlora_quantize_batch_workspace_bytes([]) == 0


def test_linear_batch_argument_errors(q):
    """The batched forward checks every job before any launch (fake buffers),
    takes count 0 as nothing to do, and sizes its workspace as the jobs' own
    workspaces side by side (decode partials for M <= 16)."""
    lib = q.lib()
    P = ctypes.c_void_p
    fake = 0x100000
    d1, d2 = _desc(q, rows=1024, cols=4096), _desc(q, rows=4096, cols=1024)
    J = q.LinearJob * 2
    good = J(q.LinearJob(ctypes.pointer(d1), P(fake), P(fake), P(fake), P(fake), None),
             q.LinearJob(ctypes.pointer(d2), P(fake), P(fake), P(fake), P(fake), None))
    for M in (1, 16):
        need = lib.qlora_linear_batch_workspace_bytes(good, 2, M, 16)
        parts = []
        for rows, cols in ((1024, 4096), (4096, 1024)):
            parts.append(-(-(cols // 512) * M * rows * 4 // 256) * 256 +
                         -(-(cols // 512) * M * 16 * 4 // 256) * 256)
        assert need == sum(parts), (M, need, parts)
        assert lib.qlora_linear_fwd_batch(good, 2, M, 16, ctypes.c_float(32.0), P(fake), need - 1,
                                          None) == q.QLORA_ERR_WORKSPACE
    big = lib.qlora_linear_batch_workspace_bytes(good, 2, 64, 16)
    assert big == q.qlora_linear_workspace_bytes(64, 1024, 4096, 16) + \
        q.qlora_linear_workspace_bytes(64, 4096, 1024, 16)
    bad = J(good[0], q.LinearJob(ctypes.pointer(d2), P(fake), P(fake), P(fake), None, None))
    assert lib.qlora_linear_fwd_batch(bad, 2, 1, 16, ctypes.c_float(32.0), P(fake), 1 << 30,
                                      None) == q.QLORA_ERR_INVALID_ARG
    d3 = _desc(q, rows=64, cols=96)        # K not a multiple of 64
    odd = J(good[0], q.LinearJob(ctypes.pointer(d3), P(fake), P(fake), P(fake), P(fake), None))
    assert lib.qlora_linear_fwd_batch(odd, 2, 1, 16, ctypes.c_float(32.0), P(fake), 1 << 30,
                                      None) == q.QLORA_ERR_UNSUPPORTED
    assert lib.qlora_linear_fwd_batch(good, -1, 1, 16, ctypes.c_float(32.0), P(fake), 1 << 30,
                                      None) == q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_linear_fwd_batch(good, 2, 1, 0, ctypes.c_float(32.0), P(fake), 1 << 30,
                                      None) == q.QLORA_ERR_INVALID_ARG
    assert lib.qlora_linear_fwd_batch(None, 0, 1, 16, ctypes.c_float(32.0), None, 0, None) == \
        q.QLORA_OK
