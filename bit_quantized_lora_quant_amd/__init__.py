"""MI355X (gfx950) frozen-NF4 linear with a LoRA side path.

A thin ctypes binding over ``libqlora_nf4.so`` (C ABI in ``include/qlora_nf4.h``).
Functions carry the C names and only marshal arguments: torch supplies device
memory and the current HIP stream, every step of the computation runs in the
library's HIP kernels.  There is no CPU fallback: if the library is missing,
every call raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora_nf4.so")

QLORA_OK, QLORA_ERR_INVALID_ARG, QLORA_ERR_UNSUPPORTED, QLORA_ERR_WORKSPACE, QLORA_ERR_HIP = range(5)
QLORA_F32, QLORA_BF16 = 0, 1
QUANT_TYPES = {"nf4": 0, "int4": 1}   # QLORA_QUANT_NF4, QLORA_QUANT_INT4
NF4_BLOCK = 64
DQ_BLOCK = 256
MAX_RANK = 128

EXPORTS = [
    "qlora_nf4_codebook", "qlora_codebook", "qlora_status_string",
    "qlora_quantize_workspace_bytes",
    "qlora_quantize_nf4", "qlora_quantize_nf4_noalloc", "qlora_dequantize_nf4",
    "qlora_dequantize_absmax", "qlora_quantize_batch_workspace_bytes",
    "qlora_quantize_nf4_batch", "qlora_dequantize_nf4_batch",
    "qlora_linear_workspace_bytes", "qlora_linear_fwd", "qlora_linear_bwd",
    "qlora_linear_batch_workspace_bytes", "qlora_linear_fwd_batch",
    "qlora_linear_fwd_dropout", "qlora_linear_bwd_dropout", "qlora_dropout_mask",
    "qlora_adamw_step", "qlora_adamw8_step", "qlora_host_state_alloc", "qlora_host_state_free",
    "qlora_merge_workspace_bytes", "qlora_merge_requantize",
    "qlora_grouped_workspace_bytes", "qlora_grouped_fwd", "qlora_grouped_bwd",
    "qlora_trace_begin", "qlora_trace_pause", "qlora_trace_end",
]
KERNELS = {"fwd_gemm": 0, "dx_gemm": 1, "quantize": 2, "dequant": 3, "gemv": 4,
           "split_reduce": 5, "adamw": 6, "adamw8": 7}
ADAMW8_BLOCK = 256


class QloraError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (status %d)" % (what, status_string(status), status))
        self.status = status


class NF4Descriptor(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("block", ctypes.c_int32), ("dq_block", ctypes.c_int32),
                ("codes", ctypes.c_void_p), ("absmax_q", ctypes.c_void_p),
                ("absmax_scale", ctypes.c_void_p), ("absmax_mean", ctypes.c_void_p),
                ("absmax", ctypes.c_void_p), ("quant_type", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class QloraDropout(ctypes.Structure):
    """LoRA dropout of the adapter input: drop probability p, generator seed."""
    _fields_ = [("p", ctypes.c_double), ("seed", ctypes.c_uint64)]


class AdamWTensor(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("exp_avg", ctypes.c_void_p), ("exp_avg_sq", ctypes.c_void_p),
                ("param_bf16", ctypes.c_void_p), ("numel", ctypes.c_int64)]


class AdamW8Tensor(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("exp_avg_q", ctypes.c_void_p), ("exp_avg_scale", ctypes.c_void_p),
                ("exp_avg_sq_q", ctypes.c_void_p), ("exp_avg_sq_scale", ctypes.c_void_p),
                ("param_bf16", ctypes.c_void_p), ("numel", ctypes.c_int64)]


class AdamWHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libqlora_nf4.so is not built (run __graft_entry__.build() or "
                               "python bit_quantized_lora_quant_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, F, SZ = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                              ctypes.c_size_t)
        D = ctypes.POINTER(NF4Descriptor)
        L.qlora_nf4_codebook.argtypes = [P]
        L.qlora_nf4_codebook.restype = None
        L.qlora_codebook.argtypes = [I32, P]
        L.qlora_codebook.restype = ctypes.c_int
        L.qlora_status_string.argtypes = [ctypes.c_int]
        L.qlora_status_string.restype = ctypes.c_char_p
        L.qlora_quantize_workspace_bytes.argtypes = [I64, I64]
        L.qlora_quantize_workspace_bytes.restype = SZ
        L.qlora_quantize_nf4.argtypes = [P, D, P, SZ, P]
        L.qlora_quantize_nf4_noalloc.argtypes = [P, D, P]
        L.qlora_dequantize_nf4.argtypes = [D, ctypes.c_int, P, P]
        L.qlora_dequantize_absmax.argtypes = [D, P, P]
        L.qlora_quantize_batch_workspace_bytes.argtypes = [P, P, I32]
        L.qlora_quantize_batch_workspace_bytes.restype = SZ
        L.qlora_quantize_nf4_batch.argtypes = [P, P, I32, P, SZ, P]
        L.qlora_dequantize_nf4_batch.argtypes = [P, I32, ctypes.c_int, P, P]
        L.qlora_linear_workspace_bytes.argtypes = [I64, I64, I64, I32]
        L.qlora_linear_workspace_bytes.restype = SZ
        L.qlora_linear_fwd.argtypes = [D, P, I64, P, P, I32, F, P, P, P, SZ, P]
        L.qlora_linear_batch_workspace_bytes.argtypes = [P, I32, I64, I32]
        L.qlora_linear_batch_workspace_bytes.restype = SZ
        L.qlora_linear_fwd_batch.argtypes = [P, I32, I64, I32, F, P, SZ, P]
        L.qlora_linear_bwd.argtypes = [D, P, I64, P, P, I32, F, P, P, P, P, P, P, SZ, P]
        L.qlora_linear_fwd_dropout.argtypes = [D, P, I64, P, P, I32, F, P, P, P, P, P, SZ, P]
        L.qlora_linear_bwd_dropout.argtypes = [D, P, I64, P, P, I32, F, P, P, P, P, P, P, P, P,
                                               SZ, P]
        L.qlora_dropout_mask.argtypes = [I64, I64, P, P, P]
        L.qlora_adamw_step.argtypes = [P, I64, P, I32, P]
        L.qlora_adamw8_step.argtypes = [P, I64, P, I32, P]
        L.qlora_grouped_workspace_bytes.restype = SZ
        L.qlora_grouped_workspace_bytes.argtypes = [I64, I64, I64, I32, I32]
        L.qlora_grouped_fwd.argtypes = [D, P, I64, P, P, I32, I32, P, F, P, P, P, SZ, P]
        L.qlora_grouped_bwd.argtypes = [D, P, I64, P, P, I32, I32, P, F, P, P, P, P, P, P, SZ,
                                        P]
        L.qlora_merge_workspace_bytes.restype = SZ
        L.qlora_merge_workspace_bytes.argtypes = [I64, I64]
        L.qlora_merge_requantize.argtypes = [D, P, P, I32, F, D, P, P, SZ, P]
        L.qlora_host_state_alloc.argtypes = [SZ, P]
        L.qlora_host_state_free.argtypes = [P]
        L.qlora_trace_begin.argtypes = [ctypes.c_uint32, I32]
        L.qlora_trace_pause.argtypes = [I32]
        L.qlora_trace_end.argtypes = [P, P]
        for name in ("qlora_quantize_nf4", "qlora_dequantize_nf4", "qlora_dequantize_absmax",
                     "qlora_linear_fwd", "qlora_linear_bwd", "qlora_trace_begin",
                     "qlora_trace_pause", "qlora_trace_end"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().qlora_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != QLORA_OK:
        raise QloraError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def qlora_nf4_codebook():
    """The 16 NF4 levels as a list of floats (host copy)."""
    buf = (ctypes.c_float * 16)()
    lib().qlora_nf4_codebook(buf)
    return [float(v) for v in buf]


def qlora_codebook(quant_type: str = "nf4"):
    """The 16 levels of a 4-bit type ("nf4" or "int4") as a list of floats."""
    buf = (ctypes.c_float * 16)()
    _check(lib().qlora_codebook(QUANT_TYPES[quant_type], buf), "qlora_codebook")
    return [float(v) for v in buf]


class NF4Tensor:
    """Quantised frozen weight: device buffers owned by torch.  quant_type
    "nf4" or "int4"; double_quant False keeps float32 block constants."""

    def __init__(self, rows: int, cols: int, device, quant_type: str = "nf4",
                 double_quant: bool = True):
        n = rows * cols
        nb = (n + NF4_BLOCK - 1) // NF4_BLOCK
        nd = (nb + DQ_BLOCK - 1) // DQ_BLOCK
        self.rows, self.cols = rows, cols
        self.quant_type, self.double_quant = quant_type, double_quant
        self.codes = torch.empty((n + 1) // 2, dtype=torch.uint8, device=device)
        self.absmax_q = self.absmax_scale = self.absmax_mean = self.absmax = None
        if double_quant:
            self.absmax_q = torch.empty(nb, dtype=torch.int8, device=device)
            self.absmax_scale = torch.empty(nd, dtype=torch.float32, device=device)
            self.absmax_mean = torch.empty(1, dtype=torch.float32, device=device)
        else:
            self.absmax = torch.empty(nb, dtype=torch.float32, device=device)

    @property
    def numel(self):
        return self.rows * self.cols

    @property
    def num_blocks(self):
        return (self.numel + NF4_BLOCK - 1) // NF4_BLOCK

    def descriptor(self) -> NF4Descriptor:
        p = lambda t: 0 if t is None else t.data_ptr()  # noqa: E731
        return NF4Descriptor(self.rows, self.cols, NF4_BLOCK, DQ_BLOCK if self.double_quant else 0,
                             p(self.codes), p(self.absmax_q), p(self.absmax_scale),
                             p(self.absmax_mean), p(self.absmax), QUANT_TYPES[self.quant_type], 0)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size()
                   for t in (self.codes, self.absmax_q, self.absmax_scale, self.absmax_mean,
                             self.absmax) if t is not None)


def qlora_quantize_workspace_bytes(rows: int, cols: int) -> int:
    return int(lib().qlora_quantize_workspace_bytes(rows, cols))


def qlora_linear_workspace_bytes(M: int, N: int, K: int, r: int) -> int:
    return int(lib().qlora_linear_workspace_bytes(M, N, K, r))


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def qlora_quantize_nf4(W: torch.Tensor, q: NF4Tensor = None, ws: torch.Tensor = None,
                       quant_type: str = "nf4", double_quant: bool = True):
    """Quantise a float32 [rows, cols] device tensor; returns (NF4Tensor,
    workspace).  With double quantisation the workspace's first nb floats hold
    the exact block absmax; without it the tensor's absmax holds them."""
    assert W.dtype == torch.float32 and W.is_contiguous() and W.dim() == 2
    rows, cols = W.shape
    if q is None:
        q = NF4Tensor(rows, cols, W.device, quant_type, double_quant)
    need = qlora_quantize_workspace_bytes(rows, cols)
    if ws is None:
        ws = workspace(need, W.device)
    d = q.descriptor()
    _check(lib().qlora_quantize_nf4(_ptr(W), ctypes.byref(d), _ptr(ws), ws.numel(), _stream()),
           "qlora_quantize_nf4")
    return q, ws


def qlora_dequantize_nf4(q: NF4Tensor, dtype=torch.bfloat16, out: torch.Tensor = None):
    if out is None:
        out = torch.empty((q.rows, q.cols), dtype=dtype, device=q.codes.device)
    code = QLORA_BF16 if out.dtype == torch.bfloat16 else QLORA_F32
    assert out.dtype in (torch.bfloat16, torch.float32) and out.is_contiguous()
    d = q.descriptor()
    _check(lib().qlora_dequantize_nf4(ctypes.byref(d), code, _ptr(out), _stream()),
           "qlora_dequantize_nf4")
    return out


def qlora_quantize_batch_workspace_bytes(shapes) -> int:
    """Workspace bytes for qlora_quantize_nf4_batch over (rows, cols) pairs."""
    shapes = list(shapes)
    rows = (ctypes.c_int64 * max(len(shapes), 1))(*[r for r, _ in shapes])
    cols = (ctypes.c_int64 * max(len(shapes), 1))(*[c for _, c in shapes])
    return int(lib().qlora_quantize_batch_workspace_bytes(rows, cols, len(shapes)))


def qlora_quantize_nf4_batch(Ws, qs, ws: torch.Tensor = None):
    """Quantise float32 [rows, cols] device tensors Ws[i] into the NF4Tensors
    qs[i], up to 32 tensors per launch; returns the workspace."""
    Ws, qs = list(Ws), list(qs)
    assert len(Ws) == len(qs)
    for W, q in zip(Ws, qs):
        assert W.dtype == torch.float32 and W.is_contiguous() and W.dim() == 2
        assert tuple(W.shape) == (q.rows, q.cols)
    if ws is None:
        need = qlora_quantize_batch_workspace_bytes([(q.rows, q.cols) for q in qs])
        ws = workspace(need, Ws[0].device if Ws else "cpu")
    n = len(qs)
    ptrs = (ctypes.c_void_p * max(n, 1))(*[_ptr(W) for W in Ws])
    descs = (NF4Descriptor * max(n, 1))(*[q.descriptor() for q in qs])
    _check(lib().qlora_quantize_nf4_batch(ptrs, descs, n, _ptr(ws), ws.numel(), _stream()),
           "qlora_quantize_nf4_batch")
    return ws


def qlora_dequantize_nf4_batch(qs, outs):
    """Dequantise NF4Tensors qs[i] into contiguous device tensors outs[i]
    (all bf16 or all float32), up to 32 tensors per launch."""
    qs, outs = list(qs), list(outs)
    assert len(qs) == len(outs)
    dt = outs[0].dtype if outs else torch.bfloat16
    for q, o in zip(qs, outs):
        assert o.dtype == dt and dt in (torch.bfloat16, torch.float32) and o.is_contiguous()
        assert o.numel() == q.numel
    n = len(qs)
    ptrs = (ctypes.c_void_p * max(n, 1))(*[_ptr(o) for o in outs])
    descs = (NF4Descriptor * max(n, 1))(*[q.descriptor() for q in qs])
    code = QLORA_BF16 if dt == torch.bfloat16 else QLORA_F32
    _check(lib().qlora_dequantize_nf4_batch(descs, n, code, ptrs, _stream()),
           "qlora_dequantize_nf4_batch")
    return outs


def qlora_dequantize_absmax(q: NF4Tensor, out: torch.Tensor = None):
    if out is None:
        out = torch.empty(q.num_blocks, dtype=torch.float32, device=q.codes.device)
    d = q.descriptor()
    _check(lib().qlora_dequantize_absmax(ctypes.byref(d), _ptr(out), _stream()),
           "qlora_dequantize_absmax")
    return out


def _bf16(t):
    assert t.dtype == torch.bfloat16 and t.is_contiguous(), "expected contiguous bf16"
    return t


def _dropout(dropout):
    """None, or a QloraDropout from (p, seed)."""
    if dropout is None:
        return None
    p, seed = dropout
    return QloraDropout(float(p), int(seed) & 0xFFFFFFFFFFFFFFFF)


def qlora_dropout_mask(M: int, K: int, dropout, device, out=None):
    """uint8 [M, K] keep flags of the dropout (p, seed) of an [M, K] input."""
    if out is None:
        out = torch.empty((M, K), dtype=torch.uint8, device=device)
    d = _dropout(dropout)
    _check(lib().qlora_dropout_mask(M, K, ctypes.byref(d), _ptr(out) if out.numel() else None,
                                    _stream()), "qlora_dropout_mask")
    return out


def keep_bits_buffer(M: int, K: int, device):
    """uint8 [M * K / 8] for the forward's dropout keep bits."""
    return torch.empty((M * K + 7) // 8, dtype=torch.uint8, device=device)


def qlora_linear_fwd(q: NF4Tensor, X, A, B, alpha: float, Y=None, XA_out=None, ws=None,
                     return_xa: bool = False, dropout=None, keep_bits=None):
    """Y = X W'^T + (alpha/r) (D(X) A^T) B^T.  Returns Y, or (Y, XA) with
    return_xa.  dropout = (p, seed) drops adapter-input elements (D(X) = X
    without it); keep_bits (from keep_bits_buffer) receives the mask."""
    M, K = X.shape
    r = A.shape[0]
    _bf16(X), _bf16(A), _bf16(B)
    assert K == q.cols and A.shape[1] == K and B.shape == (q.rows, r)
    if Y is None:
        Y = torch.empty((M, q.rows), dtype=torch.bfloat16, device=X.device)
    if return_xa and XA_out is None:
        XA_out = torch.empty((M, r), dtype=torch.bfloat16, device=X.device)
    if ws is None:
        ws = workspace(qlora_linear_workspace_bytes(M, q.rows, K, r), X.device)
    d = q.descriptor()
    if dropout is None:
        _check(lib().qlora_linear_fwd(ctypes.byref(d), _ptr(X), M, _ptr(A), _ptr(B), r,
                                      ctypes.c_float(alpha), _ptr(Y), _ptr(XA_out), _ptr(ws),
                                      ws.numel(), _stream()), "qlora_linear_fwd")
    else:
        dr = _dropout(dropout)
        _check(lib().qlora_linear_fwd_dropout(ctypes.byref(d), _ptr(X), M, _ptr(A), _ptr(B), r,
                                              ctypes.c_float(alpha), ctypes.byref(dr),
                                              _ptr(keep_bits), _ptr(Y), _ptr(XA_out), _ptr(ws),
                                              ws.numel(), _stream()),
               "qlora_linear_fwd_dropout")
    return (Y, XA_out) if return_xa else Y


class LinearJob(ctypes.Structure):
    """qlora_linear_job: one linear of a batched forward."""
    _fields_ = [("W", ctypes.POINTER(NF4Descriptor)), ("X", ctypes.c_void_p),
                ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("Y", ctypes.c_void_p),
                ("XA_out", ctypes.c_void_p)]


def _linear_jobs(jobs):
    descs = [q.descriptor() for q, *_ in jobs]
    arr = (LinearJob * max(len(jobs), 1))()
    for i, ((q, X, A, B, Y, XA), d) in enumerate(zip(jobs, descs)):
        arr[i] = LinearJob(ctypes.pointer(d), _ptr(X), _ptr(A), _ptr(B), _ptr(Y), _ptr(XA))
    return arr, descs


def qlora_linear_batch_workspace_bytes(qs, M: int, r: int) -> int:
    jobs = [(q, None, None, None, None, None) for q in qs]
    arr, keep = _linear_jobs(jobs)
    return int(lib().qlora_linear_batch_workspace_bytes(arr, len(jobs), M, r))


def qlora_linear_fwd_batch(jobs, alpha: float, ws=None, return_xa: bool = False, XA_out=None):
    """Forward of independent linears (q, X, A, B[, Y]) with one M and rank r;
    for M <= 16 up to 8 share each launch pair, for M > 16 consecutive pairs
    of one K share a GEMM launch.  XA_out (optional): one [M, r] buffer per
    job.  Returns the list of Y (or of (Y, XA) with return_xa)."""
    jobs = list(jobs)
    M, r = jobs[0][1].shape[0], jobs[0][2].shape[0]
    full = []
    for job in jobs:
        q, X, A, B = job[:4]
        _bf16(X), _bf16(A), _bf16(B)
        assert X.shape == (M, q.cols) and A.shape == (r, q.cols) and B.shape == (q.rows, r)
        Y = job[4] if len(job) > 4 and job[4] is not None else \
            torch.empty((M, q.rows), dtype=torch.bfloat16, device=X.device)
        if XA_out is not None:
            XA = XA_out[len(full)]
        else:
            XA = torch.empty((M, r), dtype=torch.bfloat16, device=X.device) if return_xa else None
        full.append((q, X, A, B, Y, XA))
    arr, keep = _linear_jobs(full)
    if ws is None:
        ws = workspace(lib().qlora_linear_batch_workspace_bytes(arr, len(full), M, r),
                       jobs[0][1].device)
    _check(lib().qlora_linear_fwd_batch(arr, len(full), M, r, ctypes.c_float(alpha), _ptr(ws),
                                        ws.numel(), _stream()), "qlora_linear_fwd_batch")
    return [(j[4], j[5]) if return_xa else j[4] for j in full]


def qlora_linear_bwd(q: NF4Tensor, X, A, B, alpha: float, dY, XA_in=None, need_dx: bool = True,
                     dX=None, dA=None, dB=None, ws=None, dropout=None, keep_bits=None):
    """Returns (dX or None, dA float32 [r, K], dB float32 [N, r]).  dropout
    must be the forward's (p, seed); keep_bits (optional) its stored mask."""
    M, K = X.shape
    r = A.shape[0]
    N = q.rows
    _bf16(X), _bf16(A), _bf16(B), _bf16(dY)
    assert dY.shape == (M, N)
    if need_dx and dX is None:
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=X.device)
    if dA is None:
        dA = torch.empty((r, K), dtype=torch.float32, device=X.device)
    if dB is None:
        dB = torch.empty((N, r), dtype=torch.float32, device=X.device)
    if ws is None:
        ws = workspace(qlora_linear_workspace_bytes(M, N, K, r), X.device)
    d = q.descriptor()
    if dropout is None:
        _check(lib().qlora_linear_bwd(ctypes.byref(d), _ptr(X), M, _ptr(A), _ptr(B), r,
                                      ctypes.c_float(alpha), _ptr(dY), _ptr(XA_in),
                                      _ptr(dX) if need_dx else None, _ptr(dA), _ptr(dB),
                                      _ptr(ws), ws.numel(), _stream()), "qlora_linear_bwd")
    else:
        dr = _dropout(dropout)
        _check(lib().qlora_linear_bwd_dropout(ctypes.byref(d), _ptr(X), M, _ptr(A), _ptr(B), r,
                                              ctypes.c_float(alpha), ctypes.byref(dr),
                                              _ptr(keep_bits), _ptr(dY),
                                              _ptr(XA_in), _ptr(dX) if need_dx else None,
                                              _ptr(dA), _ptr(dB), _ptr(ws), ws.numel(),
                                              _stream()), "qlora_linear_bwd_dropout")
    return (dX if need_dx else None), dA, dB


def qlora_grouped_workspace_bytes(M: int, N: int, K: int, r: int, groups: int) -> int:
    return int(lib().qlora_grouped_workspace_bytes(M, N, K, r, groups))


def _rows_arg(group_rows):
    arr = (ctypes.c_int64 * len(group_rows))(*[int(n) for n in group_rows])
    return arr


def qlora_grouped_fwd(q: NF4Tensor, X, A, B, r: int, group_rows, alpha: float, Y=None,
                      XA_out=None, ws=None, return_xa: bool = False):
    """Fused projections of one input: q holds the concatenated rows, A [G r, K]
    the stacked A_g, B [N, G r] the block-diagonal B_g.  Returns Y [M, N] (or
    (Y, XA [M, G r]))."""
    M, K = X.shape
    G = len(group_rows)
    _bf16(X), _bf16(A), _bf16(B)
    assert A.shape == (G * r, K) and B.shape == (q.rows, G * r) and K == q.cols
    if Y is None:
        Y = torch.empty((M, q.rows), dtype=torch.bfloat16, device=X.device)
    if return_xa and XA_out is None:
        XA_out = torch.empty((M, G * r), dtype=torch.bfloat16, device=X.device)
    if ws is None:
        ws = workspace(qlora_grouped_workspace_bytes(M, q.rows, K, r, G), X.device)
    d = q.descriptor()
    rows = _rows_arg(group_rows)
    _check(lib().qlora_grouped_fwd(ctypes.byref(d), _ptr(X), M, _ptr(A), _ptr(B), r, G, rows,
                                   ctypes.c_float(alpha), _ptr(Y), _ptr(XA_out), _ptr(ws),
                                   ws.numel(), _stream()), "qlora_grouped_fwd")
    return (Y, XA_out) if return_xa else Y


def qlora_grouped_bwd(q: NF4Tensor, X, A, B, r: int, group_rows, alpha: float, dY, XA_in=None,
                      need_dx: bool = True, dX=None, dA=None, dB=None, ws=None):
    """Returns (dX or None, dA float32 [G r, K], dB float32 [N, G r] block-diagonal)."""
    M, K = X.shape
    G = len(group_rows)
    N = q.rows
    _bf16(X), _bf16(A), _bf16(B), _bf16(dY)
    if need_dx and dX is None:
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=X.device)
    if dA is None:
        dA = torch.empty((G * r, K), dtype=torch.float32, device=X.device)
    if dB is None:
        dB = torch.empty((N, G * r), dtype=torch.float32, device=X.device)
    if ws is None:
        ws = workspace(qlora_grouped_workspace_bytes(M, N, K, r, G), X.device)
    d = q.descriptor()
    rows = _rows_arg(group_rows)
    _check(lib().qlora_grouped_bwd(ctypes.byref(d), _ptr(X), M, _ptr(A), _ptr(B), r, G, rows,
                                   ctypes.c_float(alpha), _ptr(dY), _ptr(XA_in),
                                   _ptr(dX) if need_dx else None, _ptr(dA), _ptr(dB), _ptr(ws),
                                   ws.numel(), _stream()), "qlora_grouped_bwd")
    return (dX if need_dx else None), dA, dB


def qlora_merge_workspace_bytes(rows: int, cols: int) -> int:
    return int(lib().qlora_merge_workspace_bytes(rows, cols))


def qlora_merge_requantize(q: NF4Tensor, A, B, alpha: float, out: NF4Tensor = None,
                           merged=None, ws=None, return_merged: bool = False):
    """Folds the adapters into the weight (W' + (alpha/r) B A) and quantises the
    result into `out` (a new tensor of q's type by default; q itself for an
    in-place merge).  Returns out, or (out, merged float32 [N, K]) with
    return_merged."""
    _bf16(A), _bf16(B)
    r = A.shape[0]
    assert A.shape == (r, q.cols) and B.shape == (q.rows, r)
    dev = A.device
    if out is None:
        out = NF4Tensor(q.rows, q.cols, dev, q.quant_type, q.double_quant)
    if return_merged and merged is None:
        merged = torch.empty((q.rows, q.cols), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(qlora_merge_workspace_bytes(q.rows, q.cols), dev)
    d, do = q.descriptor(), out.descriptor()
    _check(lib().qlora_merge_requantize(ctypes.byref(d), _ptr(A), _ptr(B), r,
                                        ctypes.c_float(alpha), ctypes.byref(do), _ptr(merged),
                                        _ptr(ws), ws.numel(), _stream()),
           "qlora_merge_requantize")
    return (out, merged) if return_merged else out


def qlora_adamw_step(tensors, step: int, lr: float, beta1: float = 0.9, beta2: float = 0.999,
                     eps: float = 1e-8, weight_decay: float = 0.0):
    """One AdamW step.  tensors: list of (param, grad, exp_avg, exp_avg_sq,
    param_bf16 or None); float32 contiguous tensors of one numel each (device
    tensors, or host-state tensors from qlora_host_state_alloc for the two
    statistics), param_bf16 bf16."""
    arr = (AdamWTensor * max(len(tensors), 1))()
    for i, (p, g, m, v, pb) in enumerate(tensors):
        n = p.numel()
        for t in (p, g, m, v):
            assert t.dtype == torch.float32 and t.is_contiguous() and t.numel() == n
        if pb is not None:
            assert pb.dtype == torch.bfloat16 and pb.is_contiguous() and pb.numel() == n
        arr[i] = AdamWTensor(_ptr(p), _ptr(g), _ptr(m), _ptr(v),
                             _ptr(pb) if pb is not None else None, n)
    h = AdamWHparams(lr, beta1, beta2, eps, weight_decay)
    _check(lib().qlora_adamw_step(ctypes.byref(h), step, arr, len(tensors), _stream()),
           "qlora_adamw_step")


def qlora_adamw8_step(tensors, step: int, lr: float, beta1: float = 0.9, beta2: float = 0.999,
                      eps: float = 1e-8, weight_decay: float = 0.0):
    """One AdamW step with 8-bit statistics.  tensors: list of (param, grad,
    state, param_bf16 or None) with param and grad float32 contiguous tensors
    of one numel and state an AdamW8State of that numel (device or host)."""
    arr = (AdamW8Tensor * max(len(tensors), 1))()
    for i, (p, g, st, pb) in enumerate(tensors):
        n = p.numel()
        for t in (p, g):
            assert t.dtype == torch.float32 and t.is_contiguous() and t.numel() == n
        assert st.numel == n
        if pb is not None:
            assert pb.dtype == torch.bfloat16 and pb.is_contiguous() and pb.numel() == n
        arr[i] = AdamW8Tensor(_ptr(p), _ptr(g), _ptr(st.m_q), _ptr(st.m_scale), _ptr(st.v_q),
                              _ptr(st.v_scale), _ptr(pb) if pb is not None else None, n)
    h = AdamWHparams(lr, beta1, beta2, eps, weight_decay)
    _check(lib().qlora_adamw8_step(ctypes.byref(h), step, arr, len(tensors), _stream()),
           "qlora_adamw8_step")


class HostState:
    """Pinned, device-mapped host memory for optimiser statistics, viewed as a
    CPU tensor of `dtype` (``.tensor``).  Freed by ``free()`` or when
    collected; views taken of ``.tensor`` must not outlive it, and no queued
    GPU work may still use the memory when it is freed (synchronise first)."""

    def __init__(self, numel: int, dtype=torch.float32):
        size = torch.empty(0, dtype=dtype).element_size()
        ptr = ctypes.c_void_p()
        _check(lib().qlora_host_state_alloc(max(size * numel, 1), ctypes.byref(ptr)),
               "qlora_host_state_alloc")
        self.ptr = ptr.value
        buf = (ctypes.c_byte * max(size * numel, 1)).from_address(self.ptr)
        self.tensor = torch.frombuffer(buf, dtype=dtype, count=numel)

    def free(self):
        if self.ptr:
            self.tensor = None
            _check(lib().qlora_host_state_free(self.ptr), "qlora_host_state_free")
            self.ptr = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def qlora_host_state_alloc(numel: int, dtype=torch.float32) -> HostState:
    return HostState(numel, dtype)


class AdamW8State:
    """The 8-bit statistics of one tensor of `numel` parameters, zero (the
    state before step 1): int8 codes of m and uint8 codes of sqrt(v), one
    float32 scale of each per 256 parameters.  host=True keeps them in
    pinned, device-mapped host memory (the paged placement)."""

    def __init__(self, numel: int, device, host: bool = False):
        nb = (numel + ADAMW8_BLOCK - 1) // ADAMW8_BLOCK
        self.numel = numel
        self.on_host = bool(host)
        self._host = []
        if host:
            bufs = [HostState(numel, torch.int8), HostState(nb, torch.float32),
                    HostState(numel, torch.uint8), HostState(nb, torch.float32)]
            self._host = bufs
            for b in bufs:
                b.tensor.zero_()
            self.m_q, self.m_scale, self.v_q, self.v_scale = (b.tensor for b in bufs)
        else:
            self.m_q = torch.zeros(numel, dtype=torch.int8, device=device)
            self.m_scale = torch.zeros(nb, dtype=torch.float32, device=device)
            self.v_q = torch.zeros(numel, dtype=torch.uint8, device=device)
            self.v_scale = torch.zeros(nb, dtype=torch.float32, device=device)

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.m_q, self.m_scale, self.v_q,
                                                           self.v_scale))

    def free(self):
        """Release host buffers (synchronise first); device ones go with the object."""
        self.m_q = self.m_scale = self.v_q = self.v_scale = None
        for b in self._host:
            b.free()
        self._host = []


def adamw8_state_bytes(numel: int) -> int:
    """Bytes of the 8-bit statistics of `numel` parameters (two codes per
    parameter, two float32 scales per 256)."""
    return 2 * numel + 8 * ((numel + ADAMW8_BLOCK - 1) // ADAMW8_BLOCK)


def plan_state_placement(state_bytes, hbm_budget: int):
    """Placement of optimiser statistics under an HBM budget (the paged
    optimiser of the pages, made explicit: this part has no managed memory to
    migrate pages on demand).  Every step reads and writes every tensor's
    statistics once, so the bytes left in host memory cross the host link each
    step; keeping the largest tensors in HBM first leaves the fewest of them
    there for a given budget.  Returns, per tensor in the given order, True
    when its statistics go to pinned, device-mapped host memory.  No tensor
    placed in host memory would have fit in the budget left over."""
    sizes = [int(b) for b in state_bytes]
    left = int(hbm_budget)
    host = [True] * len(sizes)
    for i in sorted(range(len(sizes)), key=lambda i: (-sizes[i], i)):
        if sizes[i] <= left:
            host[i] = False
            left -= sizes[i]
    return host


def adamw8_states(numels, device, hbm_budget: int = None):
    """AdamW8State for each tensor size, placed by plan_state_placement
    (all in HBM without a budget)."""
    numels = [int(n) for n in numels]
    host = ([False] * len(numels) if hbm_budget is None else
            plan_state_placement([adamw8_state_bytes(n) for n in numels], hbm_budget))
    return [AdamW8State(n, device, host=h) for n, h in zip(numels, host)]


def qlora_trace_begin(kernels, capacity: int = 4096):
    """Start timing launches of the named kernels (see KERNELS) with HIP events."""
    mask = 0
    for k in kernels:
        mask |= 1 << KERNELS[k]
    _check(lib().qlora_trace_begin(mask, capacity), "qlora_trace_begin")


def qlora_trace_pause(paused: bool):
    """Stop (True) or resume (False) recording between begin and end."""
    _check(lib().qlora_trace_pause(1 if paused else 0), "qlora_trace_pause")


def qlora_trace_end():
    """{kernel name: (launches, total_ms)} for the kernels timed since begin."""
    n = (ctypes.c_int32 * len(KERNELS))()
    ms = (ctypes.c_double * len(KERNELS))()
    _check(lib().qlora_trace_end(n, ms), "qlora_trace_end")
    return {name: (int(n[i]), float(ms[i])) for name, i in KERNELS.items() if n[i] > 0}


class QLoRALinearFn(torch.autograd.Function):
    """autograd wrapper: frozen NF4 weight, trainable bf16 adapters A and B."""

    @staticmethod
    def forward(ctx, X, A, B, q, alpha, dropout=None):
        bits = keep_bits_buffer(X.shape[0], X.shape[1], X.device) if dropout else None
        Y, XA = qlora_linear_fwd(q, X.contiguous(), A.contiguous(), B.contiguous(), alpha,
                                 return_xa=True, dropout=dropout, keep_bits=bits)
        ctx.save_for_backward(X, A, B, XA)
        ctx.q, ctx.alpha, ctx.dropout, ctx.bits = q, alpha, dropout, bits
        return Y

    @staticmethod
    def backward(ctx, dY):
        X, A, B, XA = ctx.saved_tensors
        dX, dA, dB = qlora_linear_bwd(ctx.q, X, A, B, ctx.alpha, dY.contiguous(), XA_in=XA,
                                      need_dx=ctx.needs_input_grad[0], dropout=ctx.dropout,
                                      keep_bits=ctx.bits)
        return dX, dA.to(A.dtype), dB.to(B.dtype), None, None, None
