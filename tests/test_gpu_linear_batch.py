"""GPU parity of the batched forward (qlora_linear_fwd_batch): independent
linears with one token count and rank.  At M <= 16 up to 8 of them share one
streaming launch and one finish launch; every job's Y and XA must equal what
qlora_linear_fwd gives for that job alone, bit for bit (the same kernels and
split order), and match the float64 oracle within the forward's tolerance.
Jobs mix shapes (ragged N, several K), both 4-bit tables and both constant
types; more than 8 jobs take two launch pairs; M > 16 runs the GEMM path."""
import numpy as np
import pytest
import torch

from gpu_common import DEV, assert_close, bf16_np, oracle, say, to_dev

pytestmark = pytest.mark.gpu

R, ALPHA = 16, 32.0
SHAPES = [(1024, 4096, "nf4", True), (100, 1024, "nf4", True), (4096, 1024, "int4", True),
          (300, 2048, "nf4", False), (64, 512, "int4", False), (1536, 4096, "nf4", True),
          (2000, 1024, "nf4", True), (128, 64, "nf4", True), (777, 2048, "int4", True),
          (1024, 1024, "nf4", True)]


@pytest.fixture(scope="module")
def q():
    import bit_quantized_lora_quant_amd as q
    q.lib()
    return q


def _jobs(q, M, shapes, seed):
    rng = np.random.default_rng(seed)
    out = []
    for N, K, kind, dq in shapes:
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        qq, _ = q.qlora_quantize_nf4(to_dev(w), quant_type=kind, double_quant=dq)
        x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
        lim = 1.0 / np.sqrt(K)
        a = torch.from_numpy(rng.uniform(-lim, lim, (R, K)).astype(np.float32)).to(torch.bfloat16)
        b = torch.from_numpy((rng.standard_normal((N, R)) * 0.01).astype(np.float32)).to(torch.bfloat16)
        out.append((qq, to_dev(x), to_dev(a), to_dev(b), w, kind, dq))
    return out


@pytest.mark.parametrize("M", [1, 4, 16, 40])
@pytest.mark.parametrize("count", [3, 10])
def test_batch_equals_single_calls(q, M, count):
    jobs = _jobs(q, M, SHAPES[:count], seed=M * 31 + count)
    say("linear batch M=%d jobs=%d" % (M, count))
    got = q.qlora_linear_fwd_batch([j[:4] for j in jobs], ALPHA, return_xa=True)
    single = [q.qlora_linear_fwd(qq, X, A, B, ALPHA, return_xa=True) for qq, X, A, B, *_ in jobs]
    torch.cuda.synchronize()
    for i, ((Yb, XAb), (Ys, XAs)) in enumerate(zip(got, single)):
        assert torch.equal(Yb.view(torch.int16), Ys.view(torch.int16)), "Y of job %d" % i
        assert torch.equal(XAb.view(torch.int16), XAs.view(torch.int16)), "XA of job %d" % i
    # and the oracle, for the first two jobs
    for i in range(2):
        qq, X, A, B, w, kind, dq = jobs[i]
        wd = oracle.dequantize(oracle.quantize(w.reshape(-1), kind=kind, dq=dq)).reshape(w.shape)
        y_ref, xa_ref = oracle.linear_fwd(wd.astype(np.float64), bf16_np(X), bf16_np(A),
                                          bf16_np(B), ALPHA)
        assert_close("Y", bf16_np(got[i][0]), y_ref)
        assert_close("XA", bf16_np(got[i][1]), xa_ref)


def test_batch_of_a_70b_layer_attention_inputs(q):
    """The 70B q, k and v projections (8192 -> 8192, 1024, 1024) at one token
    in one batch: each equals its single call."""
    shapes = [(8192, 8192, "nf4", True), (1024, 8192, "nf4", True), (1024, 8192, "nf4", True)]
    jobs = _jobs(q, 1, shapes, seed=70)
    say("linear batch 70B q/k/v M=1")
    got = q.qlora_linear_fwd_batch([j[:4] for j in jobs], ALPHA)
    single = [q.qlora_linear_fwd(qq, X, A, B, ALPHA) for qq, X, A, B, *_ in jobs]
    torch.cuda.synchronize()
    for i, (Yb, Ys) in enumerate(zip(got, single)):
        assert torch.equal(Yb.view(torch.int16), Ys.view(torch.int16)), "Y of job %d" % i


PAIR_SHAPES = [(1000, 512, "nf4", True), (777, 512, "nf4", True), (640, 512, "int4", True),
               (300, 512, "int4", False), (1500, 1024, "nf4", True), (256, 512, "nf4", True)]


def test_gemm_pairs_equal_single_calls(q):
    """M = 300 tokens with K = 512 (no split of K at any N): consecutive jobs
    of one K and table share a GEMM launch -- (1000, 777) and (640, 300),
    then 1500 alone (another K) and 256 alone -- and every Y and XA equals
    the single call's bit for bit; two of them also against the oracle."""
    M = 300
    jobs = _jobs(q, M, PAIR_SHAPES, seed=300)
    say("linear batch GEMM pairs M=%d" % M)
    got = q.qlora_linear_fwd_batch([j[:4] for j in jobs], ALPHA, return_xa=True)
    single = [q.qlora_linear_fwd(qq, X, A, B, ALPHA, return_xa=True) for qq, X, A, B, *_ in jobs]
    torch.cuda.synchronize()
    for i, ((Yb, XAb), (Ys, XAs)) in enumerate(zip(got, single)):
        assert torch.equal(Yb.view(torch.int16), Ys.view(torch.int16)), "Y of job %d" % i
        assert torch.equal(XAb.view(torch.int16), XAs.view(torch.int16)), "XA of job %d" % i
    for i in (1, 3):
        qq, X, A, B, w, kind, dq = jobs[i]
        wd = oracle.dequantize(oracle.quantize(w.reshape(-1), kind=kind, dq=dq)).reshape(w.shape)
        y_ref, xa_ref = oracle.linear_fwd(wd.astype(np.float64), bf16_np(X), bf16_np(A),
                                          bf16_np(B), ALPHA)
        assert_close("Y", bf16_np(got[i][0]), y_ref)
        assert_close("XA", bf16_np(got[i][1]), xa_ref)


def test_gemm_pair_of_the_65b_gate_and_up(q):
    """The LLaMA-65B gate and up projections (8192 -> 22016 each, r = 64) at
    4096 tokens as one paired GEMM launch (2752 tiles): both outputs equal
    the single calls' bit for bit."""
    g = torch.Generator(device=DEV)
    g.manual_seed(65)
    M, K, N, r = 4096, 8192, 22016, 64
    say("linear batch 65B gate/up pair")
    jobs = []
    for _ in range(2):
        W = torch.randn((N, K), generator=g, device=DEV) * 0.02
        qq, _ = q.qlora_quantize_nf4(W)
        del W
        X = torch.randn((M, K), generator=g, device=DEV).to(torch.bfloat16)
        A = (torch.randn((r, K), generator=g, device=DEV) * 0.01).to(torch.bfloat16)
        B = (torch.randn((N, r), generator=g, device=DEV) * 0.01).to(torch.bfloat16)
        jobs.append((qq, X, A, B))
    jobs[1] = (jobs[1][0], jobs[0][1], jobs[1][2], jobs[1][3])   # one shared input
    got = q.qlora_linear_fwd_batch(jobs, 16.0)
    single = [q.qlora_linear_fwd(*j, 16.0) for j in jobs]
    torch.cuda.synchronize()
    for i in range(2):
        assert torch.equal(got[i].view(torch.int16), single[i].view(torch.int16)), "Y %d" % i
