#!/usr/bin/env python
"""Benchmark of the frozen-NF4 LoRA linear on one MI355X.

Headline step: forward then backward (reverse order) through 80 LLaMA-65B
layers, each with its own NF4 weights (double quantisation) for the seven
projections (q, k, v, o 8192 -> 8192, gate/up 8192 -> 22016, down 22016 ->
8192, about 33 GB of quantised state resident in HBM), 4 x 1024 = 4096 tokens,
LoRA r = 64, alpha = 16, each projection with its own adapter pair.  ``value``
is tokens per second of that step with every input resident in HBM.  The JSON
line also carries the dominant kernel's roofline (HIP-event durations measured
on the library's stream during the timed region, algorithmic flops per launch,
HBM bytes per launch from the committed rocprofv3 counter summary), the CPU
oracle timed on a bounded sample of the same step, and the other legs of the
path: the Llama-3.1-8B layer step (2048 tokens, r = 16, layer driver), that
step with LoRA dropout and as 7 separate linears, quantise + dequantise of the
full 8.03B-parameter weight set, the NF4 / INT4 and constant variants, the
AdamW step over every 8B adapter, and the 70B-shaped decode GEMV at 1 / 4 / 16
tokens.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs all|none|...]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def log(msg):
    print("[bench] %s" % msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs", default="all",
                    help="all, none, or a comma list of layer8b, quant, variants, dropout, driver, "
                         "adamw, decode")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--headline", choices=["on", "off"], default="on",
                    help="off: skip the headline step (and the CPU baseline) and print only "
                         "the legs, for profiling a leg on its own")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run 3 plain device-to-device copies of MIB MiB (the known-size "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def calibrate_copy(torch, mib):
    """Three device-to-device copies of `mib` MiB: reads and writes exactly
    mib MiB each, so a counter pass over it gives the counter's bytes per KiB."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy calibration: 3 x %d MiB device-to-device" % mib)
    del src, dst
    torch.cuda.empty_cache()


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_quantized_lora_quant_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel):
    """HBM bytes per launch of `kernel` (FETCH_SIZE + WRITE_SIZE, each scaled by
    a plain copy's reading) from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        t = json.load(open(path)).get(kernel)
    except ValueError:
        return None
    if not t or t.get("source_sha") != src_hash(*t.get("sources", [])):
        return None
    return t.get("hbm_bytes_per_launch")


def graph_of(torch, fn):
    """Capture the launches `fn` makes (on torch's current stream, which the
    library enqueues on) into a HIP graph; one eager run first, off-capture."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def timed(torch, fn, reps):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / reps


# ---------------------------------------------------------------- headline
def linear_flops(M, N, K, r):
    """Algorithmic flops of fwd + bwd of one adapted frozen linear (no dW):
    fwd 2MNK + 2Mr(K+N); bwd dX 2MNK + 2MrK, G 2MNr, dA 2MrK, dB 2MNr."""
    return 4 * M * N * K + 6 * M * r * (K + N)


# The layer driver: the projections that read one input run as one grouped
# weight (q/k/v: N = 6144 with three adapter pairs; gate/up: N = 28672 with
# two), o and down alone -- 4 fused-GEMM pairs per step instead of 7.
GROUPS = [[0, 1, 2], [3], [4, 5], [6]]


def build_units(q, torch, layers, host_w, M, r):
    dev = "cuda:0"
    units = []
    for idx in GROUPS:
        if len(idx) == 1:
            units.append(dict(single=True, **layers[idx[0]]))
            continue
        Ls = [layers[i] for i in idx]
        rows = [L["N"] for L in Ls]
        N, K, G = sum(rows), Ls[0]["K"], len(Ls)
        qq, _ = q.qlora_quantize_nf4(torch.cat([torch.from_numpy(host_w[i]) for i in idx], 0)
                                     .to(dev))
        A = torch.cat([L["A"] for L in Ls], 0).contiguous()
        B = torch.zeros((N, G * r), dtype=torch.bfloat16, device=dev)
        e = 0
        for g, L in enumerate(Ls):
            B[e:e + L["N"], g * r:(g + 1) * r] = L["B"]
            e += L["N"]
        dY = torch.cat([L["dY"] for L in Ls], 1).contiguous()
        units.append(dict(single=False, rows=rows, N=N, K=K, G=G, q=qq, X=Ls[0]["X"], A=A, B=B,
                          dY=dY, Y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                          XA=torch.empty((M, G * r), dtype=torch.bfloat16, device=dev),
                          dX=torch.empty((M, K), dtype=torch.bfloat16, device=dev),
                          dA=torch.empty((G * r, K), dtype=torch.float32, device=dev),
                          dB=torch.empty((N, G * r), dtype=torch.float32, device=dev),
                          ws=q.workspace(q.qlora_grouped_workspace_bytes(M, N, K, r, G), dev)))
    return units


def unit_step(q, units, r, alpha):
    """Forward of every unit in layer order, then the backward in reverse."""
    for u in units:
        if u["single"]:
            q.qlora_linear_fwd(u["q"], u["X"], u["A"], u["B"], alpha, Y=u["Y"], XA_out=u["XA"],
                               ws=u["ws"], return_xa=True)
        else:
            q.qlora_grouped_fwd(u["q"], u["X"], u["A"], u["B"], r, u["rows"], alpha, Y=u["Y"],
                                XA_out=u["XA"], ws=u["ws"], return_xa=True)
    for u in reversed(units):
        if u["single"]:
            q.qlora_linear_bwd(u["q"], u["X"], u["A"], u["B"], alpha, u["dY"], XA_in=u["XA"],
                               dX=u["dX"], dA=u["dA"], dB=u["dB"], ws=u["ws"])
        else:
            q.qlora_grouped_bwd(u["q"], u["X"], u["A"], u["B"], r, u["rows"], alpha, u["dY"],
                                XA_in=u["XA"], dX=u["dX"], dA=u["dA"], dB=u["dB"], ws=u["ws"])


def separate_step(q, layers, alpha):
    for L in layers:
        q.qlora_linear_fwd(L["q"], L["X"], L["A"], L["B"], alpha, Y=L["Y"], XA_out=L["XA"],
                           ws=L["ws"], return_xa=True)
    for L in reversed(layers):
        q.qlora_linear_bwd(L["q"], L["X"], L["A"], L["B"], alpha, L["dY"], XA_in=L["XA"],
                           dX=L["dX"], dA=L["dA"], dB=L["dB"], ws=L["ws"])


def kernel_table(tr, kflops, launches_per_step, sampled):
    """Per-kernel averages from the traced launches: `kflops[name]` is the
    algorithmic flops of one step's launches of that kernel."""
    kern = {}
    for name, (n, ms) in tr.items():
        if not n:
            continue
        ent = {"launches": n, "avg_launch_us": round(ms * 1e3 / n, 2),
               "us_per_step": round(ms * 1e3 / len(sampled), 2)}
        if name in kflops:
            per_launch = kflops[name] / launches_per_step[name]
            tf = per_launch * n / (ms * 1e-3) / 1e12
            ent.update({"flops_per_launch": per_launch, "tflops": round(tf, 2),
                        "frac": round(tf / PEAK_BF16_TFLOPS, 4)})
        kern[name] = ent
    return kern


KERNEL_SYMBOL = {"fwd_gemm": "k_qlora_fwd_nt", "dx_gemm": "k_qlora_dx_nn_dma<false>"}


def roofline_of(kern):
    """The roofline object of whichever GEMM takes more time per step."""
    dom = max((k for k in kern if "tflops" in kern[k]), key=lambda k: kern[k]["us_per_step"])
    d = kern[dom]
    roof = {"kernel": KERNEL_SYMBOL[dom], "bound": "mfma", "achieved": d["tflops"],
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": d["frac"], "traffic": None,
            "avg_launch_us": d["avg_launch_us"], "flops_per_launch": d["flops_per_launch"]}
    roof["traffic"] = traffic_for(roof["kernel"])
    return roof


def timed_steps(args, q, torch, step, traced, capacity):
    """W untimed steps, then K timed steps between two synchronisations.  The
    kernels in `traced` record their own start and end on a sample of the
    timed steps (every tenth, at least one): a self-timed dispatch idles the
    GPU for a few microseconds around it, so the step time carries little of
    that cost."""
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    sampled = [i for i in range(args.steps) if i % 10 == 5] or [args.steps - 1]
    q.qlora_trace_begin(traced, capacity=capacity * len(sampled) + 8)
    q.qlora_trace_pause(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i in sampled:
            q.qlora_trace_pause(False)
            step()
            q.qlora_trace_pause(True)
        else:
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    tr = q.qlora_trace_end()
    return (t1 - t0) / args.steps, tr, sampled


def headline(args, q, torch, workloads):
    """fwd + bwd through 80 LLaMA-65B layers (7 linears each, distinct NF4
    weights), 4096 tokens, r = 64, alpha = 16.  The layers' weights are drawn
    and quantised on the device; the activations, adapters and output buffers
    of one shape are shared by the layers (they are a few hundred MB, the
    weights 33 GB)."""
    dev = "cuda:0"
    wl = workloads.LLAMA65B_LAYER
    M, r, alpha = wl.m, wl.r, wl.alpha
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    qws = q.workspace(max(q.qlora_quantize_workspace_bytes(n, k) for _, k, n in wl.linears), dev)
    lin = []
    for layer in range(wl.layers):
        for t, (name, K, N) in enumerate(wl.linears):
            W = workloads.device_weight(3, layer, t, N, K)
            Q, _ = q.qlora_quantize_nf4(W, ws=qws)
            del W
            lin.append((Q, K, N))
        if layer % 20 == 19:
            torch.cuda.synchronize()
            log("headline: %d/%d layers quantised" % (layer + 1, wl.layers))
    del qws
    torch.cuda.empty_cache()
    shp = {(K, N) for _, K, N in wl.linears}
    X = {K: torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16) for K, _ in shp}
    dY = {N: torch.randn((M, N), generator=g, device=dev).to(torch.bfloat16) for _, N in shp}
    A = {K: ((torch.rand((r, K), generator=g, device=dev) * 2 - 1) * K ** -0.5).to(torch.bfloat16)
         for K, _ in shp}
    B = {N: (torch.randn((N, r), generator=g, device=dev) * 0.01).to(torch.bfloat16) for _, N in shp}
    # one output and XA per projection of a layer (the batched forward writes
    # several at once)
    Y = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _, _, N in wl.linears]
    XA = [torch.empty((M, r), dtype=torch.bfloat16, device=dev) for _ in wl.linears]
    dX = {K: torch.empty((M, K), dtype=torch.bfloat16, device=dev) for K, _ in shp}
    dA = {K: torch.empty((r, K), dtype=torch.float32, device=dev) for K, _ in shp}
    dB = {N: torch.empty((N, r), dtype=torch.float32, device=dev) for _, N in shp}
    ws = q.workspace(max(q.qlora_linear_workspace_bytes(M, N, K, r) for K, N in shp), dev)
    # the layer driver's forward: the projections that read one input (q/k/v,
    # gate/up) as one batched call, whose consecutive same-K pairs share a
    # GEMM launch (q+k, gate+up: 5 forward GEMM launches per layer)
    names = [nm for nm, _, _ in wl.linears]
    groups = [[names.index(n) for n in grp] for grp in (("q_proj", "k_proj", "v_proj"),
                                                         ("o_proj",), ("gate_proj", "up_proj"),
                                                         ("down_proj",))]
    per = len(wl.linears)
    bws = q.workspace(max(q.qlora_linear_batch_workspace_bytes([lin[i][0] for i in grp], M, r)
                          for grp in groups), dev)
    fwd_launches = wl.layers * sum((len(grp) + 1) // 2 for grp in groups)
    torch.cuda.synchronize()
    log("headline inputs ready (%d linears, %.1f GB of quantised weights)"
        % (len(lin), sum(Q.nbytes() for Q, _, _ in lin) / 1e9))

    def step():
        for layer in range(wl.layers):
            for grp in groups:
                jobs = [(lin[layer * per + t][0], X[lin[layer * per + t][1]],
                         A[lin[layer * per + t][1]], B[lin[layer * per + t][2]], Y[t]) for t in grp]
                if len(jobs) == 1:
                    Q, Xj, Aj, Bj, Yj = jobs[0]
                    q.qlora_linear_fwd(Q, Xj, Aj, Bj, alpha, Y=Yj, XA_out=XA[grp[0]], ws=ws,
                                       return_xa=True)
                else:
                    q.qlora_linear_fwd_batch(jobs, alpha, ws=bws, XA_out=[XA[t] for t in grp])
        for i in reversed(range(len(lin))):
            Q, K, N = lin[i]
            q.qlora_linear_bwd(Q, X[K], A[K], B[N], alpha, dY[N], XA_in=XA[i % per], dX=dX[K],
                               dA=dA[K], dB=dB[N], ws=ws)

    sec, tr, sampled = timed_steps(args, q, torch, step, ["fwd_gemm", "dx_gemm", "split_reduce"],
                                   capacity=2 * len(lin) + 8)
    flops = sum(linear_flops(M, N, K, r) for _, K, N in lin)
    # per-kernel algorithmic flops: fwd GEMM 2MN(K + r), dX GEMM 2MK(N + r)
    kflops = {"fwd_gemm": sum(2 * M * N * (K + r) for _, K, N in lin),
              "dx_gemm": sum(2 * M * K * (N + r) for _, K, N in lin)}
    kern = kernel_table(tr, kflops, {"fwd_gemm": fwd_launches, "dx_gemm": len(lin)}, sampled)
    roof = roofline_of(kern)
    roof["timed_steps"] = sampled
    log("headline: %.4f s/step, %.1f TFLOP/s" % (sec, flops / sec / 1e12))
    res = dict(sec=sec, tokens=M, flops=flops, roofline=roof, kernels=kern)
    del lin, X, dY, A, B, Y, dX, dA, dB, XA, ws, bws
    torch.cuda.empty_cache()
    return res


def leg_layer8b(args, q, torch, workloads):
    """fwd + bwd through the seven Llama-3.1-8B layer projections at 2048
    tokens, r = 16, alpha = 32, run by the layer driver (q/k/v and gate/up as
    grouped weights: 4 fused-GEMM pairs)."""
    wl = workloads.LLAMA8B_LAYER
    dev = "cuda:0"
    M, r, alpha = wl.m, wl.r, wl.alpha
    layers = []
    host_w = []
    for t, (name, K, N) in enumerate(wl.linears):
        w, x, a, b, dy = workloads.linear_inputs(wl, 0, t)
        qq, _ = q.qlora_quantize_nf4(torch.from_numpy(w).to(dev))
        host_w.append(w)
        L = dict(name=name, N=N, K=K, q=qq, X=x.to(dev), A=a.to(dev), B=b.to(dev), dY=dy.to(dev))
        L["Y"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        L["XA"] = torch.empty((M, r), dtype=torch.bfloat16, device=dev)
        L["dX"] = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        L["dA"] = torch.empty((r, K), dtype=torch.float32, device=dev)
        L["dB"] = torch.empty((N, r), dtype=torch.float32, device=dev)
        L["ws"] = q.workspace(q.qlora_linear_workspace_bytes(M, N, K, r), dev)
        layers.append(L)
    units = build_units(q, torch, layers, host_w, M, r)
    torch.cuda.synchronize()
    log("8B layer leg: inputs ready (%d linears in %d units)" % (len(layers), len(units)))

    def step():
        unit_step(q, units, r, alpha)

    sec, tr, sampled = timed_steps(args, q, torch, step, ["fwd_gemm", "dx_gemm", "split_reduce"],
                                   capacity=4 * len(units) + 8)
    flops = sum(linear_flops(M, L["N"], L["K"], r) for L in layers)
    # fwd GEMM 2MN(K + r) (each row of W meets one adapter of rank r), dX
    # GEMM 2MK(N + G r) (G adapters of a grouped unit)
    kflops = {"fwd_gemm": sum(2 * M * u["N"] * (u["K"] + r) for u in units),
              "dx_gemm": sum(2 * M * u["K"] * (u["N"] + u.get("G", 1) * r) for u in units)}
    kern = kernel_table(tr, kflops, {"fwd_gemm": len(units), "dx_gemm": len(units)}, sampled)
    res = {"workload": "Llama-3.1-8B layer linears q/k/v/o/gate/up/down, 2048 tokens, LoRA r=16 "
                       "alpha=32, NF4 + double quant, fwd+bwd, layer driver (q/k/v and gate/up "
                       "grouped: 4 fused-GEMM pairs)",
           "ms_per_step": round(sec * 1e3, 4), "tokens/s": round(M / sec, 1),
           "TFLOP/s": round(flops / sec / 1e12, 2),
           "frac_mfma": round(flops / sec / 1e12 / PEAK_BF16_TFLOPS, 4),
           "kernels": kern, "timed_steps": sampled}
    log("8B layer leg: %.3f ms/step, %.1f TFLOP/s" % (sec * 1e3, flops / sec / 1e12))
    return res, layers, units


# ---------------------------------------------------------- cpu baseline
def cpu_baseline(workloads, sample_tokens=256):
    """The oracle as it stands, on a bounded sample of the headline step: for
    layer 0 of the 65B stack, the float32 dequantisation of its seven weights
    (once per step, as the GPU path rebuilds them every step) plus the
    float64 fwd+bwd of `sample_tokens` of the 4096 tokens; the linear part is
    scaled to 4096 tokens and the layer to 80 layers."""
    import numpy as np
    import oracle
    try:
        import threadpoolctl
        blas = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    except Exception:
        blas = 1
    wl = workloads.LLAMA65B_LAYER
    t_deq = t_lin = 0.0
    for t, (name, K, N) in enumerate(wl.linears):
        w = workloads.weight(wl.key, 0, t, N, K)
        qt = oracle.quantize(w)                            # load-time, untimed
        del w
        x = workloads.activations(wl.key, 0, t, sample_tokens, K)
        dy = workloads.activations(wl.key, 0, t, sample_tokens, N, workloads.ROLE_DY)
        a = workloads.lora_a(wl.key, 0, t, wl.r, K)
        b = workloads.lora_b(wl.key, 0, t, N, wl.r)
        xs, dys = workloads.bf16_to_f64(x), workloads.bf16_to_f64(dy)
        af, bfl = workloads.bf16_to_f64(a), workloads.bf16_to_f64(b)
        t0 = time.perf_counter()
        wd = oracle.dequantize(qt).reshape(N, K)
        t1 = time.perf_counter()
        oracle.linear_fwd(wd, xs, af, bfl, wl.alpha)
        oracle.linear_bwd(wd, xs, af, bfl, wl.alpha, dys)
        t2 = time.perf_counter()
        t_deq += t1 - t0
        t_lin += t2 - t1
        del qt, wd
    layer = t_deq + t_lin * (wl.m / sample_tokens)
    step = wl.layers * layer
    return {"value": round(wl.m / step, 3), "unit": "tokens/s",
            "cores": int(max(blas, oracle.threads())), "nproc": os.cpu_count(),
            "kind": "oracle",
            "sample": ("layer 0 of the 65B stack: dequantise its 7 weights (%.2f s) + float64 "
                       "fwd+bwd of %d of the 4096 tokens (%.2f s); linear part scaled x%d, "
                       "layer x%d" % (t_deq, sample_tokens, t_lin, wl.m // sample_tokens,
                                      wl.layers))}


# -------------------------------------------------------------------- legs
def leg_quant_dequant(q, torch, workloads, passes=3):
    """Quantise then dequantise (to bf16) every 2-D weight of the 8.03B set,
    each pass one batched call over all the tensors (up to 32 per launch)."""
    dev = "cuda:0"
    specs = workloads.llama8b_weight_set()
    Ws, Qs = [], []
    for i, (name, layer, rows, cols) in enumerate(specs):
        Ws.append(workloads.device_weight(2, layer, i, rows, cols))
        Qs.append(q.NF4Tensor(rows, cols, dev))
    ws = q.workspace(q.qlora_quantize_batch_workspace_bytes([(r, c) for _, _, r, c in specs]), dev)
    out = torch.empty(sum(r * c for _, _, r, c in specs), dtype=torch.bfloat16, device=dev)
    outs, off = [], 0
    for Q in Qs:
        outs.append(out[off: off + Q.numel].view(Q.rows, Q.cols))
        off += (Q.numel + 7) // 8 * 8            # 16-byte aligned starts
    params = sum(r * c for _, _, r, c in specs)
    log("quant leg: %d tensors, %.3fB params on device" % (len(specs), params / 1e9))

    def quant_pass():
        q.qlora_quantize_nf4_batch(Ws, Qs, ws)

    def deq_pass():
        q.qlora_dequantize_nf4_batch(Qs, outs)

    single_ws = q.workspace(max(q.qlora_quantize_workspace_bytes(r, c) for _, _, r, c in specs), dev)

    def quant_single():
        for W, Q in zip(Ws, Qs):
            q.qlora_quantize_nf4(W, Q, single_ws)

    quant_pass(); deq_pass(); quant_single()
    torch.cuda.synchronize()
    # eager passes, kernel durations traced
    q.qlora_trace_begin(["quantize", "dequant"], capacity=len(specs) * passes + 4)
    tq_eager = timed(torch, quant_pass, passes)
    td_eager = timed(torch, deq_pass, passes)
    tr = q.qlora_trace_end()
    # the batched calls and, for comparison, the per-tensor calls replayed from
    # HIP graphs (no host work between the launches)
    gq, gd, gs = graph_of(torch, quant_pass), graph_of(torch, deq_pass), graph_of(torch, quant_single)
    tq = timed(torch, gq.replay, passes)
    td = timed(torch, gd.replay, passes)
    tq_single = timed(torch, gs.replay, passes)
    del gq, gd, gs
    nbytes = sum(Q.nbytes() for Q in Qs)
    bpp = 8.0 * nbytes / params
    # algorithmic bytes: quantise reads 4 B and writes the 4.127-bit state;
    # dequantise reads the state and writes 2 B (bf16)
    qbytes = 4 * params + nbytes
    dbytes = nbytes + 2 * params
    res = {"params": params, "bits_per_param": round(bpp, 5),
           "quantize": {"ms": round(tq * 1e3, 3), "GB/s": round(qbytes / tq / 1e9, 1),
                        "frac_hbm": round(qbytes / tq / 1e9 / PEAK_HBM_GBS, 4),
                        "launch": "hip graph of one batched call",
                        "eager_ms": round(tq_eager * 1e3, 3),
                        "per_tensor_calls_graph_ms": round(tq_single * 1e3, 3)},
           "dequantize_bf16": {"ms": round(td * 1e3, 3), "GB/s": round(dbytes / td / 1e9, 1),
                               "frac_hbm": round(dbytes / td / 1e9 / PEAK_HBM_GBS, 4),
                               "launch": "hip graph of one batched call",
                               "eager_ms": round(td_eager * 1e3, 3)}}
    for name, (n, ms) in tr.items():
        # the code kernel alone (quantise: 4 B in, half a byte of codes and the
        # float32 absmax out per weight); n launches over `passes` passes
        kb = (4 * params + params / 2 + params / 16) if name == "quantize" else dbytes
        res[name + "_kernel"] = {"launches": n, "avg_us": round(ms / n * 1e3, 2),
                                 "GB/s": round(kb * passes / (ms * 1e-3) / 1e9, 1)}
    del Ws, Qs, out, outs, ws, single_ws
    torch.cuda.empty_cache()
    log("quant leg: quantise %.2f ms, dequantise %.2f ms, %.4f bits/param" % (tq * 1e3, td * 1e3, bpp))
    return res


def leg_dropout(q, torch, layers, M, r, alpha, p=0.05, steps=10):
    """The headline layer step with LoRA dropout p on every adapter input
    (the Practical Implementation section's lora_dropout), against the same
    step without: eager step time and the dX GEMM's average launch (which
    starts its accumulators from the masked LoRA term), from HIP events."""

    bits = [q.keep_bits_buffer(M, L["K"], "cuda:0") for L in layers]

    def step(drop, keep):
        for i, L in enumerate(layers):
            d = None if drop is None else (drop, 1000 + i)
            q.qlora_linear_fwd(L["q"], L["X"], L["A"], L["B"], alpha, Y=L["Y"], XA_out=L["XA"],
                               ws=L["ws"], return_xa=True, dropout=d,
                               keep_bits=bits[i] if keep else None)
        for i, L in reversed(list(enumerate(layers))):
            d = None if drop is None else (drop, 1000 + i)
            q.qlora_linear_bwd(L["q"], L["X"], L["A"], L["B"], alpha, L["dY"], XA_in=L["XA"],
                               dX=L["dX"], dA=L["dA"], dB=L["dB"], ws=L["ws"], dropout=d,
                               keep_bits=bits[i] if keep else None)

    res = {"p": p, "seeds": "1000 + linear index",
           "dropout": "the forward stores the keep bits, the backward reads them",
           "dropout_regenerate": "the backward runs the generator again"}
    cfgs = (("no_dropout", None, False), ("dropout", p, True), ("dropout_regenerate", p, False))
    best = {}
    for _ in range(3):   # alternate the configurations; keep each one's best
        for label, drop, keep in cfgs:
            step(drop, keep)
            sec = timed(torch, lambda: step(drop, keep), steps)
            best[label] = min(best.get(label, sec), sec)
    for label, drop, keep in cfgs:
        sec = best[label]
        q.qlora_trace_begin(["dx_gemm"], capacity=len(layers) + 1)
        step(drop, keep)
        tr = q.qlora_trace_end()
        n, ms = tr.get("dx_gemm", (0, 0.0))
        res["step_ms_" + label] = round(sec * 1e3, 4)
        res["dx_gemm_avg_us_" + label] = round(ms * 1e3 / max(n, 1), 2)
    res["tokens_per_s_dropout"] = round(M / (res["step_ms_dropout"] * 1e-3), 1)
    res["step_overhead_pct"] = round(
        100.0 * (res["step_ms_dropout"] / res["step_ms_no_dropout"] - 1.0), 2)
    log("dropout leg: %.3f ms/step with p=%.2f, %.3f without" %
        (res["step_ms_dropout"], p, res["step_ms_no_dropout"]))
    return res


def leg_layer_driver(q, torch, layers, units, M, r, alpha, steps=10):
    """The layer step as 7 separate linears against the grouped units of the
    headline (q/k/v and gate/up each one grouped weight), both eager, on the
    same inputs."""
    res = {"units": "q/k/v grouped, o, gate/up grouped, down"}
    best = {}
    for _ in range(3):   # alternate the two; keep each one's best
        for label, fn in (("separate_7", lambda: separate_step(q, layers, alpha)),
                          ("grouped_4", lambda: unit_step(q, units, r, alpha))):
            fn()
            sec = timed(torch, fn, steps)
            best[label] = min(best.get(label, sec), sec)
    for label, sec in best.items():
        res["step_ms_" + label] = round(sec * 1e3, 4)
        res["tokens_per_s_" + label] = round(M / sec, 1)
    res["speedup"] = round(res["step_ms_separate_7"] / res["step_ms_grouped_4"], 4)
    log("layer driver leg: %.3f ms grouped, %.3f ms separate" %
        (res["step_ms_grouped_4"], res["step_ms_separate_7"]))
    return res


def leg_adamw(q, torch, workloads, reps=10):
    """The adapter optimiser step over every adapter of Llama-3.1-8B at r = 16
    (32 layers x 7 projections x {A, B} = 448 tensors, 41.9M parameters):
    float32 masters, gradients and statistics, bf16 copies written in the same
    pass.  Algorithmic HBM bytes per parameter: 16 read + 14 written.  Then the
    same step with both statistics in mapped host memory (16 bytes per
    parameter cross the host link), and both again with 8-bit statistics
    (2 + 8/256 bytes of state per parameter)."""
    dev = "cuda:0"
    wl = workloads.LLAMA8B_LAYER
    r = wl.r
    shapes = []
    for _ in range(wl.layers):
        for _, K, N in wl.linears:
            shapes += [(r, K), (N, r)]
    total = sum(a * b for a, b in shapes)
    g = torch.Generator(device=dev)
    g.manual_seed(8)
    P = torch.randn(total, generator=g, device=dev) * 0.02
    G = torch.randn(total, generator=g, device=dev) * 1e-3
    M = torch.zeros(total, device=dev)
    V = torch.zeros(total, device=dev)
    PB = torch.empty(total, dtype=torch.bfloat16, device=dev)

    def views(m_all, v_all):
        out, off = [], 0
        for a, b in shapes:
            n = a * b
            out.append((P[off:off + n], G[off:off + n], m_all[off:off + n], v_all[off:off + n],
                        PB[off:off + n]))
            off += n
        return out

    res = {"tensors": len(shapes), "params": total, "hparams": "lr 2e-4, betas (0.9, 0.999), "
           "eps 1e-8, weight decay 0.01",
           "flat": "device_statistics_flat: the same parameters as one flat tensor"}
    hs = []
    for label in ("device_statistics", "device_statistics_flat", "host_statistics"):
        if label == "host_statistics":
            hs = [q.qlora_host_state_alloc(total) for _ in range(2)]
            hs[0].tensor.zero_()
            hs[1].tensor.zero_()
            ts = views(hs[0].tensor, hs[1].tensor)
        elif label == "device_statistics_flat":
            ts = [(P, G, M, V, PB)]
        else:
            ts = views(M, V)

        def step():
            q.qlora_adamw_step(ts, 1, 2e-4, 0.9, 0.999, 1e-8, 0.01)

        step()
        gr = graph_of(torch, step)
        sec = timed(torch, gr.replay, reps)
        del gr
        q.qlora_trace_begin(["adamw"], capacity=64)
        step()
        tr = q.qlora_trace_end()
        n, ms = tr.get("adamw", (0, 0.0))
        ent = {"step_ms": round(sec * 1e3, 4), "launches": n,
               "kernel_ms": round(ms, 4)}
        if label != "host_statistics":
            gbs = 30.0 * total / sec / 1e9
            ent.update({"hbm_GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
        else:
            ent["host_link_GB/s"] = round(16.0 * total / sec / 1e9, 2)
        res[label] = ent
    for h in hs:
        h.free()
    del M, V
    # 8-bit statistics (blocks of 256, codes plus a float32 scale per block):
    # every adapter size is a multiple of 256, so each tensor's state is a
    # view of one flat state on block boundaries
    for label, on_host in (("device_statistics_8bit", False), ("host_statistics_8bit", True)):
        flat = q.AdamW8State(total, dev, host=on_host)
        ts, off = [], 0
        for a, b in shapes:
            n = a * b
            assert n % q.ADAMW8_BLOCK == 0
            v = type("StateView", (), {})()
            v.numel = n
            v.m_q, v.v_q = flat.m_q[off:off + n], flat.v_q[off:off + n]
            bo, bn = off // q.ADAMW8_BLOCK, n // q.ADAMW8_BLOCK
            v.m_scale, v.v_scale = flat.m_scale[bo:bo + bn], flat.v_scale[bo:bo + bn]
            ts.append((P[off:off + n], G[off:off + n], v, PB[off:off + n]))
            off += n

        def step8():
            q.qlora_adamw8_step(ts, 1, 2e-4, 0.9, 0.999, 1e-8, 0.01)

        step8()
        gr = graph_of(torch, step8)
        sec = timed(torch, gr.replay, reps)
        del gr
        q.qlora_trace_begin(["adamw8"], capacity=64)
        step8()
        tr = q.qlora_trace_end()
        n, ms = tr.get("adamw8", (0, 0.0))
        ent = {"step_ms": round(sec * 1e3, 4), "launches": n, "kernel_ms": round(ms, 4),
               "state_bytes_per_param": round(flat.nbytes() / total, 4)}
        # algorithmic bytes: p, g, 2 codes and 2/256 scales read; p, 2 codes,
        # 2/256 scales and the bf16 copy written
        if not on_host:
            gbs = (18.0 + 16.0 / 256) * total / sec / 1e9
            ent.update({"hbm_GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
        else:
            ent["host_link_GB/s"] = round((4.0 + 16.0 / 256) * total / sec / 1e9, 2)
        res[label] = ent
        torch.cuda.synchronize()
        ts = None
        flat.free()
        del flat
    # the placement policy: an HBM budget of half the 8-bit statistics' bytes;
    # the largest tensors' statistics stay on the device, the rest are mapped
    # from host memory
    numels = [a * b for a, b in shapes]
    need = sum(q.adamw8_state_bytes(n) for n in numels)
    states = q.adamw8_states(numels, dev, hbm_budget=need // 2)
    ts, off = [], 0
    for n, st in zip(numels, states):
        ts.append((P[off:off + n], G[off:off + n], st, PB[off:off + n]))
        off += n

    def step_half():
        q.qlora_adamw8_step(ts, 1, 2e-4, 0.9, 0.999, 1e-8, 0.01)

    step_half()
    gr = graph_of(torch, step_half)
    sec = timed(torch, gr.replay, reps)
    del gr
    on_host = sum(st.nbytes() for st in states if st.on_host)
    res["half_hbm_statistics_8bit"] = {
        "step_ms": round(sec * 1e3, 4), "hbm_budget_bytes": need // 2,
        "host_state_bytes": on_host, "host_tensors": sum(1 for st in states if st.on_host),
        "placement": "plan_state_placement: largest tensors in HBM until the budget is spent"}
    torch.cuda.synchronize()
    ts = None
    for st in states:
        st.free()
    del states
    del P, G, PB
    torch.cuda.empty_cache()
    log("adamw leg: %.3f / %.3f ms with float32 / 8-bit device statistics, %.3f / %.3f ms "
        "with host statistics" % (res["device_statistics"]["step_ms"],
                                  res["device_statistics_8bit"]["step_ms"],
                                  res["host_statistics"]["step_ms"],
                                  res["host_statistics_8bit"]["step_ms"]))
    return res


def leg_variants(q, torch, workloads, passes=3):
    """The 4-bit type and constant variants on the same kernels, over the seven
    weights of one Llama-3.1-8B layer: quantise and dequantise (bf16) GB/s and
    bits/param for NF4 and INT4, with and without double quantisation; the
    reconstruction error of each type on these N(0, 0.02) weights; and the
    fused fwd+bwd of the gate projection at 2048 tokens for each variant."""
    dev = "cuda:0"
    wl = workloads.LLAMA8B_LAYER
    Ws = [workloads.device_weight(5, 0, t, n, k) for t, (_, k, n) in enumerate(wl.linears)]
    params = sum(W.numel() for W in Ws)
    ws = q.workspace(max(q.qlora_quantize_workspace_bytes(*W.shape) for W in Ws), dev)
    out = torch.empty(max(W.numel() for W in Ws), dtype=torch.bfloat16, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(6)
    M, r, alpha = wl.m, wl.r, wl.alpha
    _, Kg, Ng = wl.linears[4]   # gate projection
    X = torch.randn((M, Kg), generator=g, device=dev).to(torch.bfloat16)
    A = (torch.rand((r, Kg), generator=g, device=dev) * 2 - 1).mul_(Kg ** -0.5).to(torch.bfloat16)
    B = (torch.randn((Ng, r), generator=g, device=dev) * 0.01).to(torch.bfloat16)
    dY = torch.randn((M, Ng), generator=g, device=dev).to(torch.bfloat16)
    lws = q.workspace(q.qlora_linear_workspace_bytes(M, Ng, Kg, r), dev)
    res = {"tensors": "q/k/v/o/gate/up/down of one Llama-3.1-8B layer", "params": params}
    for kind in ("nf4", "int4"):
        for dq in (True, False):
            Qs = [q.NF4Tensor(W.shape[0], W.shape[1], dev, kind, dq) for W in Ws]

            def quant_pass():
                for W, Q in zip(Ws, Qs):
                    q.qlora_quantize_nf4(W, Q, ws)

            def deq_pass():
                for Q in Qs:
                    q.qlora_dequantize_nf4(Q, out=out[: Q.numel].view(Q.rows, Q.cols))

            quant_pass(); deq_pass()
            gq, gd = graph_of(torch, quant_pass), graph_of(torch, deq_pass)
            tq = timed(torch, gq.replay, passes)
            td = timed(torch, gd.replay, passes)
            del gq, gd
            nbytes = sum(Q.nbytes() for Q in Qs)
            sq = 0.0
            for W, Q in zip(Ws, Qs):
                back = q.qlora_dequantize_nf4(Q, torch.float32)
                sq += float(((back.double() - W.double()) ** 2).sum().item())
            Qg = Qs[4]
            q.qlora_linear_fwd(Qg, X, A, B, alpha, ws=lws)
            torch.cuda.synchronize()

            def step():
                Y = q.qlora_linear_fwd(Qg, X, A, B, alpha, ws=lws)
                q.qlora_linear_bwd(Qg, X, A, B, alpha, dY, ws=lws)
                return Y

            tg = timed(torch, step, 5)
            res["%s_%s" % (kind, "dq" if dq else "f32_constants")] = {
                "bits_per_param": round(8.0 * nbytes / params, 5),
                "quantize_GB/s": round((4 * params + nbytes) / tq / 1e9, 1),
                "dequantize_bf16_GB/s": round((nbytes + 2 * params) / td / 1e9, 1),
                "mse": float("%.5g" % (sq / params)),
                "gate_fwd_bwd_ms": round(tg * 1e3, 3)}
            del Qs
    res["mse_ratio_nf4_over_int4"] = round(res["nf4_dq"]["mse"] / res["int4_dq"]["mse"], 4)
    del Ws, ws, out, lws
    torch.cuda.empty_cache()
    log("variants leg: NF4 / INT4 error ratio %.3f" % res["mse_ratio_nf4_over_int4"])
    return res


def leg_decode(q, torch, workloads, steps=5):
    """Decode forward through 80 layers x 7 70B-shaped linears (distinct NF4
    weights, ~35 GB) at M = 1, 4, 16 tokens: as 560 separate calls, and as the
    layer driver (q/k/v and gate/up batched: 4 launch pairs per layer)."""
    dev = "cuda:0"
    wl = workloads.LLAMA70B_DECODE
    r, alpha = wl.r, wl.alpha
    lin = []
    qws = q.workspace(max(q.qlora_quantize_workspace_bytes(n, k) for _, k, n in wl.linears), dev)
    for layer in range(wl.layers):
        for t, (name, K, N) in enumerate(wl.linears):
            W = workloads.device_weight(4, layer, t, N, K)
            Q, _ = q.qlora_quantize_nf4(W, ws=qws)
            del W
            lin.append((Q, K, N))
        if layer % 20 == 19:
            torch.cuda.synchronize()
            log("decode leg: %d/%d layers quantised" % (layer + 1, wl.layers))
    del qws
    torch.cuda.empty_cache()
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    A = {K: (torch.rand((r, K), generator=g, device=dev) * 2 - 1).mul_(K ** -0.5).to(torch.bfloat16)
         for _, K, _ in wl.linears}
    B = {N: (torch.randn((N, r), generator=g, device=dev) * 0.01).to(torch.bfloat16)
         for _, _, N in wl.linears}
    out = {}
    for M in wl.decode_m:
        X = {K: torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16) for _, K, _ in wl.linears}
        Y = {N: torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _, _, N in wl.linears}
        ws = q.workspace(max(q.qlora_linear_workspace_bytes(M, N, K, r) for _, K, N in wl.linears), dev)
        names = [nm for nm, _, _ in wl.linears]
        # the layer driver: the projections that read one input (q/k/v, then
        # gate/up) as one batched call, o and down alone
        groups = [[names.index(n) for n in g] for g in (("q_proj", "k_proj", "v_proj"),
                                                         ("o_proj",), ("gate_proj", "up_proj"),
                                                         ("down_proj",))]
        Yl = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _, _, N in wl.linears]
        per = len(wl.linears)
        bws = q.workspace(max(q.qlora_linear_batch_workspace_bytes(
            [lin[i][0] for i in g], M, r) for g in groups), dev)

        def step():
            for Q, K, N in lin:
                q.qlora_linear_fwd(Q, X[K], A[K], B[N], alpha, Y=Y[N], ws=ws)

        def step_batched():
            for layer in range(wl.layers):
                for g in groups:
                    jobs = [(lin[layer * per + i][0], X[lin[layer * per + i][1]],
                             A[lin[layer * per + i][1]], B[lin[layer * per + i][2]], Yl[i])
                            for i in g]
                    if len(jobs) == 1:
                        Q, Xj, Aj, Bj, Yj = jobs[0]
                        q.qlora_linear_fwd(Q, Xj, Aj, Bj, alpha, Y=Yj, ws=ws)
                    else:
                        q.qlora_linear_fwd_batch(jobs, alpha, ws=bws)

        step()
        torch.cuda.synchronize()
        q.qlora_trace_begin(["gemv"], capacity=len(lin) * steps + 4)
        sec_eager = timed(torch, step, steps)
        tr = q.qlora_trace_end()
        # the 560 calls of a token step replayed from one HIP graph
        gstep = graph_of(torch, step)
        sec_sep = timed(torch, gstep.replay, steps)
        del gstep
        gstep = graph_of(torch, step_batched)
        sec = timed(torch, gstep.replay, steps)
        del gstep
        nb = sum(Q.nbytes() + 2 * r * (K + N) + 2 * M * (K + N) for Q, K, N in lin)
        code_bytes = sum(Q.nbytes() for Q, _, _ in lin)
        ent = {"ms_per_token_step": round(sec * 1e3, 3), "tokens/s": round(M / sec, 1),
               "GB/s": round(nb / sec / 1e9, 1), "frac_hbm": round(nb / sec / 1e9 / PEAK_HBM_GBS, 4),
               "launch": "hip graph; q/k/v and gate/up as batched calls (4 launch pairs per layer)",
               "separate_calls_ms_per_token_step": round(sec_sep * 1e3, 3),
               "eager_ms_per_token_step": round(sec_eager * 1e3, 3)}
        if "gemv" in tr:
            n, ms = tr["gemv"]
            ent["gemv_kernel"] = {"launches": n, "avg_us": round(ms / n * 1e3, 2),
                                  "GB/s": round(code_bytes * (n / len(lin)) / (ms * 1e-3) / 1e9, 1)}
        out["M=%d" % M] = ent
        log("decode leg M=%d: %.3f ms per token step" % (M, sec * 1e3))
    del lin
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the path is measured on a single MI355X "
              "(--gpus %d / WORLD_SIZE %d requested)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_quantized_lora_quant_amd as q
    import workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    q.lib()
    if args.calibrate_copy:
        calibrate_copy(torch, args.calibrate_copy)
    head = headline(args, q, torch, workloads) if args.headline == "on" else None
    cpu = None
    if head is not None and args.cpu_baseline == "on":
        cpu = cpu_baseline(workloads)
        log("cpu baseline: %s tokens/s on %d threads" % (cpu["value"], cpu["cores"]))
    legs = {}
    want = {"layer8b", "quant", "variants", "dropout", "driver", "adamw", "decode"} \
        if args.legs == "all" else (
        set() if args.legs == "none" else set(args.legs.split(",")))
    if want & {"layer8b", "dropout", "driver"}:
        wl = workloads.LLAMA8B_LAYER
        legs["llama8b_layer_step"], layers, units = leg_layer8b(args, q, torch, workloads)
        if "dropout" in want:
            legs["llama8b_layer_lora_dropout"] = leg_dropout(q, torch, layers, wl.m, wl.r,
                                                             wl.alpha)
        if "driver" in want:
            legs["llama8b_layer_driver_grouped"] = leg_layer_driver(q, torch, layers, units,
                                                                    wl.m, wl.r, wl.alpha)
        del layers, units
        torch.cuda.empty_cache()
    if "quant" in want:
        legs["llama8b_weight_set_quant_dequant"] = leg_quant_dequant(q, torch, workloads)
    if "variants" in want:
        legs["nf4_int4_and_constant_variants"] = leg_variants(q, torch, workloads)
    if "adamw" in want:
        legs["llama8b_adapters_adamw_step"] = leg_adamw(q, torch, workloads)
    if "decode" in want:
        legs["llama70b_decode_gemv"] = leg_decode(q, torch, workloads)
    if head is None:
        print(json.dumps({"headline": None, "legs": legs}), flush=True)
        return
    tokens_s = head["tokens"] / head["sec"]
    tflops = head["flops"] / head["sec"] / 1e12
    line = {
        "metric": "QLoRA linear fwd+bwd tokens/s (TFLOP/s, % MFMA peak); NF4 dequant/GEMV GB/s",
        "value": round(tokens_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["sec"] * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; random NF4-quantised weights, no checkpoint)",
        "config": {"workload": "LLaMA-65B layer linears q/k/v/o 8192->8192, gate/up "
                               "8192->22016, down 22016->8192, repeated 80x (distinct NF4 + "
                               "double-quant weights per layer), 4x1024 = 4096 tokens, LoRA "
                               "r=64 alpha=16 on all seven, fwd+bwd",
                   "tokens": 4096, "rank": 64, "layers": 80, "linears_per_layer": 7},
        "tflops": round(tflops, 2),
        "frac_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": head["roofline"],
        "kernels": head["kernels"],
        "cpu_baseline": cpu,
        "legs": legs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
