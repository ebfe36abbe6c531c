"""Benchmark of the split-backward stage on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama7b_stage4]

A step is one whole iteration of the stage's hot path over one batch: the
dW buffers are cleared, then F, B and W run for every microbatch in the
zero-bubble order (memory limit 2p) that the library's generator produces
for stage 3 of an emulated 8-stage pipeline, back to back on one stream with
all inputs already in HBM.  Adjacent W(j), W(j+1) of the order run as one W
pass over both microbatches (--no-w-pairs: each on its own).  `value` = linear-layer FLOPs of F + B + W
(2*M*N*K per product, attention and RMSNorm excluded from the count but not
from the time) / wall time of the step; `tflops_incl_attention` adds the
causal attention core's algorithmic flops to the numerator.

Extra fields on the JSON line:
* roofline: the W-pass GEMM kernel (the kernel with the largest share of the
  step time), its algorithmic flops / its average launch time, the launches
  replayed on the benchmark stream and timed with HIP events.  `traffic` is
  the HBM bytes per launch from the committed --pmc summary, or null when
  that summary was taken on other kernel sources.
* cpu_baseline: the fp64 oracle timed on this host on a bounded sample
  (one decoder layer, one microbatch, 256 tokens, full widths).
* executor_p8_stage3: the stage replayed with emulated arrivals (device-clock
  waits) for the 1F1B and zero-bubble orders; in-window idle of each, beside
  the simulator's prediction (see executor_idle); and interleaved 1F1B with
  the stage split into two chunks (interleaved_idle).
* memory_limit_sweep_p8_stage3: ZB(M) for M = 8 .. 16 replayed the same way,
  with the stash each order keeps resident at its peak (memory_limit_sweep).
* two_iterations_p8_stage3: two iterations back to back with a per-stage
  optimizer step between them (multi_iteration).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_FP8_TFLOPS = 5033.2   # MI355X dense fp8 MFMA (256 CU x 8192 flop/clk x 2.4 GHz)


def calibrate(stage, xs, ys, dys, dxs, n=5):
    """Median over n passes of the F, B and W pass times of microbatch 0 (ms)."""
    import torch
    samples = []
    for _ in range(n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        stage.zero_grad()
        ev[0].record()
        stage.fwd(0, xs[0], ys[0])
        ev[1].record()
        stage.bwd_input(0, dys[0], dxs[0])
        ev[2].record()
        stage.bwd_weight(0)
        ev[3].record()
        torch.cuda.synchronize()
        samples.append([ev[i].elapsed_time(ev[i + 1]) for i in range(3)])
    return tuple(sorted(col)[len(col) // 2] for col in zip(*samples))


def linear_flops_per_mb(s) -> float:
    """2*M*N*K of every linear product of F, B and W for one microbatch."""
    T, H, F = s.tokens, s.hidden, s.ffn
    if s.kind == "linear":
        return 3 * 2.0 * T * H * F
    if s.kind == "mlp":
        return 3 * 2 * 2.0 * T * H * F
    qkv = s.q_dim + 2 * s.kv_dim
    per_pass = 2.0 * T * H * (qkv + s.q_dim + 2 * F + F)
    return 3 * per_pass * s.n_layers


def attention_flops_per_mb(s) -> float:
    """Algorithmic flops of the causal attention core for one microbatch:
    forward 2 products over the causal half (4*T^2*d*heads/2), backward 2.5x
    the forward (5 products).  Not in `value`; reported beside it."""
    if s.kind != "llama":
        return 0.0
    fwd = 4.0 * s.tokens * s.tokens * s.head_dim * s.n_heads / 2
    return 3.5 * fwd * s.n_layers


def w_pass_gemms(s):
    """(M, N, K) of the W-pass products of one microbatch."""
    T, H, F = s.tokens, s.hidden, s.ffn
    if s.kind == "llama":
        qkv = s.q_dim + 2 * s.kv_dim
        return [(qkv, H, T), (H, s.q_dim, T), (2 * F, H, T), (H, F, T)] * s.n_layers
    if s.kind == "mlp":
        return [(F, H, T), (H, F, T)]
    return [(F, H, T)]


def issue_plan(order, pair_w=True):
    """The calls that issue `order` ((type, mb) ops): adjacent W(j), W(j+1)
    become one ("P", j), a W pass over both microbatches
    (zb_bwd_weight_accum_pair): the same work in the same order, with one
    fp32 read-modify-write of dW for the two."""
    plan, i = [], 0
    while i < len(order):
        t, j = order[i]
        if pair_w and t == "W" and i + 1 < len(order) and tuple(order[i + 1]) == ("W", j + 1):
            plan.append(("P", j))
            i += 2
        else:
            plan.append((t, j))
            i += 1
    return plan


def make_inputs(shape, m, device):
    import torch
    import synth
    xs = [synth.to_device(synth.make_x(shape, j), device) for j in range(m)]
    dys = [synth.to_device(synth.make_dy(shape, j), device) for j in range(m)]
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    out_w = shape.ffn if shape.kind == "linear" else shape.hidden
    ys = [torch.empty((shape.tokens, out_w), dtype=dt, device=device) for _ in range(m)]
    dxs = [torch.empty((shape.tokens, shape.hidden), dtype=dt, device=device) for _ in range(m)]
    return xs, ys, dys, dxs


def w_kernel_launches(shape, device):
    """Buffers and a closure that launches the W-pass GEMM kernel once per
    product of the stage (dW += dY^T X at the step's shapes, fp32 in place),
    through the C ABI on the current stream."""
    import torch
    import split_backward_amd as zb
    gem = w_pass_gemms(shape)
    bufs = []
    for (M, N, K) in gem:
        A = torch.randn((K, M), device=device).to(torch.bfloat16)
        B = torch.randn((K, N), device=device).to(torch.bfloat16)
        C = torch.zeros((M, N), device=device, dtype=torch.float32)
        bufs.append((A, B, C, M, N, K))

    def once():  # the W pass's products in one grouped launch, as the stage issues them
        zb.gemm_wgrad_group([b[0] for b in bufs], [b[1] for b in bufs], [b[2] for b in bufs],
                            [b[3] for b in bufs], [b[4] for b in bufs], [b[5] for b in bufs])

    return gem, once


W_KERNEL = "gemm_v2_group_kernel<false,false,EPI_ACCUM_F32>"
W_KERNEL_SOURCES = ("split_backward_amd/csrc/gemm_v2.hip", "split_backward_amd/csrc/common.h")
# Counter summaries of the W kernel's HBM traffic, by workload.
TRAFFIC_SUMMARIES = {"llama7b_stage4": "profiles/gemm_w_kernel_hbm_traffic_llama7b_stage4.md",
                     "llama7b_stage4_fp8": "profiles/gemm_w_fp8_kernel_hbm_traffic_llama7b_stage4_fp8.md",
                     "llama70b_slice2": "profiles/gemm_w_kernel_hbm_traffic_llama70b_slice2.md"}


COMMON_H_END = "// ------------------------------------------------- elementwise / norms ----"


def kernel_source_hash() -> str:
    """sha256 prefix of the W kernel's sources with comments and whitespace
    removed (a comment edit does not invalidate the measured traffic): all of
    gemm_v2.hip, and common.h up to its elementwise / norms section (the
    types and GEMM declarations the kernel is built from)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in W_KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            src = fh.read()
        if f.endswith("common.h"):
            cut = src.find(COMMON_H_END)
            if cut < 0:
                raise RuntimeError(f"{f}: section marker missing")
            src = src[:cut]
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update("".join(src.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per W-kernel launch from the committed rocprofv3 --pmc
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the same counters' reading
    for a copy kernel of known size), or None when the summary is missing,
    covers another workload or was taken on other kernel sources."""
    import re
    if workload not in TRAFFIC_SUMMARIES:
        return None
    try:
        with open(os.path.join(ROOT, TRAFFIC_SUMMARIES[workload])) as fh:
            txt = fh.read()
    except OSError:
        return None
    mh = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", txt)
    mb = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    mw = re.search(r"workload:\s*(\S+)", txt)
    if not mh or not mb or not mw or mh.group(1) != kernel_source_hash() or mw.group(1) != workload:
        return None
    return float(mb.group(1))


def time_w_kernel(shape, workload, device, reps=5):
    """Average launch time of the W-pass GEMM kernel at the step's shapes,
    launched through the C ABI on the current stream, timed with events."""
    import torch
    gem, once = w_kernel_launches(shape, device)
    once()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        once()
    e1.record()
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    launches = reps * ((len(gem) + 15) // 16)  # 16 products per grouped launch
    flops = reps * sum(2.0 * M * N * K for M, N, K in gem)
    avg_ms = ms_total / launches
    achieved = flops / (ms_total * 1e-3) / 1e12
    algo_bytes = sum(2 * K * (M + N) + 2 * 4 * M * N for M, N, K in gem) / ((len(gem) + 15) // 16)
    traffic = measured_traffic(workload)
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
            "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes_per_launch": algo_bytes,
            # stash reads (dY, X) and the fp32 dW read-modify-write per launch,
            # over the launch time; and the measured HBM traffic over the same time
            "stash_and_dw_GBps": round(algo_bytes / (avg_ms * 1e-3) / 1e9, 1),
            "hbm_GBps": round(traffic / (avg_ms * 1e-3) / 1e9, 1) if traffic else None,
            "kernel": W_KERNEL + " (W pass: dW += dY^T X for every product of a microbatch, fp32 in place)",
            "avg_launch_us": round(avg_ms * 1e3, 1), "launches_timed": launches}


def w_kernel_launches_fp8(shape, device):
    """The fp8 stage's W-pass products (E4M3 codes of dY^T and X^T, both
    K-contiguous, fp32 dW in place) at the step's shapes, and a closure
    issuing them as one grouped launch per 16 products.  The codes are the
    library's own quantization of normal bf16 [K, M] and [K, N] tensors into
    their transposed layout, as the stage stashes its activations and
    gradients (uniformly random codes would not have the value distribution
    of the stage's operands)."""
    import torch
    import split_backward_amd as zb
    gem = w_pass_gemms(shape)
    As, eas, Bs, ebs, Cs = [], [], [], [], []
    for (M, N, K) in gem:
        for rows_out, codes, exps in ((M, As, eas), (N, Bs, ebs)):
            src = torch.randn((K, rows_out), device=device).to(torch.bfloat16)
            qt = torch.empty((rows_out, K), dtype=torch.uint8, device=device)
            _, _, e = zb.quantize_e4m3(src, qt=qt)
            codes.append(qt)
            exps.append(e)
            del src
        Cs.append(torch.zeros((M, N), dtype=torch.float32, device=device))
    torch.cuda.synchronize()
    return gem, lambda: zb.gemm_fp8_wgrad_group(As, eas, Bs, ebs, Cs)


def time_w_kernel_fp8(shape, workload, device, reps=5):
    """The fp8 stage's W-pass launch (16 products on E4M3 codes, fp32 dW
    accumulated in place) at the step's shapes, replayed on the current
    stream and timed with HIP events, against the fp8 dense peak."""
    import torch
    gem, once = w_kernel_launches_fp8(shape, device)
    once()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        once()
    e1.record()
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    launches = reps * ((len(gem) + 15) // 16)
    flops = reps * sum(2.0 * M * N * K for M, N, K in gem)
    achieved = flops / (ms_total * 1e-3) / 1e12
    algo_bytes = sum(K * (M + N) + 2 * 4 * M * N for M, N, K in gem) / ((len(gem) + 15) // 16)
    avg_ms = ms_total / launches
    traffic = measured_traffic(workload)
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
            "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes_per_launch": algo_bytes,
            "stash_and_dw_GBps": round(algo_bytes / (avg_ms * 1e-3) / 1e9, 1),
            "hbm_GBps": round(traffic / (avg_ms * 1e-3) / 1e9, 1) if traffic else None,
            "kernel": "gemm_f8_group_kernel<EPI_ACCUM_F32> (fp8 W pass: dW += dY^T X on E4M3 codes, fp32 in place)",
            "avg_launch_us": round(avg_ms * 1e3, 1), "launches_timed": launches}


def traffic_probe(shape, device, fp8=False):
    """Workload for the rocprofv3 --pmc passes: a copy of known size (1 GiB
    read, 1 GiB written, elementwise negation) three times, then the W-pass
    launches (bf16, or fp8 for the fp8 stage) twice.  Prints the
    kernel-source hash the counters belong to."""
    import torch
    n = 1 << 28  # fp32 elements = 1 GiB
    src = torch.ones(n, device=device)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    gem, once = (w_kernel_launches_fp8 if fp8 else w_kernel_launches)(shape, device)
    for _ in range(2):
        once()
    torch.cuda.synchronize()
    print(json.dumps({"traffic_probe": True, "copy_bytes_each_way": 4 * n, "w_launches": 2 * ((len(gem) + 15) // 16),
                      "shapes_MNK": gem, "kernel_source_sha256": kernel_source_hash()}), flush=True)


def blas_comparison(shape, device, reps=20):
    """The stage's bf16 linear products, each timed through the library's
    kernels as the stage runs them and through torch.mm (hipBLASLt), with HIP
    events: F (Y = X W^T), B (dX = dY W; the library multiplies by the
    stage's transposed weight copy, torch.mm by W) and W (dW = dY^T X).
    torch.mm writes a bf16 product; the library's W product accumulates into
    fp32 dW in place (its extra read-modify-write is in its time).  Context
    for the kernels' rates, not part of the step."""
    import torch
    import split_backward_amd as zb

    def timeit(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    T = shape.tokens
    seen, rows = set(), []
    for (M, N, K) in w_pass_gemms(shape):  # W: dW[M, N] += dY[K, M]^T X[K, N]
        if (M, N, K) in seen:
            continue
        seen.add((M, N, K))
        fl = 2.0 * M * N * K
        A = torch.randn(K, M, device=device).to(torch.bfloat16)
        B = torch.randn(K, N, device=device).to(torch.bfloat16)
        C = torch.zeros(M, N, device=device, dtype=torch.float32)
        Cb = torch.empty(M, N, device=device, dtype=torch.bfloat16)
        t_lib = timeit(lambda: zb.gemm(A, B, C, a_kmajor=False, b_kmajor=False, M=M, N=N, K=K, accumulate=True))
        t_mm = timeit(lambda: torch.mm(A.t(), B, out=Cb))
        rows.append({"pass": "W", "MNK": [M, N, K], "lib_tflops": round(fl / t_lib / 1e9, 1),
                     "torch_mm_tflops": round(fl / t_mm / 1e9, 1)})
        # the F product with this weight (Y[T, M] = X[T, N] W[M, N]^T) and its B (dX[T, N] = dY[T, M] W[M, N])
        X = torch.randn(T, N, device=device).to(torch.bfloat16)
        Wt = torch.randn(M, N, device=device).to(torch.bfloat16)
        Y = torch.empty(T, M, device=device, dtype=torch.bfloat16)
        t_lib = timeit(lambda: zb.gemm(X, Wt, Y, a_kmajor=True, b_kmajor=True, M=T, N=M, K=N))
        t_mm = timeit(lambda: torch.mm(X, Wt.t(), out=Y))
        rows.append({"pass": "F", "MNK": [T, M, N], "lib_tflops": round(fl / t_lib / 1e9, 1),
                     "torch_mm_tflops": round(fl / t_mm / 1e9, 1)})
        # the stage's B pass multiplies by its transposed weight copy [in][out]
        dY = torch.randn(T, M, device=device).to(torch.bfloat16)
        dX = torch.empty(T, N, device=device, dtype=torch.bfloat16)
        WtT = Wt.t().contiguous()
        t_lib = timeit(lambda: zb.gemm(dY, WtT, dX, a_kmajor=True, b_kmajor=True, M=T, N=N, K=M))
        t_mm = timeit(lambda: torch.mm(dY, Wt, out=dX))
        rows.append({"pass": "B", "MNK": [T, N, M], "lib_tflops": round(fl / t_lib / 1e9, 1),
                     "torch_mm_tflops": round(fl / t_mm / 1e9, 1)})
        del A, B, C, Cb, X, Wt, Y, dY, dX, WtT
    return rows


def cpu_baseline(shape, m, fp8=False):
    """The oracle timed on this host on a bounded sample.

    value: the fp64 loop-nest oracle (oracle/loopnest.c, OpenMP over output
    rows) running F, B and W of every linear product of one decoder layer
    (the whole block for the small kinds) at a reduced token count, in
    linear-layer TFLOP/s like the metric; `extrapolated_step_s` is the whole
    step's linear work at that rate.  `oracle_stage_numpy`: the numpy
    oracle's whole stage step (attention and norms included, products
    through numpy's BLAS) on one layer at 256 tokens, for context.  The fp8
    line times the fp8 oracle stage instead of the loop nests."""
    import numpy as np
    import synth
    from oracle import dense as od
    from oracle import fp8 as o8
    from oracle import loopnest as ln
    try:
        affinity = len(os.sched_getaffinity(0))
    except Exception:
        affinity = None
    env = {"nproc": os.cpu_count(), "affinity_cpus": affinity, "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}
    full_linear = linear_flops_per_mb(shape) * m

    def numpy_stage():
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:
            cores = os.cpu_count() or 1
        if shape.kind == "llama":
            sample = synth.StageShape("llama", 256, shape.hidden, shape.ffn, n_layers=1, n_heads=shape.n_heads,
                                      n_kv_heads=shape.n_kv_heads, head_dim=shape.head_dim)
            desc = f"one decoder layer, one microbatch, 256 tokens, h={shape.hidden}, ffn={shape.ffn}"
        elif shape.kind == "mlp":
            sample = synth.StageShape("mlp", 512, shape.hidden, shape.ffn)
            desc = f"one microbatch, 512 tokens, h={shape.hidden}, ffn={shape.ffn}"
        else:
            sample = shape
            desc = "one microbatch of the full shape"
        w = synth.make_weights(sample)
        dims = od.LlamaDims(sample.hidden, sample.ffn, sample.n_heads, sample.n_kv_heads, sample.head_dim) \
            if sample.kind == "llama" else None
        x = synth.make_x(sample, 0).f64
        dy = synth.make_dy(sample, 0).f64
        reps, t_total = 0, 0.0
        while t_total < 8.0 and reps < 50:
            st = (o8.Fp8LlamaStage([t.f64 for t in w], dims, sample.n_layers) if fp8 else
                  od.Stage(sample.kind, [t.f64 for t in w], dims, sample.n_layers))
            t0 = time.perf_counter()
            st.fwd(0, x)
            st.bwd_input(0, dy)
            st.bwd_weight(0)
            t_total += time.perf_counter() - t0
            reps += 1
        per_rep = t_total / reps
        sample_work = linear_flops_per_mb(sample) + attention_flops_per_mb(sample)
        full_work = (linear_flops_per_mb(shape) + attention_flops_per_mb(shape)) * m
        kind = "fp8 oracle stage (E4M3 rounding in numpy, products through its BLAS)" if fp8 else \
            "fp64 numpy oracle stage (products through its BLAS)"
        return {"value": round(reps * linear_flops_per_mb(sample) / t_total / 1e12, 4), "unit": "TFLOP/s",
                "cores": cores, "kind": "oracle",
                "sample": f"{desc}; {kind}; {reps} repetitions in {t_total:.1f} s",
                "extrapolated_step_s": round(per_rep * full_work / sample_work, 1),
                "extrapolated_note": "EXTRAPOLATED, not measured: the full step's linear and attention flops at "
                                     "the sample's measured rate"}

    if fp8:
        return {**numpy_stage(), **env}

    # products of one layer (the whole block for the small kinds): (out, in)
    # per weight, at a token count that keeps the sample near 0.15 TFLOP
    prods = [(M, N) for (M, N, _) in w_pass_gemms(shape)]
    if shape.kind == "llama":
        prods = prods[:4]
    per_token = 6.0 * sum(M * N for M, N in prods)  # F + B + W flops per token
    tokens = shape.tokens
    while tokens > 16 and tokens * per_token > 1.6e11:
        tokens //= 2
    r = np.random.default_rng(0)
    data = [(r.standard_normal((tokens, N)), r.standard_normal((M, N)), r.standard_normal((tokens, M)),
             np.zeros((M, N))) for M, N in prods]
    reps, t_total = 0, 0.0
    while t_total < 8.0 and reps < 50:
        t0 = time.perf_counter()
        for X, W, dY, dW in data:
            ln.linear_fwd(X, W)
            ln.linear_bwd_input(dY, W)
            ln.linear_bwd_weight(dY, X, dW)
        t_total += time.perf_counter() - t0
        reps += 1
    rate = reps * tokens * per_token / t_total
    what = "one decoder layer's" if shape.kind == "llama" else "the block's"
    return {"value": round(rate / 1e12, 4), "unit": "TFLOP/s", "cores": ln.threads(), "kind": "oracle",
            "sample": f"fp64 loop-nest oracle (C, OpenMP over output rows): F, B and W of {what} {len(prods)} "
                      f"linear products at {tokens} tokens, one microbatch; {reps} repetitions in {t_total:.1f} s",
            **env,
            "extrapolated_step_s": round(full_linear / rate, 1),
            "extrapolated_note": "EXTRAPOLATED, not measured: the full step's linear flops at the sample's "
                                 "measured rate",
            "oracle_stage_numpy": numpy_stage()}


def executor_idle(stage, shape, m, xs, ys, dys, dxs, t_f, t_b, t_w):
    """Replay stage 3 of an emulated p=8 pipeline on the GPU.

    * "1f1b", "zb_M16", "zb_M8": arrivals from the generator at costs 1:1:1,
      unit u = mean of the measured F, B, W pass times (the literal
      workload definition); "zb_M16_u0.9" / "_u1.1" give its sensitivity.
    * "*_measured_costs": arrivals from the generator with the measured
      F : B : W ratio in 0.1 ms units, i.e. a pipeline of identical stages;
      the simulator's own in-window idle for that case is reported beside it.
    """
    import torch
    import split_backward_amd as zb
    unit = (t_f + t_b + t_w) / 3.0
    q = 0.1  # ms per integer cost unit for the measured-cost runs
    mc = tuple(max(1, int(round(t / q))) for t in (t_f, t_b, t_w))
    runs = [("1f1b", "1f1b", 0, (1, 1, 1), unit), ("zb_M16", "zb", 16, (1, 1, 1), unit),
            ("zb_M8", "zb", 8, (1, 1, 1), unit), ("zb_M16_u0.9", "zb", 16, (1, 1, 1), 0.9 * unit),
            ("zb_M16_u1.1", "zb", 16, (1, 1, 1), 1.1 * unit),
            ("1f1b_measured_costs", "1f1b", 0, mc, q), ("zb_M16_measured_costs", "zb", 16, mc, q),
            ("zb_M16_measured_costs_filler", "zb", 16, mc, q)]
    runs.insert(5, ("zb_M16_filler", "zb", 16, (1, 1, 1), unit))
    out = {"unit_ms": round(unit, 3), "measured_costs_0.1ms": mc}
    for name, kind, M, costs, u in runs:
        if M > stage.desc.ring_slots:
            continue
        g = zb.schedule_generate(kind, 8, m, M, costs, 3)
        stage.zero_grad()
        torch.cuda.synchronize()
        mode = zb.EXEC_FILLER if name.endswith("filler") else zb.EXEC_ORDERED
        r = stage.run_schedule(g["ops"], g["arrive_f"], g["arrive_b"], u, xs, ys, dys, dxs, mode=mode)
        win = g["last_end"] - g["first_start"]
        out[name] = {"in_window_idle": round(r["in_window_idle"], 5), "window_ms": round(r["window_ms"], 2),
                     "busy_ms": round(r["busy_ms"], 2), "stage_end_ms": round(r["t_last_end_ms"], 2),
                     "predicted_in_window_idle": round(1 - g["busy"] / win, 5),
                     "predicted_stage_end_ms": round(g["last_end"] * u, 2)}
    return out


def interleaved_idle(weights, shape, m, xs, dys, p=8, stage_idx=3, v=2):
    """Interleaved 1F1B (v = 2) on the GPU: the stage's layers split into
    two chunks of n_layers / 2 layers (two stage objects sharing the
    stage's weight tensors), replayed in the interleaved order of stage 3
    of an emulated 8-stage pipeline with arrivals at chunk costs 1:1:1 in
    units of the mean measured chunk pass time.  Reports measured in-window
    idle and stage end beside the simulator's ([Guide] "Quantitative
    Comparison": 17.9% bubble for v = 2 at p = 8, m = 16)."""
    import torch
    import split_backward_amd as zb
    L = shape.n_layers
    if L % v or m % p:
        return None
    lc = L // v
    g = zb.schedule_generate_interleaved(p, m, v, (1, 1, 1), stage_idx)
    peaks = []
    for c in range(v):
        live = peak = 0
        for t, cc, _ in g["ops"]:
            if cc == c and t in "FW":
                live += 1 if t == "F" else -1
                peak = max(peak, live)
        peaks.append(peak)
    chunks = [zb.Stage("llama", shape.tokens, shape.hidden, shape.ffn, weights[6 * lc * c:6 * lc * (c + 1)],
                       n_layers=lc, n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads, head_dim=shape.head_dim,
                       ring_slots=peaks[c]) for c in range(v)]
    ys = [[torch.empty_like(x) for x in xs] for _ in range(v)]
    dxs = [[torch.empty_like(x) for x in xs] for _ in range(v)]
    # chunk pass times: the median of five F, B, W passes of chunk 0
    samples = []
    for _ in range(5):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        chunks[0].zero_grad()
        ev[0].record()
        chunks[0].fwd(0, xs[0], ys[0][0])
        ev[1].record()
        chunks[0].bwd_input(0, dys[0], dxs[0][0])
        ev[2].record()
        chunks[0].bwd_weight(0)
        ev[3].record()
        torch.cuda.synchronize()
        samples.append([ev[i].elapsed_time(ev[i + 1]) for i in range(3)])
    tc = [sorted(col)[len(col) // 2] for col in zip(*samples)]
    unit = sum(tc) / 3.0
    for c in chunks:
        c.zero_grad()
    torch.cuda.synchronize()
    r = zb.run_schedule_chunks(chunks, g["ops"], g["arrive_f"], g["arrive_b"], unit, [xs] * v, ys, [dys] * v, dxs)
    win = g["last_end"] - g["first_start"]
    out = {"v": v, "layers_per_chunk": lc, "chunk_unit_ms": round(unit, 3),
           "chunk_pass_ms": {"F": round(tc[0], 3), "B": round(tc[1], 3), "W": round(tc[2], 3)},
           "ring_slots_per_chunk": peaks,
           "in_window_idle": round(r["in_window_idle"], 5), "window_ms": round(r["window_ms"], 2),
           "busy_ms": round(r["busy_ms"], 2), "stage_end_ms": round(r["t_last_end_ms"], 2),
           "predicted_in_window_idle": round(1 - g["busy"] / win, 5),
           "predicted_stage_end_ms": round(g["last_end"] * unit, 2),
           "predicted_bubble_over_makespan": round((g["makespan"] - g["busy"]) / g["makespan"], 5)}
    del chunks
    torch.cuda.synchronize()
    return out


def memory_limit_sweep(stage, m, xs, ys, dys, dxs, unit, p=8, stage_idx=3, weights=None, shape=None):
    """ZB(M) for M = p .. 2p on the GPU (arrivals at costs 1:1:1 in units of
    the mean pass time), replayed in ordered mode and in filler mode (W on
    the second stream): measured in-window idle and stage end beside the
    simulator's, and the stash the order keeps resident at its peak (peak
    in-flight microbatches x bytes per ring slot).  When the benchmark
    stage's ring is smaller than 2p (the Llama-70B slice keeps 8 slots), a
    second stage with a 2p-slot ring, sharing the weight tensors, runs the
    sweep."""
    import torch
    import split_backward_amd as zb
    if stage.desc.ring_slots < 2 * p and weights is not None:
        stage = zb.Stage(shape.kind, shape.tokens, shape.hidden, shape.ffn, weights, dtype=shape.dtype,
                         n_layers=shape.n_layers, n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads,
                         head_dim=shape.head_dim, ring_slots=2 * p)
    slot = stage.slot_bytes()
    rows = []
    for M in range(p, 2 * p + 1):
        if M > stage.desc.ring_slots:
            break
        g = zb.schedule_generate("zb", p, m, M, (1, 1, 1), stage_idx)
        res = {}
        for mode_name, mode in (("ordered", zb.EXEC_ORDERED), ("filler", zb.EXEC_FILLER)):
            stage.zero_grad()
            torch.cuda.synchronize()
            res[mode_name] = stage.run_schedule(g["ops"], g["arrive_f"], g["arrive_b"], unit, xs, ys, dys, dxs,
                                                mode=mode)
        win = g["last_end"] - g["first_start"]
        rows.append({"M": M, "in_window_idle": round(res["ordered"]["in_window_idle"], 5),
                     "in_window_idle_filler": round(res["filler"]["in_window_idle"], 5),
                     "predicted_in_window_idle": round(1 - g["busy"] / win, 5),
                     "stage_end_ms": round(res["ordered"]["t_last_end_ms"], 2),
                     "stage_end_ms_filler": round(res["filler"]["t_last_end_ms"], 2),
                     "predicted_stage_end_ms": round(g["last_end"] * unit, 2),
                     "peak_resident_microbatches": g["peak_active"],
                     "stash_GiB": round(g["peak_active"] * slot / 2**30, 2)})
    return {"unit_ms": round(unit, 3), "slot_GiB": round(slot / 2**30, 3), "runs": rows}


def multi_iteration(stage, m, xs, ys, dys, dxs, t_f, t_b, t_w, t_o, p=8, stage_idx=3, n_iter=2, lr=1e-4):
    """Two iterations back to back (zb_schedule_generate_iters; zero bubble
    with M = 2p, and 1F1B for comparison): each stage runs its optimizer step
    (SGD, then cleared dW) after its own last W, and its next iteration's F
    waits only for that step and the upstream F.  Replayed in ordered mode
    (and filler mode for the zero-bubble order) with arrivals at costs
    1:1:1 (units of a tenth of the mean pass time, the optimizer step rounded
    to that unit) and at the measured costs (0.1 ms units).  Reports the
    in-window idle over the whole run, the stage end and the gap between the
    stage's optimizer step and its next F, each beside the simulator's."""
    import torch
    import split_backward_amd as zb
    u = (t_f + t_b + t_w) / 3.0
    # inputs repeat every iteration; each iteration writes outputs of its own
    X, DY = xs * n_iter, dys * n_iter
    Y = list(ys) + [torch.empty_like(y) for _ in range(n_iter - 1) for y in ys]
    DX = list(dxs) + [torch.empty_like(d) for _ in range(n_iter - 1) for d in dxs]
    q = 0.1
    cases = [("costs_1:1:1", (10, 10, 10), max(1, int(round(10 * t_o / u))), u / 10),
             ("measured_costs", tuple(max(1, int(round(t / q))) for t in (t_f, t_b, t_w)), max(1, int(round(t_o / q))), q)]
    stage.set_lr(lr)
    out = {"optimizer_step_ms": round(t_o, 3), "n_iter": n_iter, "M": min(2 * p, stage.desc.ring_slots)}
    for name, costs, c_opt, unit in cases:
        for kind, M, modes in (("zb", min(2 * p, stage.desc.ring_slots),
                                (("ordered", zb.EXEC_ORDERED), ("filler", zb.EXEC_FILLER))),
                               ("1f1b", 0, (("ordered", zb.EXEC_ORDERED),))):
            g = zb.schedule_generate_iters(p, m, M, costs, c_opt, n_iter, stage_idx, kind=kind)
            ops = g["ops"]
            o_idx = [k for k, (t, _) in enumerate(ops) if t == "O"]
            pred_gap = (g["start"][o_idx[0] + 1] - g["end"][o_idx[0]]) * unit
            win = g["last_end"] - g["first_start"]
            row = {"costs": costs, "c_opt": c_opt, "unit_ms": round(unit, 4),
                   "predicted_in_window_idle": round(1 - g["busy"] / win, 5),
                   "predicted_stage_end_ms": round(g["last_end"] * unit, 2), "predicted_gap_ms": round(pred_gap, 3)}
            for mode_name, mode in modes:
                stage.zero_grad()
                torch.cuda.synchronize()
                r = stage.run_schedule(ops, g["arrive_f"], g["arrive_b"], unit, X, Y, DY, DX, mode=mode)
                om = r["op_ms"]
                row[mode_name] = {"in_window_idle": round(r["in_window_idle"], 5),
                                  "stage_end_ms": round(r["t_last_end_ms"], 2),
                                  "gap_ms": round(om[o_idx[0] + 1][0] - om[o_idx[0]][1], 3)}
                if mode == zb.EXEC_ORDERED:
                    # waits besides the iteration gap: an op starting > 0.3 ms after the
                    # previous op ended (ordered mode runs the list strictly in turn)
                    waits = [(t_, j_, round(om[k][0] - om[k - 1][1], 2)) for k, (t_, j_) in enumerate(ops)
                             if k > 0 and k != o_idx[0] + 1 and om[k][0] - om[k - 1][1] > 0.3]
                    row[mode_name]["other_waits_ms"] = round(sum(w for _, _, w in waits), 2)
                    row[mode_name]["other_waits"] = waits[:8]
            out[f"{kind}_{name}"] = row
    stage.set_lr(0.0)
    return out


# (name, order, M, mode, costs): costs None = 1:1:1 in units of the mean
# pass time, "measured" = the calibrated F, B, W times in 0.1 ms units.
REPLAY_RUNS = (("zb_M16_ordered", "zb", 16, 0, None), ("zb_M16_filler", "zb", 16, 1, None),
               ("1f1b_ordered", "1f1b", 0, 0, None),
               ("zb_M16_ordered_measured_costs", "zb", 16, 0, "measured"),
               ("zb_M16_filler_measured_costs", "zb", 16, 1, "measured"))


def replay_only(stage, m, xs, ys, dys, dxs, pass_ms, p=8, stage_idx=3):
    """The replays whose idle a rocprofv3 kernel trace measures
    independently (--replay-only under rocprofv3 --kernel-trace, then
    --trace-idle): zero bubble (M = 16) in ordered and filler mode and 1F1B
    with arrivals at costs 1:1:1 in units of the mean pass time, then zero
    bubble again with arrivals at the measured F, B, W costs, one after the
    other with the GPU idle in between."""
    import torch
    import split_backward_amd as zb
    out = []
    for name, kind, M, mode, costs in REPLAY_RUNS:
        if costs is None:
            c, unit = (1, 1, 1), sum(pass_ms) / 3.0
        else:
            c, unit = tuple(max(1, int(round(t * 10))) for t in pass_ms), 0.1
        g = zb.schedule_generate(kind, p, m, M, c, stage_idx)
        stage.zero_grad()
        torch.cuda.synchronize()
        r = stage.run_schedule(g["ops"], g["arrive_f"], g["arrive_b"], unit, xs, ys, dys, dxs, mode=mode)
        torch.cuda.synchronize()
        win = g["last_end"] - g["first_start"]
        out.append({"name": name, "n_ops": len(g["ops"]), "costs": list(c), "unit_ms": round(unit, 4),
                    "stamp_in_window_idle": round(r["in_window_idle"], 5), "stamp_window_ms": round(r["window_ms"], 3),
                    "stamp_busy_ms": round(r["busy_ms"], 3),
                    "predicted_in_window_idle": round(1 - g["busy"] / win, 5)})
    return out


def trace_idle(csv_path, replays_path):
    """In-window idle of each replay from a rocprofv3 kernel trace: the
    replays' clock-stamp kernels (1 + 2 per op, in time order) delimit them;
    inside each, busy = the union of the intervals of every kernel except the
    stamp and arrival-wait kernels, window = [first such kernel's start, last
    one's end].  Prints one JSON line per replay beside the stamp figure."""
    import csv
    with open(replays_path) as fh:
        replays = [json.loads(ln) for ln in fh if ln.strip().startswith("{")][-1]["replays"]
    kernels = []
    with open(csv_path, newline="") as fh:
        for row in csv.DictReader(fh):
            kernels.append((int(row["Start_Timestamp"]), int(row["End_Timestamp"]), row["Kernel_Name"]))
    kernels.sort()
    stamps = [k for k in kernels if "stamp_kernel" in k[2]]
    need = sum(1 + 2 * r["n_ops"] for r in replays)
    if len(stamps) != need:
        raise SystemExit(f"trace has {len(stamps)} stamp kernels, the replays need {need}")
    i = 0
    for r in replays:
        grp = stamps[i:i + 1 + 2 * r["n_ops"]]
        i += len(grp)
        lo_t, hi_t = grp[0][0], grp[-1][1]
        work = [(a, b) for a, b, nm in kernels
                if lo_t <= a and b <= hi_t and "stamp_kernel" not in nm and "wait_kernel" not in nm]
        w0, w1 = min(a for a, _ in work), max(b for _, b in work)
        busy, cs, ce = 0, work[0][0], work[0][1]
        for a, b in work[1:]:
            if a > ce:
                busy += ce - cs
                cs, ce = a, b
            else:
                ce = max(ce, b)
        busy += ce - cs
        print(json.dumps({"name": r["name"], "kernels": len(work), "trace_window_ms": round((w1 - w0) / 1e6, 3),
                          "trace_busy_ms": round(busy / 1e6, 3),
                          "trace_in_window_idle": round((w1 - w0 - busy) / (w1 - w0), 5),
                          "stamp_in_window_idle": r["stamp_in_window_idle"],
                          "predicted_in_window_idle": r["predicted_in_window_idle"]}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama7b_stage4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-executor", action="store_true")
    ap.add_argument("--no-w-pairs", action="store_true",
                    help="issue every W on its own instead of pairing adjacent W(j), W(j+1)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only run the copy + W-kernel workload that the --pmc passes count")
    ap.add_argument("--compare-blas", action="store_true",
                    help="only time the stage's bf16 products through the library and through torch.mm (hipBLASLt)")
    ap.add_argument("--replay-only", action="store_true",
                    help="only calibrate and run the replays a kernel trace measures (see trace_idle)")
    ap.add_argument("--trace-idle", nargs=2, metavar=("KERNEL_TRACE_CSV", "REPLAY_JSON"),
                    help="in-window idle of the --replay-only replays from a rocprofv3 kernel trace (no GPU)")
    args = ap.parse_args()
    if args.trace_idle:
        trace_idle(*args.trace_idle)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs one pipeline stage on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import split_backward_amd as zb
    import synth

    wl = synth.WORKLOADS[args.workload]
    shape, m = wl["shape"], wl["m"]
    stage_dtype = wl.get("stage_dtype", shape.dtype)
    fp8 = stage_dtype == "fp8"
    ring = wl.get("ring", m)
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    if args.traffic_probe:
        traffic_probe(shape, device, fp8)
        return
    if args.compare_blas:
        for row in blas_comparison(shape, device):
            print(json.dumps(row), flush=True)
        return
    weights = [synth.to_device(w, device) for w in synth.make_weights(shape)]
    stage = zb.Stage(shape.kind, shape.tokens, shape.hidden, shape.ffn, weights, dtype=stage_dtype,
                     n_layers=shape.n_layers, n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads,
                     head_dim=shape.head_dim if shape.kind == "llama" else 128, ring_slots=ring)
    xs, ys, dys, dxs = make_inputs(shape, m, device)
    # zero-bubble order of stage 3 in an emulated 8-stage pipeline, memory limit min(2p, ring)
    order = zb.schedule_generate("zb", 8, m, min(16, ring), (1, 1, 1), 3)["ops"]

    plan = issue_plan(order, pair_w=not args.no_w_pairs)
    w_pairs = sum(1 for t, _ in plan if t == "P")

    def step():
        stage.zero_grad()
        for t, j in plan:
            if t == "F":
                stage.fwd(j, xs[j], ys[j])
            elif t == "B":
                stage.bwd_input(j, dys[j], dxs[j])
            elif t == "P":
                stage.bwd_weight_pair(j)
            else:
                stage.bwd_weight(j)

    if args.replay_only:
        step()  # warm-up
        t_f, t_b, t_w = calibrate(stage, xs, ys, dys, dxs)
        print(json.dumps({"replays": replay_only(stage, m, xs, ys, dys, dxs, (t_f, t_b, t_w)),
                          "pass_ms": [t_f, t_b, t_w]}), flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    flops = linear_flops_per_mb(shape) * m
    tflops = flops / dt / 1e12

    # per-pass times (the executor's arrival unit u = mean of F, B, W, and its
    # measured-cost runs): the median of five F, B, W passes, since a single
    # pass right after the timed steps can run slower than the replay does
    t_f, t_b, t_w = calibrate(stage, xs, ys, dys, dxs)

    # The fp32 linear workload runs the fp32 GEMM (a few microseconds per
    # product, launch-bound): no roofline figure for it.
    if fp8:
        roof = time_w_kernel_fp8(shape, args.workload, device)
    elif shape.dtype == "bf16":
        roof = time_w_kernel(shape, args.workload, device)
    else:
        roof = {"bound": None, "note": "fp32 linear workload: launch-bound fp32 GEMM, no roofline figure"}
    extra = {}
    if shape.kind == "llama" and not args.no_executor and not fp8:
        extra["executor_p8_stage3"] = executor_idle(stage, shape, m, xs, ys, dys, dxs, t_f, t_b, t_w)
        extra["executor_p8_stage3"]["interleaved_1f1b_v2"] = interleaved_idle(weights, shape, m, xs, dys)
        extra["memory_limit_sweep_p8_stage3"] = memory_limit_sweep(stage, m, xs, ys, dys, dxs, (t_f + t_b + t_w) / 3.0,
                                                                   weights=weights, shape=shape)
        # the optimizer step's own time (SGD over every weight, then dW cleared)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        stage.sgd_step(0.0)
        e0.record()
        stage.sgd_step(0.0)
        e1.record()
        torch.cuda.synchronize()
        t_o = e0.elapsed_time(e1)
        extra["two_iterations_p8_stage3"] = multi_iteration(stage, m, xs, ys, dys, dxs, t_f, t_b, t_w, t_o)
    cpu = None if args.no_cpu_baseline else cpu_baseline(shape, m, fp8=fp8)

    line = {
        "metric": "stage F+B+W TFLOP/s (bf16) and % MFMA peak; stage idle fraction vs 1F1B",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3 products (fp32 accumulation), bf16 elsewhere" if fp8 else shape.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": shape.tokens, "hidden": shape.hidden, "ffn": shape.ffn,
                   "n_layers": shape.n_layers, "n_heads": shape.n_heads, "n_kv_heads": shape.n_kv_heads,
                   "microbatches": m, "ring_slots": ring, "order": "zero-bubble greedy, M=min(16, ring), stage 3 of p=8",
                   "w_pairs": w_pairs},
        "pct_of_peak": round(100 * tflops / (PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS), 2),
        "peak_tflops": PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS,
        "tflops_incl_attention": round((flops + attention_flops_per_mb(shape) * m) / dt / 1e12, 2),
        "pass_ms": {"F": round(t_f, 3), "B": round(t_b, 3), "W": round(t_w, 3)},
        "roofline": roof, "cpu_baseline": cpu,
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
