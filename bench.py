"""Benchmark: QLoRA NF4 linear forward + backward on one MI355X.

Workload (the 7B-style decoder layer linears): q, k, v, o 4096x4096, gate and
up 11008x4096, down 4096x11008, weights N(0, 0.02) quantized to NF4 with
double quantization; M = 2048 tokens (batch 1 x sequence 2048) of bf16
activations N(0, 1); LoRA r = 8, alpha = 16 (s = 2) on q, k, v, o; upstream
gradients N(0, 1).  One step = for every projection: the forward (Y, T) and
the backward (dX, dA, dB).  Outputs Y and dX are bf16, T/dA/dB fp32.  Inputs
are resident in HBM before the timed region; no allocation inside it.

Prints one JSON line.  Throughput is algorithmic: forward 2MNK + 2Mr(K+N),
backward 2MNK + 2Mr(2K+2N) flops; bytes = packed weight once per pass plus
every activation, gradient and adapter tensor at its dtype.

Other workloads (--workload), each printing its own line of the same form:
  single      one 4096x4096 linear at M = 16 tokens with LoRA r = 8, alpha =
              16, fwd + bwd on the small-m streaming paths, from a cold cache
              (2 GiB written before each step, the launches queued behind it);
              effective GB/s against HBM peak, the streaming input gradient
              as the roofline kernel.
  decode      the seven projections stacked for 32 layers (6.48e9 NF4 params,
              3.35 GB packed), forward only at M = 1 (also 4 and 16 in
              "per_m"), LoRA r = 8, alpha = 16 on q, k, v, o; one grouped
              launch per sweep; effective GB/s against HBM peak.
  quantize70b quantize + double-quantize a 70B-style layer (q, k, v, o
              8192x8192; gate, up 28672x8192; down 8192x28672; N(0, 0.015)
              with 0.1 % of the weights scaled x20); GB/s against HBM peak.
  layer70b    the same layer, fwd + bwd at M = 4096 with LoRA r = 16,
              alpha = 32 on all seven; TFLOP/s against bf16 MFMA peak.
--dtype f16 runs the NF4 workloads in the fp16 compute type (weights,
activations, adapters and 16-bit outputs fp16; the fp16 MFMA peak equals the
bf16 one).
  layer3.8b   3.8B-style layer linears (hidden 3072, intermediate 8192: q, k,
              v, o 3072x3072; gate, up 8192x3072; down 3072x8192), fwd + bwd
              at M = 4096 (seq 4096) with LoRA r = 64, alpha = 128 on all
              seven, weights in the --format block format (q8_0, u4_asym or
              nf4); TFLOP/s against bf16 MFMA peak.
"""
from __future__ import annotations

import argparse
import statistics
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
M_TOKENS = 2048
RANK, ALPHA = 8, 16
PROJ = [  # name, N (out), K (in), LoRA rank
    ("q", 4096, 4096, RANK), ("k", 4096, 4096, RANK), ("v", 4096, 4096, RANK),
    ("o", 4096, 4096, RANK), ("gate", 11008, 4096, 0), ("up", 11008, 4096, 0),
    ("down", 4096, 11008, 0),
]
WORKLOAD = ("7B-style decoder layer linears (q,k,v,o 4096x4096; gate,up 11008x4096; "
            "down 4096x11008), M=2048 tokens, LoRA r=8 alpha=16 on q,k,v,o, fwd+bwd")
METRIC = "QLoRA linear fwd+bwd TFLOP/s & effective GB/s (% roofline) on 1 MI355X"
PROJ70 = [("q", 8192, 8192), ("k", 8192, 8192), ("v", 8192, 8192), ("o", 8192, 8192),
          ("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672)]
DECODE_LAYERS = 32
DECODE_SETTLE_SWEEPS = 40   # untimed sweeps before each timed decode series
CPU_DECODE_LAYERS = 5


def flops_fwd(M, N, K, r):
    return 2 * M * N * K + 2 * M * r * (K + N)


def flops_bwd(M, N, K, r):
    return 2 * M * N * K + 2 * M * r * (2 * K + 2 * N)


# weight format: double-quantized scales (default) or one fp32 absmax per
# block (--single-level); NF4 block size (--nf4-block, 64 by default)
DQ = True
BLOCK = 64
# compute type of the NF4 workloads (--dtype): bf16, or fp16 (NF4 block 64
# with double quantization only)
DT = torch.bfloat16


def dt_name():
    return "f16" if DT == torch.float16 else "bf16"


def dnorm(*a, **k):
    """Seeded device-side draw in the compute type."""
    import synth
    return synth.device_normal_bf16(*a, dtype=DT, **k)


def packed_bytes(N, K):
    nb = N * K // BLOCK
    if not DQ:
        return N * K // 2 + 4 * nb
    return N * K // 2 + nb + 4 * ((nb + 255) // 256)


def step_bytes(M, N, K, r):
    w = packed_bytes(N, K)
    fwd = w + 2 * M * K + 2 * M * N + (2 * r * K + 2 * N * r + 4 * M * r if r else 0)
    bwd = w + 2 * M * N + 2 * M * K + (2 * M * K + 2 * r * K + 2 * N * r + 4 * M * r
                                       + 4 * r * K + 4 * N * r if r else 0)
    return fwd + bwd


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "qlora_fine_tuning_nf4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel, src_files):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    if not os.path.exists(p) or not DQ or BLOCK != 64 or DT != torch.bfloat16:   # counters: that format
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_hash") != kernel_source_hash(src_files):
        return None
    return d.get("bytes_per_launch")


def host_cpu():
    """The host the CPU baseline runs on: logical CPUs, the CPUs this process
    may run on, and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


def blas_threads():
    from threadpoolctl import threadpool_info
    return max([t.get("num_threads", 1) for t in threadpool_info()] + [1])


def with_cpu_figures(run_sample, unit, scale, full_sample, single_sample):
    """Time the oracle as it stands on `full_sample` with every BLAS thread,
    then on the smaller `single_sample` with one thread; run_sample(sample)
    returns (work, seconds, description).  value = work / seconds / scale."""
    from threadpoolctl import threadpool_limits

    work, el, desc = run_sample(full_sample)
    out = {"value": round(work / el / scale, 4), "unit": unit, "cores": blas_threads(),
           "kind": "oracle", "sample": f"{desc} ({el:.1f} s, all BLAS threads)", **host_cpu()}
    with threadpool_limits(limits=1):
        w1, e1, d1 = run_sample(single_sample)
    out["single_thread"] = {"value": round(w1 / e1 / scale, 4), "unit": unit, "cores": 1,
                            "sample": f"{d1} ({e1:.1f} s, one thread)"}
    return out


def cpu_baseline(sample_tokens: int):
    """The oracle, as it stands, on a bounded sample of the same workload: all
    seven projections with the first `sample_tokens` tokens: dequantize each
    weight, forward, backward (float64 numpy); again on 1/16 of those tokens
    with one thread."""
    import synth
    from oracle import linear as olin
    from oracle import nf4 as onf4

    lv, mid = onf4.codebook()
    packed = {}
    for i, (name, N, K, r) in enumerate(PROJ):
        W = synth.normal_bf16((N, K), 0.02, synth.tensor_seed(2, 10 * i))
        packed[i] = onf4.quantize(W, mid)          # storage, not part of the step

    def run(M):
        total_flops, elapsed = 0, 0.0
        for i, (name, N, K, r) in enumerate(PROJ):
            codes, qs, st = packed[i]
            X = synth.normal_bf16((M, K), 1.0, synth.tensor_seed(2, 10 * i + 1))
            dY = synth.normal_bf16((M, N), 1.0, synth.tensor_seed(2, 10 * i + 2))
            A = synth.normal_bf16((r, K), 0.01, synth.tensor_seed(2, 10 * i + 3)) if r else None
            B = synth.normal_bf16((N, r), 0.01, synth.tensor_seed(2, 10 * i + 4)) if r else None
            t0 = time.perf_counter()
            Wd = onf4.dequantize(codes, qs, st, lv).reshape(N, K)
            olin.forward(Wd, X, A, B, ALPHA / RANK)
            Wd = onf4.dequantize(codes, qs, st, lv).reshape(N, K)
            olin.backward(Wd, X, dY, A, B, ALPHA / RANK)
            elapsed += time.perf_counter() - t0
            total_flops += flops_fwd(M, N, K, r) + flops_bwd(M, N, K, r)
        return (total_flops, elapsed, f"all 7 projections at M={M} of the {M_TOKENS} tokens: "
                                      "dequantize + fwd + bwd in float64 numpy")
    return with_cpu_figures(run, "TFLOP/s", 1e12, sample_tokens, max(1, sample_tokens // 16))


def run_layer7b(args):
    import torch

    import synth
    from qlora_fine_tuning_nf4_amd import binding as QB

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cb = QB.device_codebook(dev)
    M = M_TOKENS
    s = ALPHA / RANK
    layers = []
    for i, (name, N, K, r) in enumerate(PROJ):
        W = dnorm((N, K), 0.02, synth.tensor_seed(2, 10 * i), device=dev)
        q = QB.qlora_quantize(W, cb, double_quant=DQ, block=BLOCK)
        del W
        L = dict(name=name, N=N, K=K, r=r, q=q)
        L["X"] = dnorm((M, K), 1.0, synth.tensor_seed(2, 10 * i + 1), device=dev)
        L["dY"] = dnorm((M, N), 1.0, synth.tensor_seed(2, 10 * i + 2), device=dev)
        L["A"] = dnorm((r, K), 0.01, synth.tensor_seed(2, 10 * i + 3), device=dev) if r else None
        L["B"] = dnorm((N, r), 0.01, synth.tensor_seed(2, 10 * i + 4), device=dev) if r else None
        L["Y"] = torch.empty((M, N), dtype=DT, device=dev)
        L["T"] = torch.empty((M, r), dtype=torch.float32, device=dev) if r else None
        L["dX"] = torch.empty((M, K), dtype=DT, device=dev)
        L["dA"] = torch.empty((r, K), dtype=torch.float32, device=dev) if r else None
        L["dB"] = torch.empty((N, r), dtype=torch.float32, device=dev) if r else None
        nws = max(QB.qlora_workspace_bytes(0, M, N, K, r), QB.qlora_workspace_bytes(1, M, N, K, r), 16)
        L["ws"] = torch.empty(nws, dtype=torch.uint8, device=dev)
        layers.append(L)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev_fwd, ev_dx = [], []

    def step(record):
        for L in layers:
            single = record and L["r"] == 0      # r = 0: the call is one GEMM launch
            if single:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            QB.qlora_linear_fwd(L["q"], cb, L["X"], L["A"], L["B"], s, out=L["Y"], T_out=L["T"],
                                workspace=L["ws"])
            if single:
                e1.record(stream)
                ev_fwd.append((e0, e1, L))
                e2 = torch.cuda.Event(enable_timing=True)
                e3 = torch.cuda.Event(enable_timing=True)
                e2.record(stream)
            QB.qlora_linear_bwd(L["q"], cb, L["X"], L["dY"], L["A"], L["B"], s, T=L["T"],
                                dX_out=L["dX"], dA_out=L["dA"], dB_out=L["dB"], workspace=L["ws"])
            if single:
                e3.record(stream)
                ev_dx.append((e2, e3, L))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    # one event per step boundary: per-step GPU times for the median and spread
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    bounds[0].record(stream)
    for i in range(args.steps):
        step(True)
        bounds[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = bounds[0].elapsed_time(bounds[-1])
    step_ms = [bounds[i].elapsed_time(bounds[i + 1]) for i in range(args.steps)]
    ms_per_step = wall * 1e3 / args.steps

    total_flops = sum(flops_fwd(M, L["N"], L["K"], L["r"]) + flops_bwd(M, L["N"], L["K"], L["r"])
                      for L in layers)
    total_bytes = sum(step_bytes(M, L["N"], L["K"], L["r"]) for L in layers)
    tflops = total_flops / (ms_per_step * 1e-3) / 1e12
    gbs = total_bytes / (ms_per_step * 1e-3) / 1e9

    def kstats(evs):
        durs = [a.elapsed_time(b) * 1e-3 for a, b, _ in evs]
        flops = [2 * M * L["N"] * L["K"] for _, _, L in evs]
        return sum(durs), sum(flops), len(durs)

    tf, ff, nf = kstats(ev_fwd)
    td, fd, nd = kstats(ev_dx)
    if td >= tf:
        kname, t_tot, f_tot, n_l, srcs = "k_gemm_dx", td, fd, nd, ["gemm.hip", "common.h"]
    else:
        kname, t_tot, f_tot, n_l, srcs = "k_gemm_fwd", tf, ff, nf, ["gemm.hip", "common.h"]
    achieved = (f_tot / n_l) / (t_tot / n_l) / 1e12
    roofline = {"bound": "mfma", "kernel": kname, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "avg_launch_us": round(t_tot / n_l * 1e6, 2),
                "traffic": traffic_from_profile(kname, srcs),
                "other_gemm": {"k_gemm_fwd": round(ff / tf / 1e12, 1) if tf else None,
                               "k_gemm_dx": round(fd / td / 1e12, 1) if td else None}}

    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "gpu_event_ms_per_step": round(gpu_ms / args.steps, 4),
        "gpu_step_ms": _spread(step_ms),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt_name(),
        "data": "synthetic (seeded N(0,0.02) weights quantized to NF4+DQ, N(0,1) activations)",
        "config": {"workload": WORKLOAD, "M": M, "r": RANK, "alpha": ALPHA, "double_quant": DQ, "nf4_block": BLOCK,
                   "projections": [[p[0], p[1], p[2], p[3]] for p in PROJ], "y_dtype": dt_name(),
                   "dx_dtype": dt_name(), "parallelism": "none (1 GPU)"},
        "effective_GBps": round(gbs, 1),
        "frac_of_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline,
    }
    if not args.no_library_baseline:
        out["library_baseline"] = library_gemm_baseline(layers, M, cb)
    if not args.no_measured_peaks:
        mp = measured_peaks()
        roofline["measured_peak"] = {"value": mp["mfma_bf16_loop_TFLOPs"], "unit": "TFLOP/s",
                                     "frac": round(achieved / mp["mfma_bf16_loop_TFLOPs"], 4), "all": mp}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_sample_tokens or M_TOKENS)
    return out


def library_gemm_baseline(layers, M, cb, iters=10):
    """The base products of the layer (Y = X deq(W)^T and dX = dY deq(W) for
    the seven projections, no LoRA) three ways, GPU time per step: the fused
    GEMMs of this library (r = 0 calls, one launch each); the library bf16 GEMM
    (torch.matmul, hipBLASLt) on weights dequantized beforehand, which keeps a
    16-bit copy of every weight resident; and dequantize-then-matmul, the
    weight expanded once for the forward and once for the backward."""
    import torch

    from qlora_fine_tuning_nf4_amd import binding as QB

    stream = torch.cuda.current_stream()
    wd = [QB.qlora_dequantize(L["q"], cb) for L in layers]

    def gpu_ms(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    def fused():
        for L in layers:
            QB.qlora_linear_fwd(L["q"], cb, L["X"], out=L["Y"], workspace=L["ws"], path="gemm")
            QB.qlora_linear_bwd(L["q"], cb, None, L["dY"], dX_out=L["dX"], workspace=L["ws"], path="gemm")

    def matmul():
        for L, W in zip(layers, wd):
            torch.matmul(L["X"], W.t(), out=L["Y"])
            torch.matmul(L["dY"], W, out=L["dX"])

    def deq_matmul():
        for L, W in zip(layers, wd):
            QB.qlora_dequantize(L["q"], cb, out=W)
            torch.matmul(L["X"], W.t(), out=L["Y"])
            QB.qlora_dequantize(L["q"], cb, out=W)
            torch.matmul(L["dY"], W, out=L["dX"])

    t_f, t_m, t_dm = gpu_ms(fused), gpu_ms(matmul), gpu_ms(deq_matmul)
    flops = sum(4.0 * M * L["N"] * L["K"] for L in layers)
    del wd
    return {"kind": "base products of the layer (fwd + dX, 7 projections, no LoRA) on the GPU",
            "fused_gemm_ms": round(t_f, 4), "fused_tflops": round(flops / t_f / 1e9, 1),
            "hipblaslt_bf16_resident_ms": round(t_m, 4), "hipblaslt_bf16_tflops": round(flops / t_m / 1e9, 1),
            "dequant_then_hipblaslt_ms": round(t_dm, 4),
            "fused_speedup_vs_dequant_then_hipblaslt": round(t_dm / t_f, 3)}


SINGLE_M = 16
SINGLE_WORKLOAD = ("single linear 4096x4096 (N(0,0.02) weight, NF4 block 64 + double quant), "
                   "M=16 tokens, LoRA r=8 alpha=16, fwd (Y, T) + bwd (dX, dA, dB), "
                   "cold cache (2 GiB written between steps)")


def run_single(args):
    """Single 4096x4096 linear at M = 16 with LoRA r = 8, forward + backward,
    each step starting from a cold cache: a 2 GiB fill runs before each step
    and the step's launches (the forward and the backward, on the small-m
    streaming paths) are enqueued behind it, so the timed interval holds the
    step's kernels back to back and no host overhead."""
    import torch

    import synth
    from qlora_fine_tuning_nf4_amd import binding as QB

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cb = QB.device_codebook(dev)
    M, N, K, r = SINGLE_M, 4096, 4096, RANK
    s = ALPHA / RANK
    W = dnorm((N, K), 0.02, synth.tensor_seed(1, 0), device=dev)
    q = QB.qlora_quantize(W, cb, double_quant=DQ, block=BLOCK)
    del W
    X = dnorm((M, K), 1.0, synth.tensor_seed(1, 1), device=dev)
    A = dnorm((r, K), 0.01, synth.tensor_seed(1, 2), device=dev)
    Bm = dnorm((N, r), 0.01, synth.tensor_seed(1, 3), device=dev)
    dY = dnorm((M, N), 1.0, synth.tensor_seed(1, 4), device=dev)
    Y = torch.empty((M, N), dtype=DT, device=dev)
    T = torch.empty((M, r), dtype=torch.float32, device=dev)
    dX = torch.empty((M, K), dtype=DT, device=dev)
    dA = torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    ws = torch.empty(max(QB.qlora_workspace_bytes(0, M, N, K, r), QB.qlora_workspace_bytes(1, M, N, K, r), 16),
                     dtype=torch.uint8, device=dev)
    dX0 = torch.empty((M, K), dtype=DT, device=dev)
    ws0 = torch.empty(max(QB.qlora_workspace_bytes(1, M, N, K, 0), 16), dtype=torch.uint8, device=dev)
    flush = torch.empty(1 << 31, dtype=torch.uint8, device=dev)

    def step():
        QB.qlora_linear_fwd(q, cb, X, A, Bm, s, y_dtype=DT, out=Y, T_out=T, workspace=ws)
        QB.qlora_linear_bwd(q, cb, X, dY, A, Bm, s, T=T, dx_dtype=DT, dX_out=dX, dA_out=dA, dB_out=dB,
                            workspace=ws)

    def dx_only():   # the streaming input gradient alone (r = 0): its kernel and split reduce
        QB.qlora_linear_bwd(q, cb, None, dY, dx_dtype=DT, dX_out=dX0, workspace=ws0)

    def cold_times(fn, n, warmup):
        """GPU time of fn after a 2 GiB fill: the host enqueues the events and
        fn's launches while the fill runs (host_us says how long that took),
        so the interval holds fn's kernels back to back."""
        out, host = [], []
        for i in range(warmup + n):
            flush.fill_(i & 255)
            e0, e1 = _events()
            h0 = time.perf_counter()
            e0.record()
            fn()
            e1.record()
            h1 = time.perf_counter()
            torch.cuda.synchronize()
            if i >= warmup:
                out.append(e0.elapsed_time(e1))
                host.append((h1 - h0) * 1e6)
        return out, statistics.median(host)

    step(); dx_only()
    torch.cuda.synchronize()
    flush.fill_(2)
    f0, f1 = _events()
    f0.record()
    flush.fill_(1)
    f1.record()
    torch.cuda.synchronize()
    fill_us = f0.elapsed_time(f1) * 1e3
    t0 = time.perf_counter()
    step_ms, host_step = cold_times(step, args.steps, args.warmup)
    wall_s = time.perf_counter() - t0
    dx_ms, host_dx = cold_times(dx_only, args.steps, args.warmup)
    ms = statistics.median(step_ms)
    flops = flops_fwd(M, N, K, r) + flops_bwd(M, N, K, r)
    nbytes = step_bytes(M, N, K, r)
    dx_bytes = packed_bytes(N, K) + 2 * M * N + 2 * M * K
    dx_us = statistics.median(dx_ms) * 1e3
    achieved = dx_bytes / (dx_us * 1e-6) / 1e9
    out = {
        "metric": METRIC, "value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "us_per_step": round(ms * 1e3, 2), "tflops": round(flops / (ms * 1e-3) / 1e12, 4),
        "wall_ms_per_step_incl_flush": round(wall_s * 1e3 / (args.steps + args.warmup), 4),
        "host_enqueue_us": {"step": round(host_step, 1), "dx": round(host_dx, 1),
                            "fill_us": round(fill_us, 1),
                            "covered_by_fill": bool(max(host_step, host_dx) < fill_us)},
        "gpu_step_ms": _spread(step_ms),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt_name(),
        "data": "synthetic (seeded N(0,0.02) weight quantized to NF4+DQ, N(0,1) X and dY, N(0,0.01) A, B)",
        "config": {"workload": SINGLE_WORKLOAD, "M": M, "N": N, "K": K, "r": r, "alpha": ALPHA,
                   "double_quant": DQ, "nf4_block": BLOCK, "path": "auto (small-m streaming)",
                   "parallelism": "none (1 GPU)"},
        "algorithmic_bytes_per_step": nbytes,
        "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": "k_gemv_dx", "interval": "k_gemv_dx + k_reduce (its split sum)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "avg_launch_us": round(dx_us, 2),
                     "bytes_per_launch": dx_bytes, "traffic": None},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_single()
    return out


def cpu_baseline_single():
    """The oracle as it stands on the same single-linear step (dequantize,
    forward, dequantize, backward in float64 numpy), repeated for about 10 s;
    then with one thread."""
    import synth
    from oracle import linear as olin
    from oracle import nf4 as onf4

    lv, mid = onf4.codebook()
    M, N, K, r = SINGLE_M, 4096, 4096, RANK
    W = synth.normal_bf16((N, K), 0.02, synth.tensor_seed(1, 0))
    codes, qs, st = onf4.quantize(W, mid)
    X = synth.normal_bf16((M, K), 1.0, synth.tensor_seed(1, 1))
    A = synth.normal_bf16((r, K), 0.01, synth.tensor_seed(1, 2))
    B = synth.normal_bf16((N, r), 0.01, synth.tensor_seed(1, 3))
    dY = synth.normal_bf16((M, N), 1.0, synth.tensor_seed(1, 4))
    nbytes = step_bytes(M, N, K, r)

    def run(budget_s):
        n, t0 = 0, time.perf_counter()
        while True:
            Wd = onf4.dequantize(codes, qs, st, lv).reshape(N, K)
            olin.forward(Wd, X, A, B, ALPHA / RANK)
            Wd = onf4.dequantize(codes, qs, st, lv).reshape(N, K)
            olin.backward(Wd, X, dY, A, B, ALPHA / RANK)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                return n * nbytes, el, f"{n} steps of the same workload"
    return with_cpu_figures(run, "GB/s", 1e9, 10.0, 5.0)


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _spread(ms):
    """Median and spread of per-step GPU times (ms)."""
    v = sorted(ms)
    return {"median": round(statistics.median(v), 4), "min": round(v[0], 4), "max": round(v[-1], 4),
            "n": len(v)}


def _timed(fn, steps, warmup):
    """Run fn warmup times, then time `steps` runs with HIP events on the
    current stream (one event per run boundary): (wall seconds per run, GPU
    seconds per run, per-run GPU milliseconds)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    return wall, ev[0].elapsed_time(ev[-1]) * 1e-3 / steps, [ev[i].elapsed_time(ev[i + 1])
                                                             for i in range(steps)]


def _traffic(kernel, srcs):
    return traffic_from_profile(kernel, srcs)


def run_decode(args):
    """Forward-only sweep over 32 layers x 7 projections at small M, one grouped
    launch (plus one for the LoRA T products) per sweep."""
    import torch

    import synth
    from qlora_fine_tuning_nf4_amd import binding as QB

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cb = QB.device_codebook(dev)
    weights = []
    for layer in range(DECODE_LAYERS):
        for i, (name, N, K, r) in enumerate(PROJ):
            W = dnorm((N, K), 0.02, synth.tensor_seed(3, 100 * layer + 10 * i),
                                         device=dev)
            weights.append((QB.qlora_quantize(W, cb, double_quant=DQ, block=BLOCK), N, K, r))
            del W
    torch.cuda.synchronize()
    per_m = {}
    kern = None
    # a sweep is under a millisecond: the clock transient after idle spans about
    # 25 sweeps, so at least 40 untimed sweeps precede each timed series
    warm = max(args.warmup, DECODE_SETTLE_SWEEPS)
    for M in (1, 4, 16):
        jobs, jobs0 = [], []
        nbytes = nbytes0 = 0
        for idx, (q, N, K, r) in enumerate(weights):
            X = dnorm((M, K), 1.0, synth.tensor_seed(3, 20000 + idx), device=dev)
            Y = torch.empty((M, N), dtype=DT, device=dev)
            j = dict(w=q, X=X, Y=Y)
            b0 = q.nbytes() + 2 * M * K + 2 * M * N
            nbytes0 += b0
            nbytes += b0
            if r:
                j.update(A=dnorm((r, K), 0.01, synth.tensor_seed(3, 40000 + idx),
                                                    device=dev),
                         B=dnorm((N, r), 0.01, synth.tensor_seed(3, 60000 + idx),
                                                    device=dev),
                         scaling=ALPHA / RANK, T=torch.empty((M, r), dtype=torch.float32, device=dev))
                nbytes += 2 * r * K + 2 * N * r + 4 * M * r
            jobs.append(j)
            jobs0.append(dict(w=q, X=X, Y=Y))
        g = QB.qlora_group_init(jobs, M, y_dtype=DT)
        g0 = QB.qlora_group_init(jobs0, M, y_dtype=DT)
        wall, gpu, sweeps = _timed(lambda: QB.qlora_linear_fwd_grouped(g, cb), args.steps, warm)
        # the streaming kernel alone: the same sweep without LoRA is one launch
        wall0, gpu0, _ = _timed(lambda: QB.qlora_linear_fwd_grouped(g0, cb), args.steps, warm)
        per_m[str(M)] = {"ms_per_sweep": round(wall * 1e3, 4), "GBps": round(nbytes / wall / 1e9, 1),
                         "frac_of_hbm_peak": round(nbytes / wall / 1e9 / PEAK_HBM_GBS, 4),
                         "kernel_us": round(gpu0 * 1e6, 1),
                         "kernel_GBps": round(nbytes0 / gpu0 / 1e9, 1),
                         "gpu_sweep_ms": _spread(sweeps)}
        if M == 1:
            kern = (nbytes0, gpu0, wall, nbytes)
        del g, g0, jobs, jobs0
    nbytes0, gpu0, wall, nbytes = kern
    achieved = nbytes0 / gpu0 / 1e9
    out = {
        "metric": "QLoRA NF4 decode-sweep forward effective GB/s (% HBM roofline) on 1 MI355X",
        "value": round(nbytes / wall / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": warm, "ms_per_step": round(wall * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dt_name(),
        "data": "synthetic (seeded N(0,0.02) weights quantized to NF4+DQ, N(0,1) activations)",
        "config": {"workload": f"decode sweep: {DECODE_LAYERS} layers x (q,k,v,o 4096x4096; gate,up "
                               "11008x4096; down 4096x11008), M=1, LoRA r=8 alpha=16 on q,k,v,o, "
                               "forward only, one grouped launch per sweep",
                   "M": 1, "layers": DECODE_LAYERS, "double_quant": DQ, "nf4_block": BLOCK, "params": sum(N * K for _, N, K, _ in weights),
                   "packed_bytes": sum(q.nbytes() for q, *_ in weights), "parallelism": "none (1 GPU)"},
        "per_m": per_m,
        "roofline": {"bound": "hbm", "kernel": "k_gemv_fwd", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "avg_launch_us": round(gpu0 * 1e6, 1),
                     "traffic": _traffic("k_gemv_fwd", ["gemv.hip", "common.h"])},
    }
    if not args.no_measured_peaks:
        mp = measured_peaks()
        out["roofline"]["measured_peak"] = {"value": mp["stream_read_GBps"], "unit": "GB/s",
                                            "frac": round(achieved / mp["stream_read_GBps"], 4), "all": mp}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode()
    return out


def cpu_baseline_decode():
    """The oracle on a bounded sample of the decode sweep: dequantize + forward
    of the seven projections of the first CPU_DECODE_LAYERS layers at M = 1
    (float64 numpy)."""
    import synth
    from oracle import linear as olin
    from oracle import nf4 as onf4

    lv, mid = onf4.codebook()

    def run(layers):
        nbytes, elapsed = 0, 0.0
        for layer in range(layers):
            for i, (name, N, K, r) in enumerate(PROJ):
                idx = 7 * layer + i
                W = synth.normal_bf16((N, K), 0.02, synth.tensor_seed(3, 100 * layer + 10 * i))
                codes, qs, st = onf4.quantize(W, mid)
                X = synth.normal_bf16((1, K), 1.0, synth.tensor_seed(3, 20000 + idx))
                A = synth.normal_bf16((r, K), 0.01, synth.tensor_seed(3, 40000 + idx)) if r else None
                B = synth.normal_bf16((N, r), 0.01, synth.tensor_seed(3, 60000 + idx)) if r else None
                t0 = time.perf_counter()
                Wd = onf4.dequantize(codes, qs, st, lv).reshape(N, K)
                olin.forward(Wd, X, A, B, ALPHA / RANK)
                elapsed += time.perf_counter() - t0
                nbytes += packed_bytes(N, K) + 2 * K + 2 * N
        return (nbytes, elapsed, f"{layers} of the {DECODE_LAYERS} layers (7 projections each) at "
                                 "M=1: dequantize + forward in float64 numpy")
    return with_cpu_figures(run, "GB/s", 1e9, CPU_DECODE_LAYERS, 1)


def _weights70(dev):
    import synth
    out = []
    for i, (name, N, K) in enumerate(PROJ70):
        out.append(dnorm((N, K), 0.015, synth.tensor_seed(4, 10 * i), device=dev,
                                            outlier_rate=0.001, outlier_scale=20))
    return out


def run_quantize70b(args):
    import torch

    from qlora_fine_tuning_nf4_amd import binding as QB

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cb = QB.device_codebook(dev)
    Ws = _weights70(dev)
    outs = [QB.NF4Weight.empty(N, K, dev, double_quant=DQ, block=BLOCK, dtype=DT) for _, N, K in PROJ70]
    params = sum(N * K for _, N, K in PROJ70)
    nbytes = sum(2 * N * K + packed_bytes(N, K) for _, N, K in PROJ70)

    def step():
        for W, o in zip(Ws, outs):
            QB.qlora_quantize(W, cb, out=o)
    wall, gpu, steps_ms = _timed(step, args.steps, args.warmup)
    # largest projection alone (one launch) for the kernel roofline
    big = 4
    kb = 2 * PROJ70[big][1] * PROJ70[big][2] + packed_bytes(PROJ70[big][1], PROJ70[big][2])
    _, gk, _ = _timed(lambda: QB.qlora_quantize(Ws[big], cb, out=outs[big]), args.steps, args.warmup)
    ach = kb / gk / 1e9
    out = {
        "metric": "NF4 + double-quant quantization GB/s (% HBM roofline) on 1 MI355X",
        "value": round(nbytes / wall / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 4), "gpu_step_ms": _spread(steps_ms),
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dt_name() + "->u8",
        "data": "synthetic (seeded N(0,0.015) bf16 weights, 0.1% outliers x20)",
        "config": {"workload": "quantize a 70B-style layer: q,k,v,o 8192x8192; gate,up 28672x8192; "
                               "down 8192x28672 (973,078,528 params)", "params": params,
                   "double_quant": DQ, "nf4_block": BLOCK,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "k_quant_nf4_dq", "achieved": round(ach, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                     "avg_launch_us": round(gk * 1e6, 1),
                     "traffic": _traffic("k_quant_nf4_dq", ["quantize.hip", "common.h"])},
    }
    if not args.no_cpu_baseline:
        import synth
        from oracle import nf4 as onf4
        _, mid = onf4.codebook()

        def run(rows):
            W = synth.normal_bf16((rows, 8192), 0.015, 77, outlier_rate=0.001, outlier_scale=20)
            t0 = time.perf_counter()
            onf4.quantize(W, mid)
            el = time.perf_counter() - t0
            return (2 * rows * 8192 + packed_bytes(rows, 8192), el,
                    f"{rows} x 8192 rows of the q projection")
        out["cpu_baseline"] = with_cpu_figures(run, "GB/s", 1e9, 16384, 4096)
    return out


def run_layer70b(args):
    import torch

    import synth
    from qlora_fine_tuning_nf4_amd import binding as QB

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cb = QB.device_codebook(dev)
    M, r, alpha = 4096, 16, 32
    s = alpha / r
    layers = []
    for i, (W, (name, N, K)) in enumerate(zip(_weights70(dev), PROJ70)):
        q = QB.qlora_quantize(W, cb, double_quant=DQ, block=BLOCK)
        del W
        L = dict(N=N, K=K, q=q)
        L["X"] = dnorm((M, K), 1.0, synth.tensor_seed(4, 10 * i + 1), device=dev)
        L["dY"] = dnorm((M, N), 1.0, synth.tensor_seed(4, 10 * i + 2), device=dev)
        L["A"] = dnorm((r, K), 0.01, synth.tensor_seed(4, 10 * i + 3), device=dev)
        L["B"] = dnorm((N, r), 0.01, synth.tensor_seed(4, 10 * i + 4), device=dev)
        L["Y"] = torch.empty((M, N), dtype=DT, device=dev)
        L["T"] = torch.empty((M, r), dtype=torch.float32, device=dev)
        L["dX"] = torch.empty((M, K), dtype=DT, device=dev)
        L["dA"] = torch.empty((r, K), dtype=torch.float32, device=dev)
        L["dB"] = torch.empty((N, r), dtype=torch.float32, device=dev)
        nws = max(QB.qlora_workspace_bytes(0, M, N, K, r), QB.qlora_workspace_bytes(1, M, N, K, r), 16)
        L["ws"] = torch.empty(nws, dtype=torch.uint8, device=dev)
        layers.append(L)
    torch.cuda.synchronize()

    def step():
        for L in layers:
            QB.qlora_linear_fwd(L["q"], cb, L["X"], L["A"], L["B"], s, out=L["Y"], T_out=L["T"],
                                workspace=L["ws"])
            QB.qlora_linear_bwd(L["q"], cb, L["X"], L["dY"], L["A"], L["B"], s, T=L["T"],
                                dX_out=L["dX"], dA_out=L["dA"], dB_out=L["dB"], workspace=L["ws"])
    wall, gpu, steps_ms = _timed(step, args.steps, args.warmup)
    flops = sum(flops_fwd(M, L["N"], L["K"], r) + flops_bwd(M, L["N"], L["K"], r) for L in layers)
    tf = flops / wall / 1e12

    # the fused-dequant GEMMs alone (LoRA off: one launch per call), timed with
    # HIP events on the stream they run on
    def gemm_only(dx):
        def f():
            for L in layers:
                if dx:
                    QB.qlora_linear_bwd(L["q"], cb, None, L["dY"], dX_out=L["dX"], workspace=L["ws"])
                else:
                    QB.qlora_linear_fwd(L["q"], cb, L["X"], out=L["Y"], workspace=L["ws"])
        return f
    kf = 2 * M * sum(L["N"] * L["K"] for L in layers)
    _, gf, _ = _timed(gemm_only(False), args.steps, args.warmup)
    _, gd, _ = _timed(gemm_only(True), args.steps, args.warmup)
    tf_f, tf_d = kf / gf / 1e12, kf / gd / 1e12
    kname, ach, t_k = ("k_gemm_dx", tf_d, gd) if gd >= gf else ("k_gemm_fwd", tf_f, gf)
    out = {
        "metric": METRIC, "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 4),
        "gpu_event_ms_per_step": round(gpu * 1e3, 4), "gpu_step_ms": _spread(steps_ms),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dt_name(),
        "data": "synthetic (seeded N(0,0.015) weights with 0.1% outliers x20, NF4+DQ; N(0,1) activations)",
        "config": {"workload": "70B-style layer linears (q,k,v,o 8192x8192; gate,up 28672x8192; down "
                               "8192x28672), M=4096 tokens, LoRA r=16 alpha=32 on all seven, fwd+bwd",
                   "M": M, "r": r, "alpha": alpha, "double_quant": DQ, "nf4_block": BLOCK, "parallelism": "none (1 GPU)"},
        "frac_of_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": kname, "achieved": round(ach, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                     "avg_launch_us": round(t_k / len(layers) * 1e6, 2),
                     "traffic": None,
                     "other_gemm": {"k_gemm_fwd": round(tf_f, 1), "k_gemm_dx": round(tf_d, 1)}},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_layer70(args.cpu_sample_tokens or 4096)
    return out


def cpu_baseline_layer70(sample_tokens):
    """The oracle on a bounded sample of the 70B-style layer: the q
    projection (8192 x 8192, its N(0, 0.015) weight with outliers) at the
    first `sample_tokens` tokens, dequantize + forward + backward with LoRA
    r = 16 in float64 numpy (quantization outside the timed part)."""
    import synth
    from oracle import linear as olin
    from oracle import nf4 as onf4

    lv, mid = onf4.codebook()
    N, K, r, s = 8192, 8192, 16, 32 / 16
    W = synth.normal_bf16((N, K), 0.015, synth.tensor_seed(6, 0), outlier_rate=0.001, outlier_scale=20)
    c, qs, st = onf4.quantize(W, mid)

    def run(M):
        X = synth.normal_bf16((M, K), 1.0, synth.tensor_seed(6, 1))
        dY = synth.normal_bf16((M, N), 1.0, synth.tensor_seed(6, 2))
        A = synth.normal_bf16((r, K), 0.01, synth.tensor_seed(6, 3))
        B = synth.normal_bf16((N, r), 0.01, synth.tensor_seed(6, 4))
        t0 = time.perf_counter()
        olin.forward(onf4.dequantize(c, qs, st, lv).reshape(N, K), X, A, B, s)
        olin.backward(onf4.dequantize(c, qs, st, lv).reshape(N, K), X, dY, A, B, s)
        el = time.perf_counter() - t0
        return (flops_fwd(M, N, K, r) + flops_bwd(M, N, K, r), el,
                f"q projection (8192 x 8192) at M={M} of the 4096 tokens: "
                "dequantize + fwd + bwd in float64 numpy")
    return with_cpu_figures(run, "TFLOP/s", 1e12, sample_tokens, max(1, sample_tokens // 16))


PROJ38 = [("q", 3072, 3072), ("k", 3072, 3072), ("v", 3072, 3072), ("o", 3072, 3072),
          ("gate", 8192, 3072), ("up", 8192, 3072), ("down", 3072, 8192)]
FORMAT_NAMES = {"q8_0": "Q8_0 (32 int8 + fp16 scale per 32)",
                "u4_asym": "asymmetric uint4 (fp32 scale + zero-point per 64)",
                "nf4": "NF4 + double quantization"}


def format_bytes(fmt, N, K):
    """Packed bytes of an N x K weight in block format `fmt`."""
    if fmt == "q8_0":
        return N * K + 2 * (N * K // 32)
    if fmt == "u4_asym":
        return N * K // 2 + 8 * (N * K // 64)
    return packed_bytes(N, K)


def cpu_baseline_layer38(fmt, sample_tokens):
    """The oracle on a bounded sample of the 3.8B-style layer: all seven
    projections at the first `sample_tokens` tokens, dequantize + forward +
    backward in float64 numpy (quantization outside the timed part)."""
    import synth
    from oracle import formats as ofmt
    from oracle import linear as olin
    from oracle import nf4 as onf4

    lv, mid = onf4.codebook()

    def run(M):
        return _layer38_sample(fmt, M, lv, mid, synth, ofmt, olin, onf4)
    return with_cpu_figures(run, "TFLOP/s", 1e12, sample_tokens, max(1, sample_tokens // 16))


def _layer38_sample(fmt, M, lv, mid, synth, ofmt, olin, onf4):
    r, s = 64, 128 / 64
    total_flops, elapsed = 0, 0.0
    for i, (name, N, K) in enumerate(PROJ38):
        W = synth.normal_bf16((N, K), 0.02, synth.tensor_seed(5, 10 * i))
        X = synth.normal_bf16((M, K), 1.0, synth.tensor_seed(5, 10 * i + 1))
        dY = synth.normal_bf16((M, N), 1.0, synth.tensor_seed(5, 10 * i + 2))
        A = synth.normal_bf16((r, K), 0.01, synth.tensor_seed(5, 10 * i + 3))
        B = synth.normal_bf16((N, r), 0.01, synth.tensor_seed(5, 10 * i + 4))
        if fmt == "q8_0":
            qv, d16 = ofmt.q8_quantize(W)
            deq = lambda: ofmt.q8_dequantize(qv, d16).reshape(N, K)   # noqa: E731
        elif fmt == "u4_asym":
            c, sc, zp = ofmt.u4_quantize(W)
            deq = lambda: ofmt.u4_dequantize(c, sc, zp).reshape(N, K)   # noqa: E731
        else:
            c, qs, st = onf4.quantize(W, mid)
            deq = lambda: onf4.dequantize(c, qs, st, lv).reshape(N, K)   # noqa: E731
        t0 = time.perf_counter()
        olin.forward(deq(), X, A, B, s)
        olin.backward(deq(), X, dY, A, B, s)
        elapsed += time.perf_counter() - t0
        total_flops += flops_fwd(M, N, K, r) + flops_bwd(M, N, K, r)
    return (total_flops, elapsed, f"all 7 projections at M={M} of the 4096 tokens: dequantize + "
                                  "fwd + bwd in float64 numpy")


def run_layer38(args):
    import torch

    import synth
    from qlora_fine_tuning_nf4_amd import binding as QB

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fmt = args.format
    fcode = QB.FORMATS[fmt]
    cb = QB.device_codebook(dev) if fmt == "nf4" else None
    M, r, alpha = 4096, 64, 128
    s = alpha / r
    layers = []
    for i, (name, N, K) in enumerate(PROJ38):
        W = synth.device_normal_bf16((N, K), 0.02, synth.tensor_seed(5, 10 * i), device=dev)
        q = QB.qlora_quantize(W, cb, double_quant=DQ, fmt=fcode, block=BLOCK if fmt == "nf4" else 64)
        del W
        L = dict(N=N, K=K, q=q)
        L["X"] = synth.device_normal_bf16((M, K), 1.0, synth.tensor_seed(5, 10 * i + 1), device=dev)
        L["dY"] = synth.device_normal_bf16((M, N), 1.0, synth.tensor_seed(5, 10 * i + 2), device=dev)
        L["A"] = synth.device_normal_bf16((r, K), 0.01, synth.tensor_seed(5, 10 * i + 3), device=dev)
        L["B"] = synth.device_normal_bf16((N, r), 0.01, synth.tensor_seed(5, 10 * i + 4), device=dev)
        L["Y"] = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        L["T"] = torch.empty((M, r), dtype=torch.float32, device=dev)
        L["dX"] = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        L["dA"] = torch.empty((r, K), dtype=torch.float32, device=dev)
        L["dB"] = torch.empty((N, r), dtype=torch.float32, device=dev)
        nws = max(QB.qlora_workspace_bytes(0, M, N, K, r), QB.qlora_workspace_bytes(1, M, N, K, r), 16)
        L["ws"] = torch.empty(nws, dtype=torch.uint8, device=dev)
        layers.append(L)
    torch.cuda.synchronize()

    def step():
        for L in layers:
            QB.qlora_linear_fwd(L["q"], cb, L["X"], L["A"], L["B"], s, out=L["Y"], T_out=L["T"],
                                workspace=L["ws"])
            QB.qlora_linear_bwd(L["q"], cb, L["X"], L["dY"], L["A"], L["B"], s, T=L["T"],
                                dX_out=L["dX"], dA_out=L["dA"], dB_out=L["dB"], workspace=L["ws"])
    wall, gpu, steps_ms = _timed(step, args.steps, args.warmup)
    flops = sum(flops_fwd(M, L["N"], L["K"], r) + flops_bwd(M, L["N"], L["K"], r) for L in layers)
    tf = flops / wall / 1e12

    # the fused-dequant GEMMs alone (LoRA off: one launch per call), timed with
    # HIP events on the stream they run on
    def gemm_only(dx):
        def f():
            for L in layers:
                if dx:
                    QB.qlora_linear_bwd(L["q"], cb, None, L["dY"], dX_out=L["dX"], workspace=L["ws"])
                else:
                    QB.qlora_linear_fwd(L["q"], cb, L["X"], out=L["Y"], workspace=L["ws"])
        return f
    kf = 2 * M * sum(L["N"] * L["K"] for L in layers)
    _, gf, _ = _timed(gemm_only(False), args.steps, args.warmup)
    _, gd, _ = _timed(gemm_only(True), args.steps, args.warmup)
    tf_f, tf_d = kf / gf / 1e12, kf / gd / 1e12
    kname, ach, t_k = ("k_gemm_dx", tf_d, gd) if gd >= gf else ("k_gemm_fwd", tf_f, gf)
    out = {
        "metric": METRIC, "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 4),
        "gpu_event_ms_per_step": round(gpu * 1e3, 4), "gpu_step_ms": _spread(steps_ms),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": f"synthetic (seeded N(0,0.02) weights in {FORMAT_NAMES[fmt]}; N(0,1) activations)",
        "config": {"workload": "3.8B-style layer linears (q,k,v,o 3072x3072; gate,up 8192x3072; down "
                               "3072x8192), M=4096 tokens (seq 4096), LoRA r=64 alpha=128 on all "
                               f"seven, fwd+bwd, weights {FORMAT_NAMES[fmt]}",
                   "M": M, "r": r, "alpha": alpha, "format": fmt,
                   "double_quant": DQ if fmt == "nf4" else None, "nf4_block": BLOCK if fmt == "nf4" else None,
                   "packed_bytes": sum(L["q"].nbytes() for L in layers),
                   "parallelism": "none (1 GPU)"},
        "frac_of_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": kname, "achieved": round(ach, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                     "avg_launch_us": round(t_k / len(layers) * 1e6, 2),
                     "traffic": None,
                     "other_gemm": {"k_gemm_fwd": round(tf_f, 1), "k_gemm_dx": round(tf_d, 1)}},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_layer38(fmt, args.cpu_sample_tokens or 128)
    return out


def measured_peaks(read_bytes=1 << 30, mfma_iters=4096, reps=10):
    """The part's measured ceilings on this machine (``libqlora_peaks.so``): a
    streaming read of `read_bytes` in two orders, a device copy of half that,
    and a bf16 MFMA 32x32x16 loop, each the median over `reps` launches timed
    with HIP events on the launching stream."""
    import torch

    from qlora_fine_tuning_nf4_amd import peaks

    dev = torch.device("cuda:0")
    buf = torch.ones(read_bytes, dtype=torch.uint8, device=dev)
    dst = torch.empty(read_bytes // 2, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def med_ms(fn):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            t.append(e0.elapsed_time(e1))
        return sorted(t)[len(t) // 2]

    t_rr = med_ms(lambda: peaks.read(buf, True, sink))
    t_rs = med_ms(lambda: peaks.read(buf, False, sink))
    half = buf[: read_bytes // 2]
    t_cp = med_ms(lambda: peaks.copy(half, dst))
    t_mf = med_ms(lambda: peaks.mfma(mfma_iters, sink))
    flops = peaks.mfma_flops(mfma_iters)
    del buf, dst
    return {"stream_read_GBps": round(read_bytes / t_rr / 1e6, 1),
            "stream_read_grid_stride_GBps": round(read_bytes / t_rs / 1e6, 1),
            "copy_GBps": round(2 * (read_bytes // 2) / t_cp / 1e6, 1),
            "mfma_bf16_loop_TFLOPs": round(flops / t_mf / 1e9, 1),
            "how": f"median of {reps} launches each (HIP events): a {read_bytes >> 20} MiB read "
                   "(4096 workgroups on contiguous ranges; and grid-stride), a copy of half of it "
                   "(read + write bytes), 1024 workgroups x 4 waves x "
                   f"{mfma_iters} iterations of 8 independent bf16 MFMA 32x32x16 chains"}


REGIME_SHAPES = [(4096, 4096), (11008, 4096), (4096, 11008)]
REGIME_M = [1, 4, 16, 32, 48, 64, 96, 128]


def run_regime(args):
    """The small-token regime split: forward and input-gradient GPU time of
    the streaming kernels (m <= 32) and of the tiled GEMMs at each m, for the
    7B projection shapes (no LoRA), warm (20 calls enqueued behind a 2 GiB
    fill, HIP events around them) and cold (2 GiB written before each call)."""
    import torch

    import synth
    from qlora_fine_tuning_nf4_amd import binding as QB

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cb = QB.device_codebook(dev)
    stream = torch.cuda.current_stream()
    flush = torch.empty(1 << 31, dtype=torch.uint8, device=dev)

    def warm_us(fn, n=20):
        # enqueued behind a 2 GiB fill, so the calls run back to back on the
        # GPU whatever the host's per-call cost
        fn()
        torch.cuda.synchronize()
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    def cold_us(fn, n=10):
        ts = []
        for _ in range(n):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return sorted(ts)[len(ts) // 2]

    rows, cross = [], {}
    for N, K in REGIME_SHAPES:
        q = QB.qlora_quantize(dnorm((N, K), 0.02, synth.tensor_seed(7, N + K), device=dev), cb)
        ws = torch.empty(max(QB.qlora_workspace_bytes(0, 128, N, K, 0),
                             QB.qlora_workspace_bytes(1, 128, N, K, 0), 16), dtype=torch.uint8, device=dev)
        Y = torch.empty((128, N), dtype=DT, device=dev)
        dXo = torch.empty((128, K), dtype=DT, device=dev)
        for M in REGIME_M:
            X = dnorm((M, K), 1.0, synth.tensor_seed(7, M), device=dev)
            dY = dnorm((M, N), 1.0, synth.tensor_seed(7, M + 1), device=dev)
            rec = {"N": N, "K": K, "M": M}
            for path in ("gemv", "gemm"):
                if path == "gemv" and M > 32:
                    continue
                f = lambda: QB.qlora_linear_fwd(q, cb, X, out=Y[:M], workspace=ws, path=path)   # noqa: E731
                b = lambda: QB.qlora_linear_bwd(q, cb, None, dY, dX_out=dXo[:M], workspace=ws, path=path)   # noqa: E731
                rec[f"fwd_{path}_warm_us"] = round(warm_us(f), 2)
                rec[f"dx_{path}_warm_us"] = round(warm_us(b), 2)
                rec[f"fwd_{path}_cold_us"] = round(cold_us(f), 2)
                rec[f"dx_{path}_cold_us"] = round(cold_us(b), 2)
            rows.append(rec)
        # largest m at which the streaming kernels are faster (warm, forward and dX)
        wins = [r["M"] for r in rows if r["N"] == N and r["K"] == K and "fwd_gemv_warm_us" in r
                and r["fwd_gemv_warm_us"] < r["fwd_gemm_warm_us"] and r["dx_gemv_warm_us"] < r["dx_gemm_warm_us"]]
        cross[f"{N}x{K}"] = max(wins) if wins else 0
        del q, ws
    del flush
    return {"metric": "small-token regime split: streaming vs tiled GEMM time per call (7B projection shapes)",
            "value": min(cross.values()), "unit": "largest m where the streaming path wins (all shapes)",
            "n_gpus": 1, "steps": 20, "warmup": 1, "ms_per_step": None, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dt_name(),
            "data": "synthetic (seeded N(0,0.02) weights, NF4+DQ; N(0,1) activations and gradients)",
            "config": {"workload": "regime split sweep, m in " + str(REGIME_M) + ", no LoRA",
                       "shapes": REGIME_SHAPES, "auto_switch_m": 32,
                       "streaming_limit_m": 32},
            "streaming_wins_up_to_m": cross, "sweep": rows}


def run_peaks(args):
    """The measured ceilings alone, as one JSON line."""
    m = measured_peaks()
    return {"metric": "MI355X measured ceilings: streaming read, device copy, bf16 MFMA loop",
            "value": m["stream_read_GBps"], "unit": "GB/s", "n_gpus": 1, "steps": 10, "warmup": 1,
            "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "u8 (read), bf16 (MFMA)", "data": "synthetic (a device buffer of ones)",
            "config": {"workload": "measured ceilings of one MI355X"},
            "measured": m,
            "roofline": {"bound": "hbm", "kernel": "k_read_ranges", "achieved": m["stream_read_GBps"],
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(m["stream_read_GBps"] / PEAK_HBM_GBS, 4), "traffic": None,
                         "mfma": {"achieved": m["mfma_bf16_loop_TFLOPs"], "peak": PEAK_BF16_TFLOPS,
                                  "unit": "TFLOP/s",
                                  "frac": round(m["mfma_bf16_loop_TFLOPs"] / PEAK_BF16_TFLOPS, 4)}}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # from idle the part runs its first steps at a higher clock, then lower for
    # a few tens of milliseconds before it settles: the default warmup covers
    # that (about 10 steps of the default workload)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-library-baseline", action="store_true",
                    help="layer7b: skip the hipBLASLt comparison of the base products")
    ap.add_argument("--no-measured-peaks", action="store_true",
                    help="layer7b, decode: skip measuring the part's ceilings beside the data-sheet peaks")
    ap.add_argument("--single-level", action="store_true",
                    help="weights without double quantization (fp32 absmax per block); "
                         "no CPU baseline (the oracle baselines time the double-quantized format)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=None,
                    help="tokens of the oracle's CPU baseline (default: all 2048 of layer7b, "
                         "128 of the 4096 of layer3.8b)")
    ap.add_argument("--workload", default="layer7b",
                    choices=["layer7b", "single", "decode", "quantize70b", "layer70b", "layer3.8b",
                             "peaks", "regime"])
    ap.add_argument("--format", default="q8_0", choices=["q8_0", "u4_asym", "nf4"],
                    help="weight block format of the layer3.8b workload")
    ap.add_argument("--nf4-block", type=int, default=64, choices=[32, 64, 128],
                    help="NF4 block size; no CPU baseline unless 64 (the oracle baselines time "
                         "block 64)")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "f16"],
                    help="compute type of the NF4 workloads (f16: block 64 with double "
                         "quantization only; no CPU baseline)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only; --gpus must be 1 "
              "(sharding over several GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)
    global DQ, BLOCK, DT
    if args.dtype == "f16":
        if args.single_level or args.nf4_block != 64 or args.workload == "layer3.8b":
            print("--dtype f16 needs NF4 at block 64 with double quantization", file=sys.stderr)
            sys.exit(2)
        DT = torch.float16
        args.no_cpu_baseline = True
    if args.single_level:
        DQ = False
        args.no_cpu_baseline = True
    BLOCK = args.nf4_block
    if BLOCK != 64:
        args.no_cpu_baseline = True

    run = {"layer7b": run_layer7b, "single": run_single, "decode": run_decode, "quantize70b": run_quantize70b,
           "layer70b": run_layer70b, "layer3.8b": run_layer38, "peaks": run_peaks,
           "regime": run_regime}[args.workload]
    out = run(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
