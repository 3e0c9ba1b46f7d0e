#!/usr/bin/env python3
"""Benchmark of the exact attention forward on one MI355X.

One step = one call of the fused bf16 kernel over the whole workload (every
head, every query row), inputs already resident in HBM.  Default workload: the
causal long-sequence case B=1, H=32, N=32768, d=128 (seeded N(0,1) inputs).

Prints ONE JSON line with the throughput in algorithmic TFLOP/s (4*d FLOPs per
(query, visible key) pair, i.e. 4*N^2*d per head halved for causal), the
roofline position of the kernel (timed live with HIP events on the launch
stream), the HBM traffic measured by rocprofv3 counters when a matching
counter summary is committed under profiles/, and the fp64 CPU oracle timed on
a bounded row sample on the host cores (which also checks those rows).

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
  python bench.py --mode bwd [--workload NAME]   # the backward (bf16 workloads)
  python bench.py --mode unfused [--workload NAME] [--heads-per-pass G]
  python bench.py --mode rows [--workload softmax_r32k_n32k|layernorm_r128k_n8k]
  python bench.py --mode fp8 [--workload NAME]   # the workload's shape with E4M3 inputs
  python bench.py --mode tilings --all-workloads  # every compiled tiling vs the I/O model's pick
  python bench.py --copy-calib BYTES   # plain device copy, for counter calibration
  python bench.py --read-calib BYTES [--read-repeats 8]   # one buffer read repeatedly

In --mode bwd one step is one attn_bwd call (its three kernels) from the
forward's O and log-sum-exp, which are computed before the timed region; the
throughput counts 10*d FLOPs per visible pair (the five products S, dP, dV, dK,
dQ of the backward, each 2*d per pair).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

# BLAS threads of the CPU oracle leg, set before numpy is first imported (torch
# imports it): every host core this process may run on, unless the caller or
# the machine already fixed a count.
_HOST_THREADS = os.environ.get("OMP_NUM_THREADS") or str(len(os.sched_getaffinity(0)))
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_var, _HOST_THREADS)

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (no sparsity)
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
DEFAULT_WORKLOAD = "bf16_causal_h32_n32k_d128"
KERNEL_SOURCE = os.path.join(ROOT, "exact_long_sequence_amd", "csrc", "attn_fwd_bf16.hip")


def kernel_source_digest() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counter_summary_path(w) -> str:
    """profiles/ summary of the HBM counters taken on workload w (bf16 kernel)."""
    kind = "causal" if w.causal else ("padded" if w.padded else "full")
    return os.path.join(ROOT, "profiles",
                        f"attn_fwd_bf16_{kind}_b{w.B}_h{w.H}_n{w.N // 1024}k_d{w.d}_counters.md")


def committed_traffic(w):
    """HBM bytes per launch from the committed counter summary of workload w, or
    None when there is none or it was taken on a different kernel source."""
    path = counter_summary_path(w)
    if w.dtype != "bf16" or not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]{16})", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_sha and m_b) or m_sha.group(1) != kernel_source_digest():
        return None
    return float(m_b.group(1))


# The pages' own figures for this method, quoted as context only (no hardware,
# precision or workload is given for either on the pages).
PAGE_CONTEXT = {
    "attenio_speedup_over_prior_solutions": {
        "value": "1.6x-8.8x", "hardware": "not stated",
        "source": "I/O Analysis is All You Need: An I/O Analysis for Long-Sequence Attention, abstract"},
    "flashattention_speedup_over_native_pytorch": {
        "value": "about 6x", "hardware": "not stated",
        "source": "Neural Circuit Diagrams abstract"},
}


def committed_counters(w, ms: float):
    """Issue and utilization figures of workload w from the committed
    rocprofv3 summaries, when they were taken on the current kernel source:
    MFMA pipe busy, other VALU instructions per MFMA, the VALU-active fraction
    (which counts MFMA issue too), LDS bank-conflict cycles per LDS-active
    cycle, the clock the kernel ran at, and the HBM bytes of
    the counter summary divided by this run's time."""
    stem = counter_summary_path(w)[:-len("_counters.md")]
    out = {}
    util = stem + "_utilization.md"
    if w.dtype == "bf16" and os.path.exists(util):
        text = open(util).read()
        m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]{16})", text)
        if m_sha and m_sha.group(1) == kernel_source_digest():
            def num(pat):
                m = re.search(pat, text)
                return float(m.group(1)) if m else None
            out["mfma_pipe_busy"] = num(r"MFMA pipe busy: .* = ([0-9.]+)")
            out["valu_per_mfma"] = num(r"other VALU instructions per MFMA: .* = ([0-9.]+)")
            out["valu_active"] = num(r"VALU active \(.*\): .* = ([0-9.]+)")
            conf = re.search(r"LDS bank conflict cycles / LDS active cycles: ([0-9.e+]+) / ([0-9.e+]+)", text)
            out["lds_bank_conflict_rate"] = float(conf.group(1)) / float(conf.group(2)) if conf else None
            out["clock_ghz"] = num(r"clock during the kernel: .* = ([0-9.]+) GHz")
            out["source"] = os.path.relpath(util, ROOT)
    traffic = committed_traffic(w)
    if traffic is not None:
        out["hbm_bytes"] = traffic
        out["achieved_hbm_GBs"] = traffic / (ms * 1e-3) / 1e9
        out["hbm_frac_of_peak"] = out["achieved_hbm_GBs"] / HBM_PEAK_GBS
    return out or None


def copy_calibration(nbytes: int) -> None:
    import torch
    n = nbytes // 4
    src = torch.ones(n, device="cuda:0", dtype=torch.float32)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "launches": 3}), flush=True)


def read_calibration(nbytes: int, repeats: int) -> None:
    """Read one device buffer of nbytes `repeats` times (one reduction kernel
    each).  With nbytes well above the 4 MiB per-XCD L2 and well below the
    256 MiB Infinity Cache, FETCH_SIZE per dispatch tells whether the counter
    sees L2 misses that the Infinity Cache serves (every dispatch reads
    nbytes) or only DRAM reads (the repeats read almost nothing)."""
    import torch
    src = torch.ones(nbytes // 4, device="cuda:0", dtype=torch.float32)
    torch.cuda.synchronize()
    acc = torch.zeros((), device="cuda:0")
    for _ in range(repeats):
        acc += src.sum()
    torch.cuda.synchronize()
    print(json.dumps({"read_calibration_bytes": nbytes, "repeats": repeats, "sum": float(acc)}), flush=True)


def cpu_baseline(w, q, k, v, kv_len, out, budget_s: float):
    """Time the fp64 oracle on a bounded seeded sample of query rows and check
    those rows against the GPU output."""
    import numpy as np
    import torch

    import oracle
    from exact_long_sequence_amd.inputs import oracle_view, sample_rows
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    kl = None if kv_len is None else kv_len.numpy()
    rows = sample_rows(w.B, w.H, w.N, 65536, w.seed, kv_len=kl)
    rng = np.random.default_rng(w.seed + 2)
    rows = rows[rng.permutation(rows.size)]
    qv, kv_, vv = oracle_view(q), oracle_view(k), oracle_view(v)
    kind = "bf16" if w.dtype == "bf16" else "f32"
    L = oracle.effective_kv_len(kl, w.B, w.N)
    done, flops, max_err, sum_err, n_el = 0, 0.0, 0.0, 0.0, 0
    t0 = time.perf_counter()
    # a first small call gives the rate; later calls fill the time budget
    n = 256
    while done < rows.size:
        elapsed = time.perf_counter() - t0
        if done:
            if elapsed >= budget_s:
                break
            rate = done / elapsed
            n = int(min(rows.size - done, max(256.0, 0.95 * (budget_s - elapsed) * rate)))
        r = rows[done:done + n]
        want = oracle.attention_fp64(qv, kv_, vv, w.scale, w.causal, kl, kind=kind, rows=r)
        i = r % w.N
        Lr = L[(r // w.N) // w.H]
        keys = np.minimum(i + 1, Lr) if w.causal else Lr
        flops += 4.0 * w.d * float(keys.sum())
        idx = torch.as_tensor(r, device=out.device, dtype=torch.long)
        got = out.reshape(-1, w.d).index_select(0, idx).float().cpu().numpy().astype(np.float64)
        err = np.abs(got - want)
        max_err = max(max_err, float(err.max()))
        sum_err += float(err.sum())
        n_el += err.size
        done += r.size
    dt = time.perf_counter() - t0
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": blas_threads if blas_threads else cores,
        "kind": "oracle",
        "sample": f"{done} seeded query rows of {w.name} (all keys each row sees), fp64 numpy, "
                  f"{dt:.1f} s on {cores} visible host cores",
        "seconds": dt,
        "rows": int(done),
        "parity_on_sample": {"max_abs_err": max_err, "mean_abs_err": sum_err / max(n_el, 1)},
    }


def bench_bwd(w, args) -> int:
    import torch

    from exact_long_sequence_amd import attnio
    from exact_long_sequence_amd.inputs import workload_inputs
    if w.dtype != "bf16":
        print("the backward is bf16 only", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    q, k, v, kv_len = workload_inputs(w)
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed + 7919)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(torch.bfloat16)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    del q, k, v, do
    kvd = None if kv_len is None else kv_len.to(dev)
    o, lse = attnio.attn_fwd_lse(qd, kd, vd, causal=w.causal, kv_len=kvd, scale=w.scale)
    dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
    ws = torch.empty(attnio.attn_bwd_workspace_bytes(w.B, w.H, w.N), dtype=torch.uint8, device=dev)
    model = attnio.attn_io_model(w.B, w.H, w.N, w.d, 2, w.causal,
                                 None if kv_len is None else kv_len.tolist())

    def step():
        attnio.attn_bwd(qd, kd, vd, o, dod, lse, causal=w.causal, kv_len=kvd, scale=w.scale,
                        dq=dq, dk=dk, dv=dv, workspace=ws)
    for _ in range(args.warmup):
        step()
    stream = torch.cuda.current_stream(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    flops = 10.0 * w.d * model["pairs"]
    tflops = flops / (ms * 1e-3) / 1e12
    # compulsory bytes: Q, K, V, O, dO read and dQ, dK, dV written once, plus
    # the per-row log-sum-exp
    t_min = 8.0 * w.B * w.H * w.N * w.d * 2 + 4.0 * w.B * w.H * w.N
    result = {
        "metric": "attention bwd TFLOP/s (algorithmic 10*d per visible query-key pair)",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V/dO)",
        "config": {**w.describe(), "pass": "backward"},
        "roofline": {
            "bound": "mfma",
            "achieved": tflops,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
            "traffic": None,
        },
        "io": {"t_min_bytes": t_min, "t_min_rate_GBs": t_min / (ms * 1e-3) / 1e9},
        "executed_flops_per_pair": 14 * w.d,
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_unfused(w, args) -> int:
    """The operator-centric baseline: three kernels per group of heads with the
    N x N scores and probabilities in HBM.  Same algorithmic FLOPs as the fused
    forward, so the two TFLOP/s figures compare directly; the fused kernel is
    timed in the same process for the ratio."""
    import torch

    from exact_long_sequence_amd import attnio
    from exact_long_sequence_amd.inputs import workload_inputs
    if w.dtype != "bf16":
        print("the unfused baseline is bf16 only", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    q, k, v, kv_len = workload_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    kvd = None if kv_len is None else kv_len.to(dev)
    out = torch.empty_like(qd)
    hp = max(1, min(args.heads_per_pass, w.B * w.H))
    ws = torch.empty(hp * attnio.attn_fwd_unfused_workspace_bytes(w.N), dtype=torch.uint8, device=dev)
    model = attnio.attn_io_model(w.B, w.H, w.N, w.d, 2, w.causal,
                                 None if kv_len is None else kv_len.tolist())
    stream = torch.cuda.current_stream(dev)

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(steps):
            fn()
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps

    ms = timed(lambda: attnio.attn_fwd_unfused(qd, kd, vd, causal=w.causal, kv_len=kvd, scale=w.scale,
                                               out=out, workspace=ws), args.steps, args.warmup)
    ms_fused = timed(lambda: attnio.attn_fwd(qd, kd, vd, causal=w.causal, kv_len=kvd, scale=w.scale,
                                             out=out), max(args.steps, 5), 2)
    tflops = model["flops"] / (ms * 1e-3) / 1e12
    traffic = None
    summary = os.path.join(ROOT, "profiles", "attn_fwd_unfused_bf16_causal_b1_h32_n32k_d128_trace_counters.md")
    if w.name == "bf16_causal_h32_n32k_d128" and hp == 8 and os.path.exists(summary):
        text = open(summary).read()
        src = os.path.join(ROOT, "exact_long_sequence_amd", "csrc", "attn_unfused_bf16.hip")
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]{16})", text)
        m_b = re.search(r"hbm_bytes_per_call:\s*([0-9.eE+]+)", text)
        if m_sha and m_b and m_sha.group(1) == digest:
            traffic = float(m_b.group(1))
    nn = float(w.N) * w.N * w.B * w.H
    # intermediates written and read once each: S (fp32) and P (bf16)
    inter = nn * (4 + 4 + 2 + 2)
    result = {
        "metric": "attention fwd TFLOP/s, operator-centric baseline (algorithmic 4*d per visible pair)",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V)",
        "config": {**w.describe(), "pass": "forward, unfused", "heads_per_pass": hp},
        "roofline": {
            "bound": "hbm",
            "achieved": (model["t_min"] + inter) / (ms * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": (model["t_min"] + inter) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": traffic,
        },
        "io": {"t_min_bytes": model["t_min"], "intermediate_bytes_min": inter},
        "fused_ms_per_step": ms_fused,
        "fused_speedup": ms / ms_fused,
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_rows(args) -> int:
    """A streaming row operator (softmax or LayerNorm) over a bf16 [R, N]
    matrix: HBM-bound, so the roofline is HBM bandwidth and the figure is the
    compulsory bytes (read x once, write y once, plus gamma and beta) per
    second."""
    import numpy as np
    import torch

    import oracle
    from exact_long_sequence_amd import attnio
    from exact_long_sequence_amd.inputs import ROW_WORKLOADS, oracle_view, row_workload_inputs
    name = args.workload if args.workload in ROW_WORKLOADS else "softmax_r32k_n32k"
    w = ROW_WORKLOADS[name]
    dev = torch.device("cuda:0")
    x, gamma, beta = row_workload_inputs(w)
    xd = x.to(dev)
    y = torch.empty_like(xd)
    gd = None if gamma is None else gamma.to(dev)
    bd = None if beta is None else beta.to(dev)
    if w.op == "softmax":
        fn = lambda: attnio.stream_softmax(xd, w.param, out=y)  # noqa: E731
    else:
        fn = lambda: attnio.stream_layernorm(xd, gd, bd, eps=w.param, out=y)  # noqa: E731
    for _ in range(args.warmup):
        fn()
    stream = torch.cuda.current_stream(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    t_min = 2.0 * w.R * w.N * 2 + (0 if gamma is None else 2 * w.N * 2)
    gbs = t_min / (ms * 1e-3) / 1e9
    # a plain device copy of the same bytes, for the achievable bandwidth
    for _ in range(2):
        y.copy_(xd)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        y.copy_(xd)
    stop.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2.0 * w.R * w.N * 2 / (start.elapsed_time(stop) / args.steps * 1e-3) / 1e9
    result = {
        "metric": f"stream_{w.op} GB/s (compulsory bytes: x read once, y written once)",
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) rows)",
        "config": w.describe(),
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None},
        "cached_in_registers": attnio.stream_rows_cached(w.N),
        "plain_copy_GBs": copy_gbs,
    }
    if not args.no_cpu_baseline:
        # the oracle on a bounded sample of rows, timed on the host cores
        rng = np.random.default_rng(w.seed + 5)
        rows = rng.permutation(w.R)
        t0 = time.perf_counter()
        done = 0
        while done < w.R and time.perf_counter() - t0 < args.cpu_budget:
            r = rows[done:done + 64]
            xs = oracle_view(x[torch.as_tensor(r)])
            if w.op == "softmax":
                oracle.softmax_rows_fp64(xs, w.param)
            else:
                oracle.layernorm_rows_fp64(xs, oracle_view(gamma), oracle_view(beta), eps=w.param)
            done += r.size
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": 2.0 * done * w.N * 2 / dt / 1e9, "unit": "GB/s",
            "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{done} seeded rows of {w.name}, fp64 numpy, {dt:.1f} s"}
    print(json.dumps(result), flush=True)
    return 0


def bench_fp8(w, args) -> int:
    """The fp8 (E4M3) forward on the workload's shape: same seeded draws,
    quantized per tensor with power-of-two descales; bf16 output.  Same
    algorithmic FLOPs as the bf16 forward; roofline = the fp8 matrix peak."""
    import numpy as np
    import torch

    import oracle
    from exact_long_sequence_amd import attnio
    from exact_long_sequence_amd.inputs import make_fp8_inputs, sample_rows
    FP8_PEAK = 5000.0
    dev = torch.device("cuda:0")
    q8, k8, v8, ds, kv_len = make_fp8_inputs(w.B, w.H, w.N, w.d, w.seed, w.padded, w.q_mul)
    qd, kd, vd = q8.to(dev), k8.to(dev), v8.to(dev)
    kvd = None if kv_len is None else kv_len.to(dev)
    out = torch.empty(q8.shape, dtype=torch.bfloat16, device=dev)
    # FLOPs do not depend on the element size; the model takes 2- or 4-byte elements
    model = attnio.attn_io_model(w.B, w.H, w.N, w.d, 2, w.causal,
                                 None if kv_len is None else kv_len.tolist())
    fn = lambda: attnio.attn_fwd_fp8(qd, kd, vd, ds, causal=w.causal, kv_len=kvd, scale=w.scale,  # noqa: E731
                                     out=out)
    for _ in range(args.warmup):
        fn()
    stream = torch.cuda.current_stream(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    tflops = model["flops"] / (ms * 1e-3) / 1e12
    result = {
        "metric": "attention fwd TFLOP/s, fp8 E4M3 inputs (algorithmic 4*d per visible pair)",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 (fp32 accumulation, bf16 output)",
        "data": "synthetic (seeded N(0,1) Q/K/V quantized per tensor)",
        "config": {**w.describe(), "dtype": "fp8-e4m3", "descale": list(ds)},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": FP8_PEAK, "unit": "TFLOP/s",
                     "frac": tflops / FP8_PEAK, "traffic": None},
    }
    if not args.no_cpu_baseline:
        rows = sample_rows(w.B, w.H, w.N, 256, w.seed)
        t0 = time.perf_counter()
        want = oracle.attention_fp8_fp64(q8.numpy(), k8.numpy(), v8.numpy(), ds, w.scale, w.causal,
                                         None if kv_len is None else kv_len.numpy(), rows=rows)
        dt = time.perf_counter() - t0
        L = oracle.effective_kv_len(None if kv_len is None else kv_len.numpy(), w.B, w.N)
        i = rows % w.N
        Lr = L[(rows // w.N) // w.H]
        keys = np.minimum(i + 1, Lr) if w.causal else Lr
        got = out.reshape(-1, w.d).index_select(0, torch.as_tensor(rows, device=dev)).float().cpu().numpy()
        result["cpu_baseline"] = {
            "value": 4.0 * w.d * float(keys.sum()) / dt / 1e12, "unit": "TFLOP/s",
            "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{rows.size} seeded query rows (fp8 decode of the whole tensors included), {dt:.1f} s",
            "parity_on_sample": {"max_abs_err": float(np.abs(got - want).max())}}
    print(json.dumps(result), flush=True)
    return 0


def bench_tilings(args) -> int:
    """Every compiled bf16 forward tiling of the workload's head size, timed
    interleaved on the same GPU (median of args.reps rounds of args.steps
    launches each), next to the I/O model's choice and predicted cost.  One
    JSON line per workload."""
    import torch

    from exact_long_sequence_amd import attnio
    from exact_long_sequence_amd.inputs import WORKLOADS, workload_inputs
    names = args.workload.split(",")
    if args.all_workloads:
        names = [n for n, w in WORKLOADS.items() if w.dtype == "bf16"]
    dev = torch.device("cuda:0")
    for name in names:
        w = WORKLOADS[name]
        q, k, v, kv_len = workload_inputs(w)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        kvd = None if kv_len is None else kv_len.to(dev)
        out = torch.empty_like(qd)
        model = attnio.attn_io_model(w.B, w.H, w.N, w.d, 2, w.causal,
                                     None if kv_len is None else kv_len.tolist())
        ranking = attnio.attn_tiling_enumerate(w.d, w.causal)
        rank_of = {e["compiled"]: r for r, e in enumerate(ranking) if e["compiled"] >= 0}
        pick = next(e["compiled"] for e in ranking if e["compiled"] >= 0)
        idx = [i for i in range(attnio.attn_tiling_count()) if attnio.attn_tiling_get(i)["d"] == w.d]
        for i in idx:
            for _ in range(args.warmup):
                attnio.attn_fwd_tiled(qd, kd, vd, i, causal=w.causal, kv_len=kvd, scale=w.scale, out=out)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream(dev)
        times = {i: [] for i in idx}
        for _ in range(args.reps):
            for i in idx:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(args.steps):
                    attnio.attn_fwd_tiled(qd, kd, vd, i, causal=w.causal, kv_len=kvd, scale=w.scale, out=out)
                e1.record(stream)
                torch.cuda.synchronize()
                times[i].append(e0.elapsed_time(e1) / args.steps)
        rows = []
        for i in idx:
            ms = sorted(times[i])[len(times[i]) // 2]
            ev = ranking[rank_of[i]]
            rows.append({"tiling": i, **attnio.attn_tiling_get(i), "model_rank": rank_of[i],
                         "model_cycles_per_pair": ev["cycles_per_pair"], "ms_median": ms,
                         "ms_all": times[i], "tflops": model["flops"] / (ms * 1e-3) / 1e12})
        best = min(rows, key=lambda r: r["ms_median"])["tiling"]
        print(json.dumps({"mode": "tilings", "workload": name, "model_pick": pick, "measured_best": best,
                          "steps": args.steps, "reps": args.reps, "results": rows}), flush=True)
        del qd, kd, vd, out
        torch.cuda.empty_cache()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--copy-calib", type=int, default=0, help="run a plain copy of this many bytes")
    ap.add_argument("--read-calib", type=int, default=0,
                    help="read a device buffer of this many bytes --read-repeats times")
    ap.add_argument("--read-repeats", type=int, default=8)
    ap.add_argument("--mode", choices=("fwd", "bwd", "unfused", "rows", "fp8", "tilings"), default="fwd")
    ap.add_argument("--reps", type=int, default=4, help="--mode tilings: interleaved rounds per tiling")
    ap.add_argument("--all-workloads", action="store_true", help="--mode tilings: every bf16 workload")
    ap.add_argument("--tiling", type=int, default=-1,
                    help="--mode fwd: run this compiled tiling (attn_tiling_get index) instead of the model's")
    ap.add_argument("--heads-per-pass", type=int, default=8,
                    help="--mode unfused: heads whose N x N intermediates share the workspace")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: every box of this setup has a single MI355X and the "
              "attention path here is the single-GPU share; run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    if args.copy_calib:
        copy_calibration(args.copy_calib)
        return 0
    if args.read_calib:
        read_calibration(args.read_calib, args.read_repeats)
        return 0

    from exact_long_sequence_amd import attnio
    from exact_long_sequence_amd.inputs import WORKLOADS, workload_inputs

    if args.mode == "rows":
        return bench_rows(args)
    if args.mode == "tilings":
        return bench_tilings(args)
    w = WORKLOADS[args.workload]
    if args.mode == "bwd":
        return bench_bwd(w, args)
    if args.mode == "unfused":
        return bench_unfused(w, args)
    if args.mode == "fp8":
        return bench_fp8(w, args)
    dev = torch.device("cuda:0")
    q, k, v, kv_len = workload_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    kvd = None if kv_len is None else kv_len.to(dev)
    out = torch.empty_like(qd)
    fn = attnio.attn_fwd if w.dtype == "bf16" else attnio.attn_fwd_f32
    if args.tiling >= 0:
        if w.dtype != "bf16":
            print("--tiling selects a bf16 tiling", file=sys.stderr)
            return 2
        fn = lambda q_, k_, v_, **kw: attnio.attn_fwd_tiled(q_, k_, v_, args.tiling, **kw)  # noqa: E731
    model = attnio.attn_io_model(w.B, w.H, w.N, w.d, 2 if w.dtype == "bf16" else 4, w.causal,
                                 None if kv_len is None else kv_len.tolist())
    if w.dtype == "bf16":
        ranking = attnio.attn_tiling_enumerate(w.d, w.causal)
        chosen = args.tiling if args.tiling >= 0 else next(e["compiled"] for e in ranking if e["compiled"] >= 0)
        tiling = {**attnio.attn_tiling_get(chosen), "index": chosen,
                  "model_pick": next(e["compiled"] for e in ranking if e["compiled"] >= 0)}
    else:
        tiling = attnio.attn_query_tiling(w.d, w.causal, "f32")

    for _ in range(args.warmup):
        fn(qd, kd, vd, causal=w.causal, kv_len=kvd, scale=w.scale, out=out)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        fn(qd, kd, vd, causal=w.causal, kv_len=kvd, scale=w.scale, out=out)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms = total_ms / args.steps

    flops = model["flops"]
    tflops = flops / (ms * 1e-3) / 1e12
    peak = MFMA_BF16_PEAK_TFLOPS if w.dtype == "bf16" else 157.3
    traffic = committed_traffic(w)
    result = {
        "metric": "attention fwd TFLOP/s (algorithmic 4*d per visible query-key pair)",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V)",
        "config": w.describe(),
        "roofline": {
            "bound": "mfma",
            "achieved": tflops,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": tflops / peak,
            "traffic": traffic,
        },
        "io": {
            "t_min_bytes": model["t_min"],
            "t_l2_model_bytes": model["t_l2"],
            "t_lds_model_bytes": model["t_lds"],
            "traffic_over_t_min": None if traffic is None else traffic / model["t_min"],
            "t_min_rate_GBs": model["t_min"] / (ms * 1e-3) / 1e9,
            "hbm_peak_GBs": HBM_PEAK_GBS,
        },
        "tiling": tiling,
        "counters": committed_counters(w, ms),
        "context": PAGE_CONTEXT,
        "kernel_source_sha256_16": kernel_source_digest(),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, kv_len, out, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
