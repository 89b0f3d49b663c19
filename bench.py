#!/usr/bin/env python3
"""Throughput of the strided, batched fp32 product on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the workload's entry point (validation, planning and
the kernel launch) over its inputs, which are resident in device memory
before timing starts.  W untimed steps, then exactly K timed steps bracketed
by device synchronisation; rank 0 prints one JSON line.  Without --warmup, W
is as many steps as fill 0.3 s (at least 5), so that the clock has ramped up
before a short kernel is timed; the line reports the W used.

Default workload: the large square product, 4 x 4096^3 with A read
transposed, alpha 0.5 and accumulation into C.  `--workload all` prints one
line per workload instead (for tables; not the headline).

The JSON line carries:
  value      whole-job TFLOP/s (2*m*n*k*batch per step, K steps / wall time)
  roofline   the dominant (only) kernel: algorithmic FLOPs per launch divided
             by its mean launch duration from HIP events recorded on the
             launch stream, against the MI355X dense fp32 matrix peak
             (157.3 TFLOP/s) -- or, for a workload below the machine balance
             (fewer than ~19.7 flops per algorithmic byte, e.g. skinny_xWt),
             its algorithmic bytes per launch against the HBM peak
             (8000 GB/s); `traffic` (HBM bytes per launch) and
             `mfma_busy` (matrix-core busy fraction) come from the committed
             rocprofv3 counter record when it was taken on the current
             library sources, else null; `achieved_tb_per_s` is the
             algorithmic bytes per launch over the same mean duration
  cpu_baseline  the CPU oracle timed on a bounded slice of the same workload
             (a block of rows of batch 0), as TFLOP/s, with its thread count,
             the host's logical CPUs and the CPUs the process may use
  configs    (default run only) the other configurations of the workload
             set, each timed in the same process after the headline: the
             64^3 product, the linear layer, attention's Q K^T and P V, and
             the spectrogram -- mean launch time, TFLOP/s, fraction of the
             fp32 matrix peak, kernel, and the oracle on a slice of each.
             Their kernels are timed back to back (1 s warm-up each), and
             the oracle slices run after the last of them.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP32_MATRIX_TFLOPS = 157.3   # MI355X dense fp32 matrix peak
PEAK_HBM_GBPS = 8000.0            # MI355X HBM3E peak bandwidth
WARMUP_SECONDS = 0.3              # default warm-up: the clock ramps up within it
CONFIG_WARMUP_SECONDS = 1.0       # the configurations' short kernels: a longer ramp, measured steadier
METRIC = "fp32 batched strided GEMM TFLOP/s and % of MI355X fp32 matrix peak"
DEFAULT_WORKLOAD = "square4096_acc"
# The other configurations of the method's workload set, timed beside the
# headline in the default run: the 64^3 product, the linear layer x W^T, the
# attention scores Q K^T and the product P V, and the spectrogram.
CONFIG_WORKLOADS = (("1", "square64"), ("2", "linear_xWt"), ("3a", "attn_qk"), ("3b", "attn_pv"),
                    ("4", "spectrogram"))
# Workloads beyond the method's set, timed after it in the default run (no
# oracle slice): fused attention plain and causal, the skinny product, the
# split-k weight gradient and the split-KV decode step.
EXTRA_WORKLOADS = ("attn_fused", "attn_fused_causal", "skinny_xWt", "linear_dw_deep", "attn_decode")
CONFIG_CPU_SECONDS = 1.5          # oracle slice per configuration (the headline's is --cpu-seconds)
CONFIG_STEPS = 100                # timed launches per configuration


def kernel_sources() -> list:
    """Every source the library is built from (kernels, planner, ABI and
    the public header), in a fixed order."""
    csrc = os.path.join(ROOT, "strided_fp32_gemm_amd", "csrc")
    files = sorted(os.path.join("strided_fp32_gemm_amd", "csrc", f) for f in os.listdir(csrc)
                   if f.endswith((".hip", ".hpp", ".cpp", ".h")))
    inc = os.path.join(ROOT, "include")
    files += sorted(os.path.join("include", f) for f in os.listdir(inc) if f.endswith(".h"))
    return files


def kernel_sources_sha256() -> str:
    h = hashlib.sha256()
    for rel in kernel_sources():
        h.update(rel.encode())
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_record(workload: str, kernel: str) -> dict:
    """HBM bytes per launch and the matrix-core busy fraction from the
    committed counter summary of this kernel and workload, if it was taken
    on the current library sources (else an empty dict)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return {}
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, _, val = line.partition(":")
                rec[key.strip("-* `").strip()] = val.strip().strip("`")
    if rec.get("kernel_sources_sha256") != kernel_sources_sha256():
        return {}
    out = {}
    for key, name in (("hbm_bytes_per_launch", "traffic"), ("mfma_busy", "mfma_busy")):
        try:
            out[name] = float(rec[key])
        except (KeyError, ValueError):
            pass
    return out


def cpu_model() -> str:
    """The host CPU's model name (Linux), for the baseline's record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores(threads: int) -> dict:
    """What the oracle ran on: its OpenMP thread count, the host's logical
    CPUs and the CPUs this process may use."""
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cores": threads, "omp_max_threads": threads, "host_cpus": os.cpu_count(),
            "usable_cpus": usable, "cpu_model": cpu_model()}


def cpu_baseline_attention(p, seconds: float) -> dict:
    """The oracle's attention on the first H (sequence, head) pairs of the
    same call (whole heads, every query row), H chosen so the run takes
    roughly `seconds`."""
    import oracle
    threads = oracle.num_threads()
    out = p.O.storage.copy()
    (ko, ki, kr, kc) = p.K.strides

    def run(heads):
        no, ni = (1, heads) if heads <= p.nb_inner else (heads // p.nb_inner, p.nb_inner)
        t0 = time.perf_counter()
        oracle.ref_attention(no, ni, p.tq, p.tk, p.d, p.alpha, p.causal, p.Q.storage, *p.Q.strides,
                             p.K.storage, ko, ki, p.g, kr, kc, p.V.storage, *p.V.strides,
                             out, *p.O.strides)
        return no * ni, time.perf_counter() - t0

    total = p.nb_outer * p.nb_inner
    heads, t = run(1)
    while t < seconds / 8 and heads < total:
        heads, t = run(min(total, heads * 4) if heads * 4 <= p.nb_inner
                       else min(total, max(p.nb_inner, heads * 4) // p.nb_inner * p.nb_inner))
    reps = 1
    if heads == total and t < seconds / 4:
        # The whole call is quick (a decode step): repeat it to fill the time.
        reps = max(2, int(seconds / 2 / max(t, 1e-6)))
        t = sum(run(heads)[1] for _ in range(reps))
    flops = 4.0 * p.d * p.visible_pairs * heads * reps
    sample = f"all {p.tq} query rows of the first {heads} (sequence, head) pairs"
    if reps > 1:
        sample = f"the whole call ({heads} (sequence, head) pairs) x {reps} repetitions"
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", **host_cores(threads), "kind": "oracle",
            "sample": f"{sample} ({flops / 1e9:.2f} GFLOP in {t:.1f} s)"}


def cpu_baseline(p, seconds: float) -> dict:
    """The oracle on rows 0..R-1 of batch 0 of the same product, R chosen so
    the run takes roughly `seconds`."""
    import oracle
    from strided_fp32_gemm_amd import workloads as wl
    if wl.kind(p.name) in ("attention", "attention_splitkv"):
        return cpu_baseline_attention(p, seconds)
    threads = oracle.num_threads()
    kind = wl.kind(p.name)
    out = (p.D if kind == "dist" else p.C).storage.copy()

    def run(rows):
        t0 = time.perf_counter()
        if kind == "dist":
            oracle.ref_sqdist(1, rows, p.n, p.k, p.X.storage, (0,) + tuple(p.X.strides[1:]),
                              p.Y.storage, (0,) + tuple(p.Y.strides[1:]), out,
                              (0,) + tuple(p.D.strides[1:]))
        elif kind == "batched2":
            # Entry (outer 0, inner 0) starts at each storage's first element.
            oracle.ref_sgemm(1, rows, p.n, p.k, p.alpha,
                             p.A.storage, 0, p.A.strides[2], p.A.strides[3],
                             p.B.storage, 0, p.B.strides[2], p.B.strides[3],
                             int(p.accumulate), out, 0, p.C.strides[2], p.C.strides[3])
        elif kind == "ex":
            sv = lambda v: (0, v.strides[1]) if v is not None else (0, 0)
            oracle.ref_sgemm_ex(1, rows, p.n, p.k, p.alpha, p.A.storage, (0, p.A.s_row, p.A.s_col),
                                p.B.storage, (0, p.B.s_row, p.B.s_col), p.beta_value, out,
                                (0, p.C.s_row, p.C.s_col),
                                row_add=p.row.storage if p.row is not None else None, sR=sv(p.row),
                                col_add=p.col.storage if p.col is not None else None, sL=sv(p.col))
        else:
            oracle.ref_sgemm(1, rows, p.n, p.k, p.alpha,
                             p.A.storage, 0, p.A.s_row, p.A.s_col,
                             p.B.storage, 0, p.B.s_row, p.B.s_col,
                             int(p.accumulate), out, 0, p.C.s_row, p.C.s_col)
        return time.perf_counter() - t0

    def run_entries(nb):
        """The first nb whole batch entries of the call (plain products)."""
        t0 = time.perf_counter()
        oracle.ref_sgemm(nb, p.m, p.n, p.k, p.alpha, p.A.storage, *p.A.strides, p.B.storage, *p.B.strides,
                         int(p.accumulate), out, *p.C.strides)
        return time.perf_counter() - t0

    rows = min(p.m, threads)
    t = run(rows)
    while t < min(0.5, seconds / 4) and rows < p.m:
        rows = min(p.m, rows * 4)
        t = run(rows)
    if t < seconds and rows < p.m:
        rows = min(p.m, max(rows, int(rows * seconds / max(t, 1e-6)) // threads * threads))
        t = run(rows)
    flops = 2.0 * rows * p.n * p.k
    sample = f"rows 0..{rows - 1} of batch 0 ({rows}x{p.n}x{p.k}"
    if rows == p.m and t < seconds / 2:
        # Small products: whole batch entries, then the whole call repeated.
        nb, reps = 1, 1
        if kind == "plain" and p.batch > 1:
            nb = min(p.batch, max(1, int(seconds / max(t, 1e-6))))
            t = run_entries(nb)
        for _ in range(3):
            if t >= seconds / 2:
                break
            reps = max(reps + 1, int(reps * seconds / max(t, 1e-6)))
            t = sum(run_entries(nb) if kind == "plain" else run(rows) for _ in range(reps))
        flops = 2.0 * rows * p.n * p.k * nb * reps
        sample = f"batch entries 0..{nb - 1} ({nb} x {p.m}x{p.n}x{p.k}) x {reps} repetitions"
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", **host_cores(threads), "kind": "oracle",
            "sample": f"{sample}, {flops / 1e9:.2f} GFLOP in {t:.2f} s)" if sample.startswith("rows")
            else f"{sample} ({flops / 1e9:.2f} GFLOP in {t:.2f} s)"}


def _step_fn(p, dev, stream):
    """Device copies of the workload's inputs and one step of it (the call
    the benchmark times), plus the plan that step launches."""
    import torch
    import strided_fp32_gemm_amd as sg
    from strided_fp32_gemm_amd import workloads as wl

    kind = wl.kind(p.name)
    if kind == "dist":
        dX, dY = torch.from_numpy(p.X.storage).to(dev), torch.from_numpy(p.Y.storage).to(dev)
        dD = torch.from_numpy(p.D.storage).to(dev)
        ws = torch.empty(p.workspace_floats, device=dev)
        args = p.call_args(dX, dY, dD, ws)
        sX, sY = p.X.strides, p.Y.strides
        info = sg.sgemm_plan_describe(p.batch, p.m, p.n, p.k, -2.0, dX.data_ptr(), *sX, dY.data_ptr(),
                                      sY[0], sY[2], sY[1], 0, dD.data_ptr(), *p.D.strides, num_cus=0)
        info["kernel"] += "_vec (after 2 sqnorms launches)"
        return (lambda: sg.sgemm_pairwise_sqdist(*args, stream=stream)), info, (dX, dY, dD, ws)
    if kind == "attention":
        dq, dk, dv, do = (torch.from_numpy(x.storage).to(dev) for x in (p.Q, p.K, p.V, p.O))
        args = p.call_args(dq, dk, dv, do)
        info = sg.sgemm_attention_describe(*p.call_args(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                                        do.data_ptr()))
        return (lambda: sg.sgemm_attention(*args, stream=stream)), info, (dq, dk, dv, do)
    if kind == "attention_splitkv":
        dq, dk, dv, do = (torch.from_numpy(x.storage).to(dev) for x in (p.Q, p.K, p.V, p.O))
        args = p.call_args(dq, dk, dv, do)
        plan = sg.sgemm_attention_splitkv_describe(*p.call_args(dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                                                do.data_ptr()), num_cus=0)
        floats = plan["workspace_floats"]
        W = torch.empty(max(floats, 1), device=dev)
        info = {"kernel": f"attn_splitkv_d64 (keys in {plan['chunks']} chunks of {plan['chunk_keys']}, then the"
                          f" merge: 2 launches per step)", "workgroups": None}
        return (lambda: sg.sgemm_attention_splitkv(*args, W, floats, stream=stream)), info, (dq, dk, dv, do, W)
    dA, dB = torch.from_numpy(p.A.storage).to(dev), torch.from_numpy(p.B.storage).to(dev)
    dC = torch.from_numpy(p.C.storage).to(dev)
    if kind == "batched2":
        args = p.call_args(dA, dB, dC)
        info = sg.sgemm_plan_describe2(*p.call_args(dA.data_ptr(), dB.data_ptr(), dC.data_ptr()),
                                       num_cus=0)
        return (lambda: sg.sgemm_strided_batched2(*args, stream=stream)), info, (dA, dB, dC)
    if kind == "splitk":
        plan = sg.sgemm_splitk_describe(*p.call_args(dA.data_ptr(), dB.data_ptr(), dC.data_ptr()), num_cus=0)
        W = torch.empty(max(plan["workspace_floats"], 1), device=dev)
        args = p.call_args(dA, dB, dC)
        floats = plan["workspace_floats"]
        info = plan["parts"]
        if plan["splits"] > 1:
            info["kernel"] += (f" (k in {plan['splits']} partitions of {plan['kc']}, then the reduction:"
                               f" {plan['launches']} launches per step)")
        return (lambda: sg.sgemm_strided_batched_splitk(*args, W, floats, stream=stream)), info, (dA, dB, dC, W)
    info = sg.sgemm_plan_describe(*p.call_args(dA.data_ptr(), dB.data_ptr(), dC.data_ptr()), num_cus=0)
    if kind == "ex":
        dr = torch.from_numpy(p.row.storage).to(dev) if p.row is not None else None
        dl = torch.from_numpy(p.col.storage).to(dev) if p.col is not None else None
        args = p.ex_call_args(dA, dB, dC, dr, dl)
        info["kernel"] += "_vec"
        return (lambda: sg.sgemm_strided_batched_ex(*args, stream=stream)), info, (dA, dB, dC, dr, dl)
    args = p.call_args(dA, dB, dC)
    return (lambda: sg.sgemm_strided_batched(*args, stream=stream)), info, (dA, dB, dC)


def measure(name: str, steps: int, warmup, warmup_seconds: float = WARMUP_SECONDS):
    """Time `steps` launches of one workload (inputs resident in device
    memory); returns the problem, its plan, the wall time of the timed region,
    the mean launch time from one HIP event pair on the launch stream around
    the timed launches, single-launch times from an untimed pass, and the
    warm-up step count used."""
    import torch
    from strided_fp32_gemm_amd import workloads as wl

    p = wl.workload(name)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    step, info, keep = _step_fn(p, dev, stream)
    if warmup is None:
        # Warm up for warmup_seconds of device time (at least 5 steps).
        warmup = 0
        t_warm = time.perf_counter()
        while warmup < 5 or time.perf_counter() - t_warm < warmup_seconds:
            for _ in range(5):
                step()
            warmup += 5
            torch.cuda.synchronize(dev)
    else:
        for _ in range(warmup):
            step()
    torch.cuda.synchronize(dev)

    # Timed region: K steps back to back, one pair of HIP events on the launch
    # stream around all of them (the mean launch duration is their span / K;
    # an event pair per launch would add its own timestamp work to each).
    first = torch.cuda.Event(enable_timing=True)
    last = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    first.record(stream)
    for _ in range(steps):
        step()
    last.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    mean_ms = first.elapsed_time(last) / steps

    # Spread of single launches, from an untimed pass with an event pair each.
    probes = min(steps, 50)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(probes)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(probes)]
    for i in range(probes):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize(dev)
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    del keep
    torch.cuda.empty_cache()
    return p, info, wall, mean_ms, launch_ms, warmup


def config_entry(label: str, name: str) -> dict:
    """One configuration of the workload set: its kernel's mean launch time
    and rate against the fp32 matrix peak (the oracle is timed afterwards,
    once every configuration's kernel has been timed)."""
    from strided_fp32_gemm_amd import workloads as wl

    p, info, _, mean_ms, launch_ms, warmup = measure(name, CONFIG_STEPS, None, CONFIG_WARMUP_SECONDS)
    flops = float(p.flops)
    achieved = flops / (mean_ms * 1e-3) / 1e12
    alg_bytes = wl.algorithmic_bytes(p)
    e = {"config": label, "workload": name, "kernel": info["kernel"], "workgroups": info["workgroups"],
         "batch": p.batch, "m": p.m, "n": p.n, "k": p.k, "flops_per_launch": flops,
         "steps": CONFIG_STEPS, "warmup": warmup,
         "launch_ms_mean": round(mean_ms, 5), "launch_ms_median": round(statistics.median(launch_ms), 5),
         "launch_ms_min": round(min(launch_ms), 5),
         "tflops": round(achieved, 3), "frac": round(achieved / PEAK_FP32_MATRIX_TFLOPS, 4),
         "algorithmic_bytes": alg_bytes,
         "achieved_tb_per_s": round(alg_bytes / (mean_ms * 1e-3) / 1e12, 3)}
    return e


def extra_entry(name: str) -> dict:
    """A workload beyond the method's set: its step's mean time (every launch
    of the step) against the roof its arithmetic intensity sets."""
    from strided_fp32_gemm_amd import workloads as wl

    p, info, _, mean_ms, _, warmup = measure(name, CONFIG_STEPS, None, CONFIG_WARMUP_SECONDS)
    flops = float(p.flops)
    e = {"config": "extra", "workload": name, "kernel": info["kernel"], "steps": CONFIG_STEPS, "warmup": warmup,
         "launch_ms_mean": round(mean_ms, 5), "tflops": round(flops / (mean_ms * 1e-3) / 1e12, 3)}
    e["roofline"] = _roofline_bound(flops, wl.algorithmic_bytes(p), mean_ms)
    return e


def bench_one(name: str, steps: int, warmup, cpu_seconds: float) -> dict:
    from strided_fp32_gemm_amd import workloads as wl

    p, info, wall, mean_ms, launch_ms, warmup = measure(name, steps, warmup)
    flops = float(p.flops)
    value = flops * steps / wall / 1e12
    counters = counter_record(name, info["kernel"])
    alg_bytes = wl.algorithmic_bytes(p)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall * 1e3 / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": _config(p, info),
        "frac_of_peak": round(value / PEAK_FP32_MATRIX_TFLOPS, 4),
        "roofline": {
            **_roofline_bound(flops, alg_bytes, mean_ms),
            "traffic": counters.get("traffic"),
            "mfma_busy": counters.get("mfma_busy"),
            "algorithmic_bytes": alg_bytes,
            "achieved_tb_per_s": round(alg_bytes / (mean_ms * 1e-3) / 1e12, 3),
            "kernel": info["kernel"],
            "launch_ms_mean": round(mean_ms, 5),
            "launch_ms_median": round(statistics.median(launch_ms), 5),
            "launch_ms_min": round(min(launch_ms), 5),
        },
    }
    if cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(p, cpu_seconds)
    return line


def _roofline_bound(flops: float, alg_bytes: int, mean_ms: float) -> dict:
    """The roof one launch is held to: matrix-core throughput when the
    workload's arithmetic intensity (flops per algorithmic byte) reaches the
    machine balance (peak flops / peak HBM bandwidth, ~19.7 flop per byte),
    HBM bandwidth below it."""
    if flops / alg_bytes >= PEAK_FP32_MATRIX_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9):
        achieved = flops / (mean_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_FP32_MATRIX_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_MATRIX_TFLOPS, 4)}
    achieved = alg_bytes / (mean_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4)}


def _config(p, info) -> dict:
    from strided_fp32_gemm_amd import workloads as wl

    if wl.kind(p.name) in ("attention", "attention_splitkv"):
        return {"workload": p.name, "op": "softmax(alpha Q K^T) V, fused", "nb_outer": p.nb_outer,
                "nb_inner": p.nb_inner, "tq": p.tq, "tk": p.tk, "d": p.d, "g": p.g, "alpha": p.alpha,
                "causal": bool(p.causal),
                "strides": {"Q": list(p.Q.strides), "K": list(p.K.strides), "V": list(p.V.strides),
                            "O": list(p.O.strides)},
                "flops_per_step": p.flops, "kernel": info["kernel"], "workgroups": info["workgroups"]}
    c = {"workload": p.name, "batch": p.batch, "m": p.m, "n": p.n, "k": p.k}
    if wl.kind(p.name) == "batched2":
        c.update({"nb_outer": p.nb_outer, "nb_inner": p.nb_inner, "gA": p.A.group, "gB": p.B.group,
                  "alpha": p.alpha, "accumulate": bool(p.accumulate),
                  "strides": {"A": list(p.A.strides), "B": list(p.B.strides), "C": list(p.C.strides)}})
    elif wl.kind(p.name) == "dist":
        c["op"] = "squared distances |x_i - y_j|^2 (sqnorms x2 + product, alpha -2, row/col terms)"
        c["strides"] = {"X": list(p.X.strides), "Y": list(p.Y.strides), "D": list(p.D.strides)}
    else:
        c["alpha"] = p.alpha
        c["accumulate"] = bool(p.accumulate)
        c["strides"] = {"A": list(p.A.strides), "B": list(p.B.strides), "C": list(p.C.strides)}
        if p.is_ex:
            c["beta"] = p.beta_value
            c["row_term"] = p.row is not None
            c["col_term"] = p.col is not None
    c["kernel"] = info["kernel"]
    c["workgroups"] = info["workgroups"]
    return c


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before timing (default: as many as fill 0.3 s, at least 5)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target duration of the CPU oracle baseline (0 skips it)")
    ap.add_argument("--no-configs", action="store_true",
                    help="time the headline workload only (no per-configuration object)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of the product, run 3 plain device copies of this many MiB "
                         "(calibrates the HBM byte counters; prints nothing else)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        return 2
    if args.steps < 1 or (args.warmup is not None and args.warmup < 0):
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_each_way": n * 4, "copies": 3}))
        return 0
    from strided_fp32_gemm_amd import workloads as wl
    names = list(wl.WORKLOADS) if args.workload == "all" else [args.workload]
    for name in names:
        line = bench_one(name, args.steps, args.warmup, args.cpu_seconds)
        if name == DEFAULT_WORKLOAD and args.workload != "all" and not args.no_configs:
            line["configs"] = configs_object(line, min(args.cpu_seconds, CONFIG_CPU_SECONDS))
        print(json.dumps(line), flush=True)
    return 0


def configs_object(headline: dict, cpu_seconds: float) -> dict:
    """Every configuration of the workload set beside the headline (config
    5), each timed in this same process, plus the attention pair together."""
    from strided_fp32_gemm_amd import workloads as wl

    # Every kernel first, back to back, so the device's clock stays where its
    # warm-up put it (an oracle slice in between leaves the GPU idle for
    # seconds); then the oracle slices.
    out = {}
    for label, name in CONFIG_WORKLOADS:
        print(f"[bench] config {label}: {name}", file=sys.stderr, flush=True)
        out[name] = config_entry(label, name)
    if cpu_seconds > 0:
        for label, name in CONFIG_WORKLOADS:
            print(f"[bench] config {label}: oracle slice", file=sys.stderr, flush=True)
            out[name]["cpu_baseline"] = cpu_baseline(wl.workload(name), cpu_seconds)
    qk, pv = out["attn_qk"], out["attn_pv"]
    ms = qk["launch_ms_mean"] + pv["launch_ms_mean"]
    fl = qk["flops_per_launch"] + pv["flops_per_launch"]
    out["attn_qk_plus_pv"] = {"config": "3", "workload": "attn_qk + attn_pv",
                              "launch_ms_mean": round(ms, 5), "tflops": round(fl / (ms * 1e-3) / 1e12, 3),
                              "frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_FP32_MATRIX_TFLOPS, 4)}
    for name in EXTRA_WORKLOADS:
        print(f"[bench] extra: {name}", file=sys.stderr, flush=True)
        out[name] = extra_entry(name)
    r = headline["roofline"]
    out["square4096_acc"] = {"config": "5", "workload": DEFAULT_WORKLOAD, "kernel": r["kernel"],
                             "launch_ms_mean": r["launch_ms_mean"], "tflops": r["achieved"],
                             "frac": r["frac"], "cpu_baseline": "see the line's cpu_baseline"}
    return out


if __name__ == "__main__":
    sys.exit(main())
