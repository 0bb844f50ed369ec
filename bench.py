#!/usr/bin/env python3
"""Throughput of the SVDQuant linear operator on one MI355X.

A step is one call of the whole per-call path (svdq_linear: smooth + quantise +
down-projection, then the residual GEMM with the up-projection epilogue) over one batch
of synthetic input already resident in HBM. Enough copies of (x, prepared weights, Y,
workspace) rotate that no call is served from the 256 MB MALL.

Prints one JSON line: value = 2*B*M*N*steps / wall time (TFLOP/s, eager launches),
the roofline of the dominant kernel (the residual GEMM, timed with HIP events the library
records around its own launches), and the CPU oracle's throughput on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1..5]   (default workload 4,
       MXFP4 4096 x 3072 x 12288, the largest single-GPU configuration)
       python bench.py --pmc-summary FETCH.csv WRITE.csv COPY_FETCH.csv COPY_WRITE.csv COPY_BYTES
       python bench.py --workload W --mfma-summary COUNTERS.csv
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "svdquant_linear TFLOP/s (2BMN) and % of MFMA/HBM roofline, 1×MI355X"
# MI355X published dense peaks
PEAK = {"hbm": 8000.0, "mxfp4": 10100.0, "int8": 5000.0, "bf16": 2500.0, "fp32": 157.3}
CSRC = os.path.join(ROOT, "rank_bit_residual_amd", "csrc")


def gemm_kernel(wl, B):
    """(kernel name, source file) of the residual GEMM that svdq_linear launches for this shape."""
    if wl.fmt == "mx" and wl.dtype == "bf16" and B <= 64:
        return "k_gemm_decode_mx", os.path.join(CSRC, "k_gemm_decode.hip")
    if wl.fmt == "mx" and wl.dtype == "bf16" and B > 64:
        return "k_gemm_mx", os.path.join(CSRC, "k_gemm_mx.hip")
    if wl.fmt == "int":
        # the large tiles once 64 x 64 tiles would need four rounds of 256 CUs
        if -(-B // 64) * -(-wl.N // 64) >= 4 * 256:
            return "k_gemm_int_big", os.path.join(CSRC, "k_gemm_mx.hip")
        return "k_gemm_int4", os.path.join(CSRC, "k_gemm_int.hip")
    # the MXFP4 kernels cover every shape of these workloads (arrays under 2 GiB)
    return "k_gemm", os.path.join(CSRC, "k_gemm.hip")


def sampling_stride(steps):
    """Every how many timed calls the residual GEMM's dispatch carries an event pair: at least
    16 sampled launches whatever the step count."""
    return max(1, steps // 16)


def algorithmic(wl, B):
    """Algorithmic work of one call and of one launch of the residual GEMM kernel.

    call_bytes: what one call must move (x, scale, Y, packed residual codes and E8M0 scales,
    both low-rank factors); gemm_bytes: the operands and output of the residual GEMM alone
    (activation codes and scales, residual codes and scales, down, L2, Y)."""
    e = 2 if wl.dtype == "bf16" else 4
    M, N, r = wl.M, wl.N, wl.rank
    mx = wl.fmt == "mx"
    code_bytes = (lambda rows, k: rows * k / 2) if (mx or wl.bits <= 4) else (lambda rows, k: rows * k)
    r_scales = M * N / 32 if mx else 4
    a_scales = B * M / 32 if mx else 4
    call = B * M * e + 4 * M + B * N * e + code_bytes(N, M) + r_scales + (M + N) * r * e
    gemm = code_bytes(B, M) + a_scales + code_bytes(N, M) + r_scales + B * r * e + N * r * e + B * N * e
    return {"flops": 2.0 * B * M * N, "call_bytes": call, "gemm_bytes": gemm}


def roofline(wl, B, work, gemm_ms, call_ms):
    """Roofline of the residual GEMM kernel (flops and its own operand bytes over its average
    launch duration) with both fractions; `bound` is whichever peak time is larger. `call`
    gives the same two fractions for a whole svdq_linear call: 2BMN and the call's
    algorithmic bytes (x, scale, Y, residual codes and scales, L1, L2) over the eager time per
    call."""
    mfma_peak = PEAK["mxfp4"] if wl.fmt == "mx" else PEAK["int8"]
    gemm_s, call_s = gemm_ms / 1e3, call_ms / 1e3
    t_mfma = work["flops"] / (mfma_peak * 1e12)
    t_hbm = work["gemm_bytes"] / (PEAK["hbm"] * 1e9)
    tf = work["flops"] / gemm_s / 1e12
    gb = work["gemm_bytes"] / gemm_s / 1e9
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": tf, "peak": mfma_peak, "unit": "TFLOP/s", "frac": tf / mfma_peak}
    else:
        roof = {"bound": "hbm", "achieved": gb, "peak": PEAK["hbm"], "unit": "GB/s", "frac": gb / PEAK["hbm"]}
    roof.update({
        "traffic": None, "kernel": gemm_kernel(wl, B)[0], "avg_ms": gemm_ms,
        "algorithmic_bytes": work["gemm_bytes"], "frac_mfma": tf / mfma_peak, "frac_hbm": gb / PEAK["hbm"],
        "call": {"bound": "mfma" if work["flops"] / (mfma_peak * 1e12) >= work["call_bytes"] / (PEAK["hbm"] * 1e9)
                 else "hbm",
                 "us": call_ms * 1e3, "tflops": work["flops"] / call_s / 1e12,
                 "frac_mfma": work["flops"] / call_s / 1e12 / mfma_peak,
                 "algorithmic_bytes": work["call_bytes"], "gbs": work["call_bytes"] / call_s / 1e9,
                 "frac_hbm": work["call_bytes"] / call_s / 1e9 / PEAK["hbm"]},
    })
    return roof


CEILINGS = os.path.join(ROOT, "profiles", "ceilings.json")


def measured_ceiling(wl, roof, path=CEILINGS):
    """The GEMM's achieved rate against the committed measured ceiling of the same kind (the
    FP4 or INT8 MFMA loop for MFMA-bound shapes, the HBM read stream for HBM-bound ones), or
    None when no ceilings were measured."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if roof["bound"] == "mfma":
        key = "fp4_mfma" if wl.fmt == "mx" else "int8_mfma"
        peak, unit = c[key]["tflops"], "TFLOP/s"
    else:
        key = "hbm_read"
        peak, unit = c[key]["gbs"], "GB/s"
    return {"probe": key, "peak": peak, "unit": unit, "frac": roof["achieved"] / peak,
            "source": os.path.relpath(path, ROOT)}


def run_ceilings(args):
    """Measured ceilings of this GPU (svdq_ceiling): the FP4 and INT8 MFMA loops, a read stream
    and a device copy over buffers rotated past the 256 MB MALL. One JSON object on stdout."""
    import torch

    from rank_bit_residual_amd import _lib as L

    lib = L.load()
    dev = torch.device("cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    scratch = torch.empty(32 << 20, dtype=torch.uint8, device=dev)  # 1 KB per block of the widest read stream

    def per_launch(fn, n):
        for _ in range(3):
            fn(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n / 1e3

    out = {"device": torch.cuda.get_device_name(dev)}
    work = ctypes.c_double()
    for kind, name in ((0, "fp4_mfma"), (1, "int8_mfma")):
        iters = 20000

        def launch(_, kind=kind, iters=iters):
            L.check(lib.svdq_ceiling(kind, iters, None, 0, ctypes.c_void_p(scratch.data_ptr()), scratch.numel(), stream,
                                     ctypes.byref(work)))

        t = per_launch(launch, 10)
        out[name] = {"tflops": work.value / t / 1e12, "launch_us": t * 1e6, "iterations": iters}
        print(f"{name}: {out[name]['tflops']:.0f} TFLOP/s", file=sys.stderr, flush=True)
    nbuf, size = 4, 256 << 20
    bufs = [torch.full((size,), i + 1, dtype=torch.uint8, device=dev) for i in range(nbuf)]
    best = None
    for blocks in (2048, 8192, 32768):
        def launch(i, blocks=blocks):
            b = bufs[i % nbuf]
            L.check(lib.svdq_ceiling(2, blocks, ctypes.c_void_p(b.data_ptr()), size,
                                     ctypes.c_void_p(scratch.data_ptr()), scratch.numel(), stream, ctypes.byref(work)))

        t = per_launch(launch, 20)
        gbs = work.value / t / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": gbs, "blocks": blocks, "bytes_per_launch": work.value, "launch_us": t * 1e6}
    out["hbm_read"] = best
    print(f"hbm_read: {best['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    dst = [torch.empty(size, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
    t = per_launch(lambda i: dst[i % nbuf].copy_(bufs[(i + 1) % nbuf]), 20)
    out["copy"] = {"gbs": 2 * size / t / 1e9, "bytes_per_launch": 2 * size, "launch_us": t * 1e6}
    out["command"] = "python bench.py --ceilings"
    print(json.dumps(out), flush=True)


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _profile_summary(wl, B, suffix):
    """A committed rocprofv3 counter summary of the GEMM for this workload, if it was taken on
    the current kernel source; else None."""
    kname, src = gemm_kernel(wl, B)
    path = os.path.join(ROOT, "profiles", f"{kname}_{wl.name}_{suffix}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    return d if d.get("source_sha") == source_sha(src) else None


def pmc_traffic(wl, B):
    """HBM bytes per GEMM launch from the committed counter summary, or None."""
    d = _profile_summary(wl, B, "traffic")
    return d.get("hbm_bytes_per_dispatch") if d else None


def pmc_mfma_util(wl, B):
    """MFMA utilisation of the GEMM (busy cycles / GPU-active cycles x SIMDs) from the committed
    counter summary, or None."""
    d = _profile_summary(wl, B, "mfma")
    return d.get("mfma_util") if d else None


def cpu_baseline(wl, x, s, prep, budget_s=10.0):
    """The oracle's forward (numpy, float64 BLAS) on a row sample, repeated to ~budget_s."""
    import torch
    from oracle import svdquant as O

    try:
        from threadpoolctl import threadpool_info

        cores = max((d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"), default=0)
    except Exception:  # pragma: no cover - threadpoolctl missing
        cores = 0
    cores = cores or len(os.sched_getaffinity(0))
    left = prep.left.to(torch.float32).numpy()
    right = prep.right.to(torch.float32).numpy()
    res = prep.residual.to(torch.float32).numpy()
    rows = min(wl.B, 64)
    t0 = time.perf_counter()
    O.forward_ref(x[:rows], s, left, right, res, wl.fmt, wl.bits, wl.dtype)
    one = time.perf_counter() - t0
    # grow the sample (rows, then repetitions) towards the budget
    if rows < wl.B and one < budget_s / 4:
        rows = min(wl.B, int(rows * max(1.0, (budget_s / 4) / max(one, 1e-3))))
    reps, done, t_total = 0, 0.0, 0.0
    while t_total < budget_s and reps < 10000:
        t0 = time.perf_counter()
        O.forward_ref(x[:rows], s, left, right, res, wl.fmt, wl.bits, wl.dtype)
        t_total += time.perf_counter() - t0
        reps += 1
        done += 2.0 * rows * wl.M * wl.N
    return {"value": done / t_total / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"oracle forward_ref on {rows} of {wl.B} rows x {reps} repetitions ({t_total:.1f} s), "
                      f"float64 numpy BLAS on the host ({_cpu_model()})"}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def run(args):
    import numpy as np
    import torch

    import rank_bit_residual_amd as R
    from rank_bit_residual_amd import _lib as L
    from workloads import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    td = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    x, w, s = make_inputs(wl)
    t_prep = time.perf_counter()
    prep = R.prepare(torch.from_numpy(w).to(td), torch.from_numpy(s), wl.rank, wl.bits, wl.fmt, device=dev,
                     keep_factors=not args.no_cpu_baseline)
    torch.cuda.synchronize()
    t_prep = time.perf_counter() - t_prep  # host fold + SVD + quantisation + blob copy (one-time)
    B, M, N = wl.B, wl.M, wl.N
    wsb = R.workspace_bytes(B, prep)
    x_g = torch.from_numpy(x).to(td).to(dev)
    footprint = x_g.numel() * x_g.element_size() + prep.blob.numel() + B * N * x_g.element_size() + wsb
    copies = max(2, math.ceil(args.rotate_mb * 2**20 / footprint))
    xs = [x_g.clone() for _ in range(copies)]
    blobs = [prep.blob.clone() for _ in range(copies)]
    ys = [torch.empty((B, N), dtype=td, device=dev) for _ in range(copies)]
    wss = [torch.empty(wsb, dtype=torch.uint8, device=dev) for _ in range(copies)]
    lib = L.load()
    stream = torch.cuda.current_stream(dev)
    fmt = L.SVDQ_FMT_MX if wl.fmt == "mx" else L.SVDQ_FMT_INT
    dt = L.SVDQ_BF16 if wl.dtype == "bf16" else L.SVDQ_F32
    call_args = [(ctypes.c_void_p(xs[i].data_ptr()), B, M, M, ctypes.c_void_p(blobs[i].data_ptr()), N, wl.rank, fmt,
                  wl.bits, dt, ctypes.c_void_p(ys[i].data_ptr()), N, ctypes.c_void_p(wss[i].data_ptr()), wsb,
                  ctypes.c_void_p(stream.cuda_stream)) for i in range(copies)]
    fn = lib.svdq_linear

    def step(i):
        st = fn(*call_args[i % copies])
        if st:
            L.check(st)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    def stage_times(steps, full=False):
        ms = (ctypes.c_float * (steps * L.NSTAGES))()
        n = ctypes.c_int()
        L.check(lib.svdq_profile_end(ms, steps, ctypes.byref(n)))
        per = np.array(ms[: n.value * L.NSTAGES], dtype=np.float64).reshape(n.value, L.NSTAGES)
        if full:
            return per
        return {name: float(per[:, k].mean()) for k, name in enumerate(L.STAGE_NAMES) if per[:, k].any()}

    def pct(a):
        return [float(v) for v in np.percentile(np.asarray(a) * 1e3, [10, 50, 90])]

    # ---- timed region: eager launches. The library passes one HIP event pair to the
    # residual-GEMM dispatch of every EVERY-th call (stage 3 only): the roofline's kernel
    # duration comes from the timed calls themselves. EVERY = steps // 16 (at least 1), so the
    # average always rests on at least 16 launches (every launch of a short run) while long
    # runs of short calls do not become host-bound on the event records.
    GEMM_STAGE = 3
    EVERY = sampling_stride(args.steps)
    L.check(lib.svdq_profile_begin_sampled(max(1, args.steps // EVERY + 1), 1 << GEMM_STAGE, EVERY))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t_eager = time.perf_counter() - t0
    gemm_per_call = stage_times(args.steps // EVERY + 1, full=True)[:, GEMM_STAGE]
    gemm_ms = float(gemm_per_call.mean())
    work = algorithmic(wl, B)
    value = work["flops"] * args.steps / t_eager / 1e12

    # ---- per-kernel breakdown of every stage (separate pass; informational)
    L.check(lib.svdq_profile_begin(args.steps, (1 << L.NSTAGES) - 1))
    for i in range(args.steps):
        step(i)
    stage_ms = stage_times(args.steps)

    # ---- per-call distribution: one HIP event pair around each call on the call's stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    call_ms = [a.elapsed_time(b) for a, b in evs]

    # ---- HIP-graph replay of the same calls (reported separately, not the headline)
    graph = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        per_graph = min(copies * 4, 64)
        cap_stream = torch.cuda.Stream(dev)
        cap_stream.wait_stream(stream)
        with torch.cuda.stream(cap_stream):
            gargs = [(a[:-1] + (ctypes.c_void_p(cap_stream.cuda_stream),)) for a in call_args]
            for i in range(copies):  # warm the capture stream
                L.check(fn(*gargs[i]))
            cap_stream.synchronize()
            with torch.cuda.graph(g, stream=cap_stream):
                for i in range(per_graph):
                    L.check(fn(*gargs[i % copies]))
        torch.cuda.synchronize()
        reps = max(1, args.steps // per_graph)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        t_graph = time.perf_counter() - t0
        graph = {"ms_per_step": t_graph / (reps * per_graph) * 1e3,
                 "value": work["flops"] * reps * per_graph / t_graph / 1e12, "calls_per_graph": per_graph}

    # ---- roofline of the dominant kernel (the residual GEMM), and of the whole call
    roof = roofline(wl, B, work, gemm_ms, t_eager / args.steps * 1e3)
    roof["traffic"] = pmc_traffic(wl, B)
    if roof["bound"] == "mfma":
        roof["mfma_util"] = pmc_mfma_util(wl, B)  # counter evidence: MFMA busy / active cycles
    roof["measured_ceiling"] = measured_ceiling(wl, roof)

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": t_eager / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "mxfp4" if wl.fmt == "mx" else "int8",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "M": M, "N": N, "rank": wl.rank, "format": wl.fmt, "bits": wl.bits,
                   "io_dtype": wl.dtype, "rotating_copies": copies},
        "roofline": roof,
        "call_gbs": work["call_bytes"] / (t_eager / args.steps) / 1e9,
        "call_us_p10_p50_p90": pct(call_ms),
        "gemm_us_p10_p50_p90": pct(gemm_per_call),
        "gemm_timed_calls": int(len(gemm_per_call)),
        "host_prepare_s": t_prep,
        "kernels_ms": stage_ms,
        "graph": graph,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, x, s, prep)
    print(json.dumps(out), flush=True)


def run_calibrate(args):
    """Smoothing-scale calibration (the step before the operator's path) on a workload's x and
    W: svdq_calibrate_scale timed over rotating copies of (x, W), GB/s of its algorithmic bytes
    (x + W + the float32 scale) against the HBM peak, and the oracle on the host beside it."""
    import numpy as np
    import torch

    from rank_bit_residual_amd import _lib as L
    from workloads import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    alpha = wl.alpha
    dev = torch.device("cuda:0")
    td = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    x, w, _ = make_inputs(wl)
    B, M, N = wl.B, wl.M, wl.N
    x_g = torch.from_numpy(x).to(td).to(dev)
    w_g = torch.from_numpy(w).to(td).to(dev)
    e = x_g.element_size()
    nbytes = (B * M + M * N) * e + 4 * M
    copies = max(2, math.ceil(args.rotate_mb * 2**20 / nbytes))
    xs = [x_g.clone() for _ in range(copies)]
    wss = [w_g.clone() for _ in range(copies)]
    lib = L.load()
    wsb = ctypes.c_size_t()
    L.check(lib.svdq_calibrate_workspace_bytes(B, M, ctypes.byref(wsb)))
    work = torch.empty(wsb.value, dtype=torch.uint8, device=dev)
    out = torch.empty(M, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    dt = L.SVDQ_BF16 if wl.dtype == "bf16" else L.SVDQ_F32

    def step(i):
        L.check(lib.svdq_calibrate_scale(ctypes.c_void_p(xs[i % copies].data_ptr()), B, M, M,
                                         ctypes.c_void_p(wss[i % copies].data_ptr()), N, N, dt, alpha,
                                         ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(work.data_ptr()),
                                         wsb.value, ctypes.c_void_p(stream.cuda_stream)))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t0
    call_ms = np.array([a.elapsed_time(b) for a, b in evs])
    gbs = nbytes / (call_ms.mean() / 1e3) / 1e9
    res = {"metric": "svdq_calibrate_scale GB/s (x + W + scale) and % of HBM roofline, 1xMI355X", "value": gbs,
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": t_wall / args.steps * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f64", "data": "synthetic",
           "config": {"workload": wl.name + "_calibration", "B": B, "M": M, "N": N, "alpha": alpha,
                      "io_dtype": wl.dtype, "rotating_copies": copies},
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK["hbm"], "unit": "GB/s",
                        "frac": gbs / PEAK["hbm"], "traffic": None, "kernel": "k_calib_colmax + k_calib_finish",
                        "avg_ms": float(call_ms.mean()), "algorithmic_bytes": nbytes},
           "call_us_p10_p50_p90": [float(v) for v in np.percentile(call_ms * 1e3, [10, 50, 90])]}
    if not args.no_cpu_baseline:
        from oracle import svdquant as O

        reps, t_total = 0, 0.0
        while t_total < 10.0 and reps < 1000:
            t1 = time.perf_counter()
            O.calibrate_scale(x, w, alpha)
            t_total += time.perf_counter() - t1
            reps += 1
        res["cpu_baseline"] = {"value": nbytes * reps / t_total / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "sample": f"oracle calibrate_scale on the whole workload x {reps} repetitions "
                                         f"({t_total:.1f} s), numpy on the host ({_cpu_model()})"}
    print(json.dumps(res), flush=True)


def run_prepare(args):
    """One-time preparation of the workload's weight (fold, truncated SVD, residual
    quantisation and packing): the host route and the route with the truncated SVD on the GPU,
    timed once each (wall clock, including the blob copy to the device)."""
    import numpy as np
    import torch

    import rank_bit_residual_amd as R
    from workloads import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    td = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    x, w, s = make_inputs(wl, B=min(wl.B, 64))
    wt = torch.from_numpy(w).to(td)
    out = {"metric": "one-time preparation seconds (fold + truncated SVD + residual quantisation)",
           "unit": "s", "higher_is_better": False, "n_gpus": 1, "data": "synthetic",
           "config": {"workload": wl.name, "M": wl.M, "N": wl.N, "rank": wl.rank, "format": wl.fmt}}
    for name, gpu in (("host", False), ("gpu_svd", True)):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        p = R.prepare(wt, torch.from_numpy(s), wl.rank, wl.bits, wl.fmt, device=dev, keep_factors=True, svd_on_gpu=gpu)
        torch.cuda.synchronize()
        out[name + "_s"] = time.perf_counter() - t0
        out[name + "_residual_fro"] = float(np.linalg.norm(p.residual.to(torch.float32).numpy()))
    print(json.dumps(out), flush=True)


def toy_experiment(dev_name="cuda:0"):
    """The exercise page's toy experiment ("SVDQuant Smoothing, Low-rank and Residual
    Quantization", "Toy experiment") through the library on the GPU, with the oracle's numbers
    beside it: relative output errors of naive W4A4, smoothing only, and the two-branch
    operator at ranks 0-6, and the leading singular values of W before and after smoothing
    (from the library's split: the column norms of L1 = U S, since L2 = V^T has orthonormal
    rows). Inputs: the toy workload (x [16, 64] with outlier channels, W [64, 48] with a
    rank-4 spike), float32."""
    import numpy as np
    import torch

    import rank_bit_residual_amd as R
    from oracle import svdquant as O
    from workloads import make_inputs

    dev = torch.device(dev_name)
    x, w, s = make_inputs(1)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    xg, wg, sg = (torch.from_numpy(a).to(dev) for a in (x, w, s))

    def err(y):
        return O.rel_fro(y, ref)

    def f64(t):
        return t.detach().to("cpu", torch.float64).numpy()

    lib = {"naive_w4a4": err(f64(R.fake_quantize(xg, 4)) @ f64(R.fake_quantize(wg, 4)))}
    xs, ws = R.smooth_inputs(xg, wg, sg)
    lib["smoothing_only"] = err(f64(R.fake_quantize(xs, 4)) @ f64(R.fake_quantize(ws, 4)))
    lib["two_branch"] = [err(f64(R.svdquant_linear(xg, wg, sg, r, 4))) for r in range(7)]
    orc = {"naive_w4a4": err(O.fake_quantize(x, 4, "f32").astype(np.float64) @ O.fake_quantize(w, 4, "f32"))}
    oxs, ows = O.smooth_inputs(x, w, s, "f32")
    orc["smoothing_only"] = err(O.fake_quantize(oxs, 4, "f32").astype(np.float64) @ O.fake_quantize(ows, 4, "f32"))
    orc["two_branch"] = [err(O.svdquant_linear(x, w, s, r, 4)) for r in range(7)]
    k = min(w.shape)
    sv_lib = {name: np.linalg.norm(f64(R.split_weight(m, k)[0]), axis=0).tolist()
              for name, m in (("W", wg.cpu()), ("smoothed_W", ws.cpu()))}
    sv_orc = {"W": np.linalg.svd(w.astype(np.float64), compute_uv=False).tolist(),
              "smoothed_W": np.linalg.svd(ows.astype(np.float64), compute_uv=False).tolist()}
    return {"library": lib, "oracle": orc, "singular_values_library": sv_lib, "singular_values_oracle": sv_orc}


def pmc_summary(fetch_csv, write_csv, cfetch_csv, cwrite_csv, copy_bytes, wl, command):
    """Per-dispatch HBM bytes of the residual GEMM from rocprofv3 counter CSVs (FETCH_SIZE and
    WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads for a plain
    device copy of copy_bytes bytes."""
    import csv

    def per_dispatch(path, counter, name_pred):
        vals = []
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") == counter and name_pred(row.get("Kernel_Name", "")):
                    vals.append(float(row["Counter_Value"]))
        return sum(vals) / len(vals) if vals else float("nan"), len(vals)

    kname, src = gemm_kernel(wl, wl.B)
    is_gemm = lambda k: (kname + "<") in k or (kname + "(") in k  # noqa: E731
    is_copy = lambda k: "copyBuffer" in k  # the runtime's device-to-device copy kernel  # noqa: E731
    f_kib, nf = per_dispatch(fetch_csv, "FETCH_SIZE", is_gemm)
    w_kib, nw = per_dispatch(write_csv, "WRITE_SIZE", is_gemm)
    cf_kib, _ = per_dispatch(cfetch_csv, "FETCH_SIZE", is_copy)
    cw_kib, _ = per_dispatch(cwrite_csv, "WRITE_SIZE", is_copy)
    rf = copy_bytes / (cf_kib * 1024)
    rw = copy_bytes / (cw_kib * 1024)
    d = {"kernel": kname, "workload": wl.name, "source_sha": source_sha(src),
         "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib, "dispatches": [nf, nw],
         "copy_factor_fetch": rf, "copy_factor_write": rw,
         "hbm_bytes_per_dispatch": f_kib * 1024 * rf + w_kib * 1024 * rw, "command": command}
    print(json.dumps(d, indent=1))


def mfma_summary(csv_path, wl, command):
    """MFMA utilisation of the residual GEMM from one rocprofv3 counter CSV holding
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_MFMA and GRBM_GUI_ACTIVE (with --kernel-trace):
    busy cycles summed over the SIMDs / (GPU-active cycles of one XCC x SIMDs), the same
    definition as rocprof's MfmaUtil. GRBM_GUI_ACTIVE is summed over the XCCs in the CSV."""
    import csv
    per = {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            k = row.get("Kernel_Name", "")
            kname, _ = gemm_kernel(wl, wl.B)
            if (kname + "<") not in k and (kname + "(") not in k:
                continue
            d = per.setdefault(row["Dispatch_Id"], {})
            d[row["Counter_Name"]] = float(row["Counter_Value"])
            d["ns"] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
    ds = [d for d in per.values() if {"SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_MFMA"} <= d.keys()]
    n = len(ds)
    avg = lambda key: sum(d[key] for d in ds) / n  # noqa: E731
    xcc, simds = 8, 1024
    busy, gui, inst, ns = avg("SQ_VALU_MFMA_BUSY_CYCLES"), avg("GRBM_GUI_ACTIVE") / xcc, avg("SQ_INSTS_MFMA"), avg("ns")
    kname, src = gemm_kernel(wl, wl.B)
    print(json.dumps({"kernel": kname, "workload": wl.name, "source_sha": source_sha(src), "dispatches": n,
                      "mfma_instructions": inst, "mfma_busy_cycles": busy, "gpu_active_cycles_per_xcc": gui,
                      "dispatch_ns": ns, "mfma_util": busy / (gui * simds),
                      "mfma_busy_fraction_at_2400MHz": busy / (simds * ns * 2.4), "command": command}, indent=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=800)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4, 5],
                    help="1 toy f32 INT4, 2 INT4 W4A4 bf16, 3 MXFP4 DiT attention, 4 MXFP4 MLP up (default: the "
                         "largest single-GPU workload), 5 MXFP4 decode")
    ap.add_argument("--rotate-mb", type=float, default=512.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--pmc-summary", nargs=5, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE", "COPY_BYTES"))
    ap.add_argument("--mfma-summary", metavar="CSV", help="MFMA utilisation of the GEMM from a counter CSV")
    ap.add_argument("--pmc-command", default="")
    ap.add_argument("--toy-experiment", action="store_true",
                    help="run the exercise page's toy experiment through the library and print its error table")
    ap.add_argument("--prepare", action="store_true",
                    help="time the one-time weight preparation on the host and with the GPU SVD products")
    ap.add_argument("--calibrate", action="store_true",
                    help="time the smoothing-scale calibration on the workload's x and W instead of the operator")
    ap.add_argument("--ceilings", action="store_true",
                    help="measure the chip's FP4/INT8 MFMA, HBM read and copy ceilings (one JSON line)")
    ap.add_argument("--copy-probe", type=int, metavar="BYTES",
                    help="only run 5 device-to-device copies of BYTES bytes (counter calibration)")
    args = ap.parse_args()
    if args.mfma_summary:
        from workloads import WORKLOADS

        mfma_summary(args.mfma_summary, WORKLOADS[args.workload], args.pmc_command)
        return 0
    if args.pmc_summary:
        from workloads import WORKLOADS

        f, w_, cf, cw, cb = args.pmc_summary
        pmc_summary(f, w_, cf, cw, float(cb), WORKLOADS[args.workload], args.pmc_command)
        return 0
    if args.copy_probe:
        import torch

        src = torch.ones(args.copy_probe // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copied {args.copy_probe} bytes 5 times", flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures the operator on one GPU only; --gpus {args.gpus} is not supported", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
    if args.ceilings:
        run_ceilings(args)
    elif args.prepare:
        run_prepare(args)
    elif args.toy_experiment:
        print(json.dumps(toy_experiment()), flush=True)
    elif args.calibrate:
        run_calibrate(args)
    else:
        run(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
