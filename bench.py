#!/usr/bin/env python3
"""Throughput of the late-layer cache fill on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole fill path over one batch of synthetic input:
rf_fill_rows (the fill-row set from the exact rows) and rf_fill (map
contraction, RMSNorm, K/V projections, RoPE and cache scatter for every late
layer; for the streamed workload also the host->device map copies).  Inputs
are resident in device memory (pinned host memory for streamed maps) before
the timed region starts.  W untimed steps, then K timed steps bracketed by
device synchronisation, with an event between steps for the median and
minimum step time; one JSON line goes to stdout, progress to stderr.

``value`` is filled rows per second over all late layers on the 27B-shaped
120K-row workload (or --workload).  Without --workload the same line also
carries the 8B-shaped, 27B-shaped (64K rows) and streamed ragged 8B-shaped
workloads under ``extra.workloads``, each measured the same way after the
previous one's buffers are freed.  The roofline entry is the dominant kernel
(the map contraction): algorithmic flops per launch, 2 d_in d_out per filled
row per layer times the rows and layers one launch processes, divided by its
mean launch time from HIP events recorded around every launch on the stream it
runs on.  ``cpu_baseline`` is the fp64 numpy oracle timed on a bounded sample
of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import re
import sys
import time

import numpy as np

import workloads

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
PEAK_FP64_TFLOPS = 78.6     # MI355X dense fp64 MFMA, published
HOST_THREADS_PER_GPU = 16   # host threads a one-GPU job may use on the measurement machines

# layers per launch used by the benchmark
GROUP = {"tiny": 4, "8b": 22, "27b": 6, "27b_120k": 6, "8b_ragged_host": 4}
# rows of the oracle's timed sample (None: every fill row), sized for 10-30 s
CPU_SAMPLE = {"tiny": None, "8b": 8192, "27b": 4096, "27b_120k": 4096, "8b_ragged_host": 8192}
# the workloads the default run adds to its line, after the headline one
EXTRA_WORKLOADS = ("8b", "27b", "8b_ragged_host")
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "late_layer_kv_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def t16(a, dev, pinned=False):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.pin_memory() if pinned else t.to(dev)


def flops_per_row_layer(s):
    """Algorithmic flops of one filled row in one late layer: the map
    (2 d_in d_out) and the key, value and indexer-key projections
    (2 d_out (2 w + idx_heads hd))."""
    return 2 * s.d_in * s.d_out, 2 * s.d_out * (2 * s.kv_width + s.idx_heads * s.head_dim)


# The sources a fill's kernels and launches come from (the fit's capture and
# solve are not on the fill path and do not change its traffic).
FILL_SOURCES = ("rf_kernels.hip", "rf_rows.hip", "rf_quant.hip", "rf_rescale.hip", "rf_internal.h", "rf_api.cpp")


def kernel_source_hash() -> str:
    """SHA-256 over the sources of the fill's kernels and of their launches."""
    import hashlib
    h = hashlib.sha256()
    for name in FILL_SOURCES:
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_path(name: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{name}.json")


def measured_traffic(name: str):
    """The traffic record of a workload, if it was taken on the current device sources."""
    try:
        with open(traffic_path(name)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t if t.get("kernel_source_sha256") == kernel_source_hash() else None


def _short_kernel(name: str) -> str:
    m = re.search(r"(\w+?)_kernel\b", name)
    return m.group(1) if m else name


def summarize_pmc(fetch_csv: str, write_csv: str, name: str, calib_bytes: int, steps: int) -> dict:
    """HBM traffic per kernel from two rocprofv3 --pmc CSVs (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads
    for a device copy of known size; per launch and per step (the profiled
    process ran `steps` steps)."""
    import csv

    lib_kernels = set()

    def per_kernel(path, counter):
        sums, n, copy = {}, {}, []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            k, v = r["Kernel_Name"], float(r["Counter_Value"])
            if "copyBuffer" in k or "copy" in k.lower():
                copy.append((int(r["Grid_Size"]), v))
                continue
            kk = _short_kernel(k)
            if "rf::" in k:
                lib_kernels.add(kk)
            sums[kk] = sums.get(kk, 0.0) + v
            n[kk] = n.get(kk, 0) + 1
        return sums, n, (max(copy)[1] if copy else None)

    fs, fn, fc = per_kernel(fetch_csv, "FETCH_SIZE")
    ws, wn, wc = per_kernel(write_csv, "WRITE_SIZE")
    kf = calib_bytes / (fc * 1024.0) if fc else 1.0
    kw = calib_bytes / (wc * 1024.0) if wc else 1.0
    kernels = {}
    for k in fs:
        bytes_total = fs[k] * 1024 * kf + ws.get(k, 0.0) * 1024 * kw
        kernels[k] = {"dispatches": fn[k], "fetch_kib_per_launch": fs[k] / fn[k],
                      "write_kib_per_launch": ws.get(k, 0.0) / max(wn.get(k, 1), 1),
                      "bytes_per_launch": bytes_total / fn[k], "bytes_per_step": bytes_total / steps}
    cmd = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc {c} -f csv -d <out>/{d} -o {d} -- "
           "python3 <repo>/bench.py --workload " + name + " --steps " + str(steps - 1)
           + " --warmup 1 --no-cpu-baseline --calibrate-copy " + str(calib_bytes >> 20))
    out = {"workload": name, "kernel_source_sha256": kernel_source_hash(), "steps_profiled": steps,
           "copy_calibration": {"bytes": calib_bytes, "fetch_kib": fc, "write_kib": wc,
                                "fetch_factor": kf, "write_factor": kw},
           "kernels": kernels,
           # the library's kernels launched every step (not the RoPE table a plan
           # builds once, nor the profiled process's own torch kernels)
           "bytes_per_step": sum(v["bytes_per_step"] for k, v in kernels.items()
                                 if k in lib_kernels and v["dispatches"] >= steps),
           "counted_per_step": sorted(k for k, v in kernels.items() if k in lib_kernels and v["dispatches"] >= steps),
           "source": {"FETCH_SIZE": cmd.format(c="FETCH_SIZE", d="fetch"),
                      "WRITE_SIZE": cmd.format(c="WRITE_SIZE", d="write"),
                      "summary": (f"python bench.py --workload {name} --pmc-summary "
                                  f"<out>/fetch/fetch_counter_collection.csv "
                                  f"<out>/write/write_counter_collection.csv {calib_bytes >> 20} {steps}")}}
    if "map_gemm" in kernels:
        out["traffic_bytes_per_launch"] = kernels["map_gemm"]["bytes_per_launch"]
    return out


def blas_reference(s, steps):
    """torch.matmul (hipBLASLt) on the fill's two contraction shapes, bf16."""
    import torch
    n_fill = s.n_rows - len(workloads.exact_row_list(s))
    out = {}
    for label, (m, n, k) in (("map", (n_fill, s.d_out, s.d_in)), ("kv", (n_fill, 2 * s.kv_width, s.d_out))):
        a = torch.randn(m, k, device="cuda:0", dtype=torch.bfloat16)
        b = torch.randn(n, k, device="cuda:0", dtype=torch.bfloat16)
        for _ in range(3):
            c = a @ b.t()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            c = a @ b.t()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        out[label] = {"m": m, "n": n, "k": k, "ms": ms, "tflops": 2 * m * n * k / (ms * 1e-3) / 1e12}
        del a, b, c
    print(json.dumps({"blas_reference": out, "workload": s.name}), flush=True)


def capture_bench(s, rows, steps, warmup):
    """rf_ridge_dev_add on `rows` rows of width d_in -> d_out: fp64 running sums
    of X^T X (upper half) and X^T Y, section 2.2 "Fitting"."""
    import torch
    from late_layer_kv_amd import binding as B
    g = torch.Generator(device="cuda:0").manual_seed(0)
    x = torch.randn((rows, s.d_in), generator=g, device="cuda:0").to(torch.bfloat16).view(torch.int16)
    y = torch.randn((rows, s.d_out), generator=g, device="cuda:0").to(torch.bfloat16).view(torch.int16)
    dev = B.RidgeDeviceSums(s.d_in, s.d_out)
    for _ in range(warmup):
        dev.add(x, y)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        dev.add(x, y)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flop = 2.0 * rows * s.d_in * (s.d_in / 2 + s.d_out)
    tf = flop / (ms * 1e-3) / 1e12
    # the solve from the same sums (fp64 blocked Cholesky + two triangular solves)
    ws = torch.empty(dev.solve_workspace_bytes(), dtype=torch.uint8, device="cuda:0")
    a = torch.empty((s.d_out, s.d_in), dtype=torch.float32, device="cuda:0")
    b = torch.empty(s.d_out, dtype=torch.float32, device="cuda:0")
    dev.solve(0.03, a=a, b=b, workspace=ws)
    t0 = time.perf_counter()
    n_solve = max(1, min(steps, 5))
    for _ in range(n_solve):
        dev.solve(0.03, a=a, b=b, workspace=ws)   # synchronises
    solve_ms = (time.perf_counter() - t0) * 1e3 / n_solve
    solve_flop = s.d_in ** 3 / 3.0 + 2.0 * s.d_in ** 2 * s.d_out
    stf = solve_flop / (solve_ms * 1e-3) / 1e12
    print(json.dumps({"capture": {"workload": s.name, "rows": rows, "d_in": s.d_in, "d_out": s.d_out,
                                  "ms_per_call": ms, "rows_per_s": rows / (ms * 1e-3),
                                  "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_FP64_TFLOPS,
                                               "unit": "TFLOP/s (fp64)", "frac": tf / PEAK_FP64_TFLOPS}},
                      "solve": {"d_in": s.d_in, "d_out": s.d_out, "ms_per_solve": solve_ms,
                                "flop": solve_flop, "achieved_tflops_fp64": stf,
                                "frac_of_fp64_peak": stf / PEAK_FP64_TFLOPS,
                                "note": "wall clock of rf_ridge_dev_solve including its final stream sync"}}),
          flush=True)


def host_facts() -> dict:
    """The host's CPU as the oracle sees it."""
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
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "model": model}


def cpu_baseline(w, fill, name):
    """The fp64 oracle on a seeded sample of fill rows, all late layers, with
    numpy's BLAS on the host threads one GPU's job may use."""
    import oracle
    host = host_facts()
    threads = max(1, min(HOST_THREADS_PER_GPU, host["usable_cpus"]))
    n = CPU_SAMPLE[name]
    rows = fill if n is None or n >= len(fill) else \
        np.sort(np.random.default_rng(0).choice(fill, size=n, replace=False)).astype(np.int32)
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=threads)
    except ImportError:   # threadpoolctl missing: numpy keeps its own pool size
        import contextlib
        limit = contextlib.nullcontext()
    with limit:
        t0 = time.perf_counter()
        oracle.fill_workload(w, rows=rows)
        dt = time.perf_counter() - t0
    host["blas_threads"] = threads
    host["note"] = (f"the oracle's BLAS uses min({HOST_THREADS_PER_GPU}, usable CPUs) threads: "
                    f"a one-GPU job's share of the host's cores")
    return {"value": len(rows) / dt, "unit": "rows/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(rows)} fill rows x all {w.spec.n_late} late layers, fp64 numpy, {dt:.1f} s",
            "host": host}


def pinned_copy_rate(dev, mib=256, reps=5) -> dict:
    """Host-to-device rate of plain copies from pinned memory (the ceiling for
    streamed maps), same process, same stream."""
    import torch
    n = mib << 20
    h = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    h.fill_(1)
    d = torch.empty(n, dtype=torch.uint8, device=dev)
    d.copy_(h, non_blocking=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        d.copy_(h, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del h, d
    return {"bytes": n, "ms": ms, "gbs": n / (ms * 1e-3) / 1e9}


def run_workload(name, args, headline: bool) -> dict:
    """Set up one workload, time it, and return its part of the JSON line."""
    import torch
    from late_layer_kv_amd import binding as B

    q8 = args.maps == "q8"
    s = workloads.spec(name, map_format=args.maps, qk_norm=args.qk_norm, idx_heads=args.indexer)
    if args.spans is not None and headline:
        s = workloads.spec(name, map_format=args.maps, qk_norm=args.qk_norm, idx_heads=args.indexer,
                           n_spans=args.spans)
    dev = "cuda:0"
    log(f"[bench] {name}: drawing inputs")
    t0 = time.perf_counter()
    w = workloads.make(s)
    log(f"[bench] {name}: inputs drawn in {time.perf_counter() - t0:.1f} s; uploading")
    host_maps = s.maps_on_host
    x = t16(w.x, dev)
    if q8:
        place = (lambda t: t.pin_memory()) if host_maps else (lambda t: t.to(dev))
        map_q = [place(torch.from_numpy(np.ascontiguousarray(q))) for q in w.map_q]
        map_s = [t16(sc, dev, host_maps) for sc in w.map_scale]
    else:
        map_a = [t16(a, dev, host_maps) for a in w.map_a]
    map_b = [t16(b, dev, host_maps) for b in w.map_b]
    gamma = [t16(g, dev) for g in w.gamma]
    k_norm = [t16(g, dev) for g in w.k_norm] if w.k_norm is not None else None
    w_idx = [t16(a, dev) for a in w.w_idx] if w.w_idx is not None else None
    w_k = [t16(a, dev) for a in w.w_k]
    w_v = [t16(a, dev) for a in w.w_v]
    positions = torch.from_numpy(w.positions).to(dev)
    exact = torch.from_numpy(w.exact_rows).to(dev)
    n_fill = s.n_rows - len(np.unique(w.exact_rows))
    kc = [torch.empty((s.n_rows, s.kv_width), dtype=torch.int16, device=dev) for _ in range(s.n_late)]
    vc = [torch.empty((s.n_rows, s.kv_width), dtype=torch.int16, device=dev) for _ in range(s.n_late)]
    ic = [torch.empty((s.n_rows, s.idx_heads * s.head_dim), dtype=torch.int16, device=dev)
          for _ in range(s.n_late)] if w_idx is not None else None

    plan = B.Plan.for_spec(s)
    g = (args.layers_per_launch if headline and args.layers_per_launch else GROUP[name])
    ws = torch.empty(plan.fill_workspace_bytes(n_fill, g), dtype=torch.uint8, device=dev)
    # The RoPE table depends only on the model (positions up to max_pos, head_dim,
    # theta): built once per plan like the weights, outside the timed steps,
    # unless --rope-per-call asks the fill to build it inside every call.
    rope = None
    if not args.rope_per_call:
        rope = torch.empty((s.max_pos, s.head_dim // 2, 2), dtype=torch.float32, device=dev)
        B.rope_table(plan, rope)
    vscale = measure = None
    if args.value_rescale:
        c_rows, c_grp = workloads.calibration_row_list(s, args.value_rescale)
        truth = [t16(t, dev) for t in workloads.make_layer_truth(s, len(c_rows), outliers=w.outlier_channels)]
        c_rows_d = torch.from_numpy(c_rows).to(dev)
        c_grp_d = torch.from_numpy(c_grp).to(dev)
        n_groups = len(s.prompt_lens)
        scales = torch.empty((s.n_late, n_groups, s.n_kv), dtype=torch.float32, device=dev)
        ws_scale = torch.empty(plan.value_scales_workspace_bytes(len(c_rows), g), dtype=torch.uint8, device=dev)
        g_of_row = torch.from_numpy(workloads.prompt_of_row(s)).to(dev)
        vscale = (scales, g_of_row, n_groups)
        measure = None if args.separate_measure else (truth, c_rows_d, c_grp_d, g_of_row, n_groups, scales, ws_scale)
    fill_rows = torch.empty(s.n_rows, dtype=torch.int32, device=dev)
    n_fill_dev = torch.empty(1, dtype=torch.int32, device=dev)
    rows_ws = torch.empty(B.fill_rows_workspace_bytes(s.n_rows), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        B.fill_rows(plan, exact, fill_rows, n_fill_dev, rows_ws)
        if vscale is not None and measure is not None:
            if q8:
                B.fill_q8(plan, x, fill_rows, n_fill, positions, None, map_q, map_s, map_b, gamma, w_k, w_v, rope,
                          kc, vc, ws, k_norm=k_norm, w_idx=w_idx, idx_cache=ic, measure=measure)
            else:
                B.fill(plan, x, fill_rows, n_fill, positions, None, map_a, map_b, gamma, w_k, w_v, rope, kc, vc, ws,
                       k_norm=k_norm, w_idx=w_idx, idx_cache=ic, measure=measure)
            return
        if vscale is not None:
            if q8:
                B.value_scales(plan, x, truth, c_rows_d, c_grp_d, n_groups, map_q, map_b, gamma, w_v, scales,
                               ws_scale, map_scale=map_s)
            else:
                B.value_scales(plan, x, truth, c_rows_d, c_grp_d, n_groups, map_a, map_b, gamma, w_v, scales,
                               ws_scale)
        if q8:
            B.fill_q8(plan, x, fill_rows, n_fill, positions, None, map_q, map_s, map_b, gamma, w_k, w_v, rope,
                      kc, vc, ws, vscale=vscale, k_norm=k_norm, w_idx=w_idx, idx_cache=ic)
        else:
            B.fill(plan, x, fill_rows, n_fill, positions, None, map_a, map_b, gamma, w_k, w_v, rope, kc, vc, ws,
                   vscale=vscale, k_norm=k_norm, w_idx=w_idx, idx_cache=ic)

    log(f"[bench] {name}: n_fill={n_fill}, {s.n_late} late layers, {g} per launch; warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(n_fill_dev.item()) == n_fill

    log(f"[bench] {name}: timing {args.steps} steps")
    plan.profile(True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(args.steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    prof = plan.profile_read()
    plan.profile(False)
    if args.calibrate_copy and headline:
        n16 = (args.calibrate_copy << 20) // 2
        src = torch.ones(n16, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    f_map, f_kv = flops_per_row_layer(s)
    step_flops = n_fill * s.n_late * (f_map + f_kv)
    map_ms, map_n = prof["map"]
    kv_ms, kv_n = prof["kv"]
    map_launch_flops = n_fill * s.n_late * f_map * args.steps / max(map_n, 1)
    map_avg_ms = map_ms / max(map_n, 1)
    map_tflops = map_launch_flops / (map_avg_ms * 1e-3) / 1e12
    rows_per_launch = n_fill * s.n_late / max(map_n / args.steps, 1)
    map_launch_bytes = (rows_per_launch / n_fill) * (s.d_out * s.d_in + s.d_out) * 2 \
        + n_fill * s.d_in * 2 + rows_per_launch * s.d_out * 2
    kv_tflops = n_fill * s.n_late * f_kv * args.steps / (kv_ms * 1e-3) / 1e12 if kv_ms else None
    kernels = {k: {"ms_per_step": v[0] / args.steps, "launches_per_step": v[1] / args.steps}
               for k, v in prof.items() if v[1]}
    log(f"[bench] {name}: {ms:.3f} ms/step (median {np.median(per_step):.3f}, min {min(per_step):.3f}), "
        f"map {map_avg_ms:.3f} ms/launch ({map_tflops:.0f} TFLOP/s), kv {kv_tflops and round(kv_tflops)} TFLOP/s")

    default_config = args.spans is None and g == GROUP[name] and not q8 and not args.indexer \
        and not args.qk_norm and not args.value_rescale and not args.rope_per_call
    traffic = measured_traffic(name) if default_config else None
    res = {
        "value": n_fill / (ms * 1e-3),
        "unit": "rows/s",
        "ms_per_step": ms,
        "step_ms": {"mean": ms, "median": float(np.median(per_step)), "min": float(min(per_step)),
                    "max": float(max(per_step))},
        "config": {"workload": name, "d_in": s.d_in, "d_out": s.d_out, "late_layers": s.n_late,
                   "kv_heads": s.n_kv, "head_dim": s.head_dim, "rows": s.n_rows, "fill_rows": n_fill,
                   "prompts": list(s.prompt_lens), "maps": "pinned host, streamed" if host_maps else "HBM",
                   "map_format": "int8 + bf16 scale per 128 weights of a row" if q8 else "bf16",
                   "value_rescale_rows": args.value_rescale or None,
                   "value_measure": (None if not args.value_rescale else
                                     "rf_value_scales, then rf_fill" if args.separate_measure else "inside rf_fill"),
                   "qk_norm": bool(args.qk_norm),
                   "indexer_key_heads": args.indexer, "exact_spans": s.n_spans,
                   "layers_per_launch": min(g, B.RF_STREAM_GROUP) if host_maps else g,
                   "rope_table": ("built inside every rf_fill call" if args.rope_per_call else
                                  "built once per plan by rf_rope_table, outside the timed steps")},
        "tflops": step_flops / (ms * 1e-3) / 1e12,
        "frac_of_bf16_peak": step_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "mfma", "kernel": "map_gemm", "achieved": map_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": map_tflops / PEAK_BF16_TFLOPS,
                     "traffic": (traffic or {}).get("traffic_bytes_per_launch"),
                     "algorithmic_bytes_per_launch": map_launch_bytes,
                     "flops_per_launch": map_launch_flops, "ms_per_launch": map_avg_ms},
        "kernels": kernels,
        "kv_gemm_tflops": kv_tflops,
    }
    if host_maps and prof["copy"][1]:
        per_layer = s.d_out * s.d_in * (1 + 2 / workloads.Q8_BLOCK if q8 else 2) + s.d_out * 2
        h2d_bytes = s.n_late * per_layer
        copy_ms = prof["copy"][0] / args.steps
        ref = pinned_copy_rate(dev)
        gbs = h2d_bytes / (copy_ms * 1e-3) / 1e9
        res["h2d"] = {"bytes_per_step": h2d_bytes, "copy_ms_per_step": copy_ms, "gbs": gbs,
                      "pinned_copy_gbs": ref["gbs"], "frac_of_pinned_copy": gbs / ref["gbs"],
                      "pcie_inclusive_rows_per_s": n_fill / (ms * 1e-3),
                      "note": "maps and biases over PCIe on a side stream, overlapped with the kernels; "
                              "pinned_copy_gbs: plain 256 MiB pinned host->device copies in the same process"}
    if traffic is not None:
        hbm = traffic["bytes_per_step"]
        res["hbm"] = {"bytes_per_step": hbm, "gbs": hbm / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                      "frac": hbm / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      "source": os.path.relpath(traffic_path(name), ROOT),
                      "note": "copy-calibrated FETCH_SIZE + WRITE_SIZE of the library's kernels of one step "
                              "(what the L2 moves to and from the MALL or HBM), over the step time measured here"}
    if q8 and prof["dequant"][1]:
        dq_ms, dq_n = prof["dequant"]
        layers_per_dq = s.n_late * args.steps / dq_n
        dq_bytes = layers_per_dq * s.d_out * s.d_in * (1 + 2 + 2 / workloads.Q8_BLOCK)
        dq_avg = dq_ms / dq_n
        res["dequant_roofline"] = {"bound": "hbm", "kernel": "dequant", "achieved": dq_bytes / (dq_avg * 1e-3) / 1e9,
                                   "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": dq_bytes / (dq_avg * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                   "algorithmic_bytes_per_launch": dq_bytes, "ms_per_launch": dq_avg}
    if headline and not args.no_cpu_baseline:
        log(f"[bench] {name}: timing the fp64 oracle on a sample")
        f = np.setdiff1d(np.arange(s.n_rows), w.exact_rows).astype(np.int32)
        res["cpu_baseline"] = cpu_baseline(w, f, name)
    plan.close()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None, choices=workloads.CONFIG_ORDER,
                    help="measure only this workload (default: 27b_120k, plus the 8b, 27b and "
                         "8b_ragged_host workloads under extra.workloads)")
    ap.add_argument("--layers-per-launch", type=int, default=None)
    ap.add_argument("--value-rescale", type=int, default=0, metavar="C",
                    help="include the value rescale measured on the first C tail rows of each prompt")
    ap.add_argument("--qk-norm", action="store_true", help="layers normalise their keys per head before RoPE")
    ap.add_argument("--separate-measure", action="store_true",
                    help="with --value-rescale: measure with rf_value_scales, then fill (default: inside the fill)")
    ap.add_argument("--spans", type=int, default=None, metavar="N",
                    help="exact 32-row spans scattered in the first prompt's prefix (default: the workload's; "
                         "e.g. 1113 keeps 30%% of the 27b_120k prefix exact, the density of the pages' 27B runs)")
    ap.add_argument("--indexer", type=int, default=0, metavar="HEADS",
                    help="layers also write HEADS head_dim-wide indexer key heads (sparse-attention layers)")
    ap.add_argument("--maps", default="bf16", choices=["bf16", "q8"],
                    help="map storage: bf16, or int8 codes with one bf16 scale for each 128-weight block of a row")
    ap.add_argument("--rope-per-call", action="store_true",
                    help="let every rf_fill call build its RoPE table (default: one table per plan)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="measure the headline workload only")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after timing, copy MIB mebibytes device-to-device once (PMC calibration)")
    ap.add_argument("--blas-reference", action="store_true",
                    help="time torch.matmul (hipBLASLt) on the two contraction shapes of --workload and exit; "
                         "a reference point for the roofline, not part of the fill")
    ap.add_argument("--capture", type=int, default=0, metavar="ROWS",
                    help="time the device capture of the ridge sums (X^T X, X^T Y) on ROWS rows of --workload's "
                         "width and exit; a separate JSON line, not the fill")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CALIB_MIB", "STEPS"),
                    help="write the traffic summary of --workload from two rocprofv3 --pmc CSVs of a run of "
                         "STEPS steps (warm-up included) and exit")
    args = ap.parse_args()
    name = args.workload or "27b_120k"
    if args.pmc_summary:
        t = summarize_pmc(args.pmc_summary[0], args.pmc_summary[1], name, int(args.pmc_summary[2]) << 20,
                          int(args.pmc_summary[3]))
        os.makedirs(os.path.dirname(traffic_path(name)), exist_ok=True)
        with open(traffic_path(name), "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} asked): the fill runs on a single MI355X. "
              "Across GPUs it would shard by late layers or by rows, each GPU running this one-GPU path on "
              "its share.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.blas_reference:
        blas_reference(workloads.spec(name), args.steps)
        return
    if args.capture:
        capture_bench(workloads.spec(name), args.capture, args.steps, args.warmup)
        return

    res = run_workload(name, args, headline=True)
    extra = {}
    if args.workload is None and not args.no_extra:
        for sub in EXTRA_WORKLOADS:
            gc.collect()
            torch.cuda.empty_cache()
            r = run_workload(sub, args, headline=False)
            extra[sub] = r
    out = {
        "metric": "filled rows/s (all late layers)",
        "value": res["value"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
    }
    out.update({k: v for k, v in res.items() if k not in ("value", "unit", "ms_per_step")})
    if extra:
        out["extra"] = {"workloads": extra}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
