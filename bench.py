#!/usr/bin/env python3
"""Throughput of the late-layer cache fill on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole fill path over one batch of synthetic input:
rf_fill_rows (the fill-row set from the exact rows) and rf_fill (map
contraction, RMSNorm, K/V projections, RoPE and cache scatter for every late
layer; for the streamed workload also the host->device map copies).  Inputs
are resident in device memory (pinned host memory for streamed maps) before
the timed region starts.  W untimed steps, then K timed steps bracketed by
device synchronisation; one JSON line goes to stdout, progress to stderr.

``value`` is filled rows per second over all late layers.  The roofline entry
is the dominant kernel (the map contraction): algorithmic flops per launch,
2 d_in d_out per filled row per layer times the rows and layers one launch
processes, divided by its mean launch time from HIP events recorded around
every launch on the stream it runs on.  ``cpu_baseline`` is the fp64 numpy
oracle timed on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

import workloads

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0

# layers per launch used by the benchmark (divides the late-layer count)
GROUP = {"tiny": 4, "8b": 22, "27b": 6, "27b_120k": 6, "8b_ragged_host": 4}
# rows of the oracle's timed sample (None: every fill row), sized for 10-30 s
CPU_SAMPLE = {"tiny": None, "8b": 8192, "27b": 4096, "27b_120k": 4096, "8b_ragged_host": 8192}
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCE = os.path.join(ROOT, "late_layer_kv_amd", "csrc", "rf_kernels.hip")


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


def kernel_source_hash() -> str:
    import hashlib
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_path(name: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_map_gemm_{name}.json")


def measured_traffic(name: str):
    """HBM bytes per map_gemm launch from the PMC runs, if taken on this kernel source."""
    try:
        with open(traffic_path(name)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t["traffic_bytes_per_launch"] if t.get("kernel_source_sha256") == kernel_source_hash() else None


def summarize_pmc(fetch_csv: str, write_csv: str, name: str, calib_bytes: int) -> dict:
    """Traffic per launch from two rocprofv3 --pmc CSVs (FETCH_SIZE, WRITE_SIZE),
    each scaled by what the same counter reads for a device copy of known size."""
    import csv

    def per_kernel(path, counter):
        sums, n = {}, {}
        copy = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            k, v = r["Kernel_Name"], float(r["Counter_Value"])
            if "map_gemm" in k or "kv_gemm" in k:
                kk = "map_gemm" if "map_gemm" in k else "kv_gemm"
                sums[kk] = sums.get(kk, 0.0) + v
                n[kk] = n.get(kk, 0) + 1
            elif "copyBuffer" in k or "copy" in k.lower():
                copy.append((int(r["Grid_Size"]), v))
        copy_kib = max(copy)[1] if copy else None
        return {k: sums[k] / n[k] for k in sums}, copy_kib

    f, fc = per_kernel(fetch_csv, "FETCH_SIZE")
    w, wc = per_kernel(write_csv, "WRITE_SIZE")
    kf = calib_bytes / (fc * 1024.0) if fc else 1.0
    kw = calib_bytes / (wc * 1024.0) if wc else 1.0
    out = {"workload": name, "kernel_source_sha256": kernel_source_hash(),
           "copy_calibration": {"bytes": calib_bytes, "fetch_kib": fc, "write_kib": wc,
                                "fetch_factor": kf, "write_factor": kw},
           "kernels": {k: {"fetch_kib_per_launch": f[k], "write_kib_per_launch": w.get(k),
                           "bytes_per_launch": f[k] * 1024 * kf + w.get(k, 0.0) * 1024 * kw} for k in f},
           "source": {pmc: ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc " + pmc + " -f csv -d <out>/" + pmc.split("_")[0].lower()
                            + " -o " + pmc.split("_")[0].lower() + " -- python3 <repo>/bench.py --workload " + name
                            + " --steps 1 --warmup 1 --no-cpu-baseline --calibrate-copy " + str(calib_bytes >> 20))
                      for pmc in ("FETCH_SIZE", "WRITE_SIZE")}}
    out["source"]["summary"] = (f"python bench.py --workload {name} --pmc-summary <out>/fetch/fetch_counter_collection.csv "
                                f"<out>/write/write_counter_collection.csv {calib_bytes >> 20}")
    out["traffic_bytes_per_launch"] = out["kernels"]["map_gemm"]["bytes_per_launch"]
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


PEAK_FP64_TFLOPS = 78.6    # MI355X dense fp64 MFMA, published


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


def cpu_baseline(w, fill, name):
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:
        cores = os.cpu_count() or 1
    n = CPU_SAMPLE[name]
    rows = fill if n is None or n >= len(fill) else \
        np.sort(np.random.default_rng(0).choice(fill, size=n, replace=False)).astype(np.int32)
    t0 = time.perf_counter()
    oracle.fill_workload(w, rows=rows)
    dt = time.perf_counter() - t0
    return {"value": len(rows) / dt, "unit": "rows/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(rows)} fill rows x all {w.spec.n_late} late layers, fp64 numpy, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="27b_120k", choices=workloads.CONFIG_ORDER)
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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="after timing, copy MIB mebibytes device-to-device once (PMC calibration)")
    ap.add_argument("--blas-reference", action="store_true",
                    help="time torch.matmul (hipBLASLt) on the two contraction shapes of --workload and exit; "
                         "a reference point for the roofline, not part of the fill")
    ap.add_argument("--capture", type=int, default=0, metavar="ROWS",
                    help="time the device capture of the ridge sums (X^T X, X^T Y) on ROWS rows of --workload's "
                         "width and exit; a separate JSON line, not the fill")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "CALIB_MIB"),
                    help="write the traffic summary for --workload from two rocprofv3 --pmc CSVs and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        t = summarize_pmc(args.pmc_summary[0], args.pmc_summary[1], args.workload,
                          int(args.pmc_summary[2]) << 20)
        os.makedirs(os.path.dirname(traffic_path(args.workload)), exist_ok=True)
        with open(traffic_path(args.workload), "w") as f:
            json.dump(t, f, indent=1)
        print(json.dumps(t))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} asked): the fill runs on a single MI355X. "
              "Across GPUs it would shard by late layers or by rows, each GPU running this one-GPU path on "
              "its share.", file=sys.stderr)
        sys.exit(2)

    import torch
    from late_layer_kv_amd import binding as B

    if args.blas_reference:
        blas_reference(workloads.spec(args.workload), args.steps)
        return
    if args.capture:
        capture_bench(workloads.spec(args.workload), args.capture, args.steps, args.warmup)
        return

    name = args.workload
    s = workloads.spec(name, map_format=args.maps, qk_norm=args.qk_norm, idx_heads=args.indexer)
    if args.spans is not None:
        s = workloads.spec(name, map_format=args.maps, qk_norm=args.qk_norm, idx_heads=args.indexer,
                           n_spans=args.spans)
    q8 = args.maps == "q8"
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
    g = args.layers_per_launch or GROUP[name]
    ws = torch.empty(plan.fill_workspace_bytes(n_fill, g), dtype=torch.uint8, device=dev)
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
                B.fill_q8(plan, x, fill_rows, n_fill, positions, None, map_q, map_s, map_b, gamma, w_k, w_v, None,
                          kc, vc, ws, k_norm=k_norm, w_idx=w_idx, idx_cache=ic, measure=measure)
            else:
                B.fill(plan, x, fill_rows, n_fill, positions, None, map_a, map_b, gamma, w_k, w_v, None, kc, vc, ws,
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
            B.fill_q8(plan, x, fill_rows, n_fill, positions, None, map_q, map_s, map_b, gamma, w_k, w_v, None,
                      kc, vc, ws, vscale=vscale, k_norm=k_norm, w_idx=w_idx, idx_cache=ic)
        else:
            B.fill(plan, x, fill_rows, n_fill, positions, None, map_a, map_b, gamma, w_k, w_v, None, kc, vc, ws,
                   vscale=vscale, k_norm=k_norm, w_idx=w_idx, idx_cache=ic)

    log(f"[bench] {name}: n_fill={n_fill}, {s.n_late} late layers, {g} per launch; warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert int(n_fill_dev.item()) == n_fill

    log(f"[bench] {name}: timing {args.steps} steps")
    plan.profile(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    prof = plan.profile_read()
    plan.profile(False)
    if args.calibrate_copy:
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
    log(f"[bench] {name}: {ms:.3f} ms/step, map {map_avg_ms:.3f} ms/launch ({map_tflops:.0f} TFLOP/s), "
        f"kv {kv_tflops and round(kv_tflops)} TFLOP/s")

    out = {
        "metric": "filled rows/s (all late layers)",
        "value": n_fill / (ms * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "d_in": s.d_in, "d_out": s.d_out, "late_layers": s.n_late,
                   "kv_heads": s.n_kv, "head_dim": s.head_dim, "rows": s.n_rows, "fill_rows": n_fill,
                   "prompts": list(s.prompt_lens), "maps": "pinned host, streamed" if host_maps else "HBM",
                   "map_format": "int8 + bf16 scale per 128 weights of a row" if q8 else "bf16",
                   "value_rescale_rows": args.value_rescale or None,
                   "value_measure": (None if not args.value_rescale else
                                     "rf_value_scales, then rf_fill" if args.separate_measure else "inside rf_fill"),
                   "qk_norm": bool(args.qk_norm),
                   "indexer_key_heads": args.indexer, "exact_spans": s.n_spans,
                   "layers_per_launch": min(g, B.RF_STREAM_GROUP) if host_maps else g},
        "tflops": step_flops / (ms * 1e-3) / 1e12,
        "frac_of_bf16_peak": step_flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "mfma", "kernel": "map_gemm", "achieved": map_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": map_tflops / PEAK_BF16_TFLOPS,
                     # the counters were taken on the default configuration of the workload
                     "traffic": (measured_traffic(name) if args.spans is None and g == GROUP[name] else None),
                     "algorithmic_bytes_per_launch": map_launch_bytes,
                     "flops_per_launch": map_launch_flops, "ms_per_launch": map_avg_ms},
        "kernels": kernels,
        "kv_gemm_tflops": kv_tflops,
    }
    if host_maps and prof["copy"][1]:
        per_layer = s.d_out * s.d_in * (1 + 2 / workloads.Q8_BLOCK if q8 else 2) + s.d_out * 2
        h2d_bytes = s.n_late * per_layer
        copy_ms = prof["copy"][0] / args.steps
        out["h2d"] = {"bytes_per_step": h2d_bytes, "copy_ms_per_step": copy_ms,
                      "gbs": h2d_bytes / (copy_ms * 1e-3) / 1e9,
                      "note": "maps and biases over PCIe on a side stream, overlapped with the kernels"}
    if q8 and prof["dequant"][1]:
        dq_ms, dq_n = prof["dequant"]
        layers_per_dq = s.n_late * args.steps / dq_n
        dq_bytes = layers_per_dq * s.d_out * s.d_in * (1 + 2 + 2 / workloads.Q8_BLOCK)
        dq_avg = dq_ms / dq_n
        out["dequant_roofline"] = {"bound": "hbm", "kernel": "dequant", "achieved": dq_bytes / (dq_avg * 1e-3) / 1e9,
                                   "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": dq_bytes / (dq_avg * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                   "algorithmic_bytes_per_launch": dq_bytes, "ms_per_launch": dq_avg}
    if not args.no_cpu_baseline:
        log(f"[bench] {name}: timing the fp64 oracle on a sample")
        f = np.setdiff1d(np.arange(s.n_rows), w.exact_rows).astype(np.int32)
        out["cpu_baseline"] = cpu_baseline(w, f, name)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
