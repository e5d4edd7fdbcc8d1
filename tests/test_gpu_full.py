"""GPU parity at the full sizes of the five workloads, in the launch
configuration the benchmark times (all late layers, the benchmark's layers per
launch).

Placement is checked bit-exactly on every row and layer.  Values are checked
against the fp64 oracle:
  * on every fill row of the tiny, 8B-shaped and ragged 8B-shaped workloads;
  * on the 27B-shaped workloads, on at least 4,096 rows: one row from every
    256-row tile of the fill index (its offset stepping through the tile, so
    every 16-row block and both row halves of the tile are met across tiles),
    the first and last fill rows, the rows on both sides of every exact span
    and prompt boundary, the largest positions, and seeded random rows.
The 120K workload also runs with 30% of its prefix exact in 1,113 spans and
an indexer head (a ragged last tile).  The deployed 27B configuration of the
pages (int8 maps and the value rescale
on the first 512 tail rows, RidgeFill sections 2.3 and 4.2) runs at the 120K
size with the measurement inside the fill.  Each case prints how many rows it
checked; the session's summary lists them (tests/conftest.py).  The 120K
fill is also checked bitwise against itself: rerun, one layer per launch,
and filled in two interleaved halves.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import workloads
from late_layer_kv_amd import binding as B
from tests import gpu_util as U

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

BENCH_GROUP = bench.GROUP  # layers per launch that bench.py times
TILE = 256                 # rows of one output tile of both contractions
SCALE_RTOL = 1e-3          # value scales, as in tests/test_gpu_rescale.py


def _say(*a):
    print(*a, flush=True)


def sample_rows(fill: np.ndarray, exact: np.ndarray, positions: np.ndarray, n_min: int = 4096, seed: int = 0):
    """Rows of `fill` to value-check at full size (see the module docstring)."""
    fset = set(fill.tolist())
    pick = {int(fill[0]), int(fill[-1])}
    n_tiles = (len(fill) + TILE - 1) // TILE
    for t in range(n_tiles):
        i = t * TILE + (t * 37 + 11) % TILE   # 37 is odd: the offsets run through every residue mod 256
        pick.add(int(fill[min(i, len(fill) - 1)]))
    edges = set()
    for r in np.asarray(exact):
        edges.update((int(r) - 1, int(r) + 1))
    starts = np.flatnonzero(positions == 0)
    edges.update(starts.tolist())
    edges.update((starts - 1).tolist())
    pick.update(r for r in edges if r in fset)
    order = np.argsort(positions[fill])
    pick.update(int(r) for r in fill[order[-4:]])
    g = np.random.default_rng(seed)
    rest = np.setdiff1d(fill, np.fromiter(pick, dtype=np.int64))
    need = max(0, n_min - len(pick))
    pick.update(int(r) for r in g.choice(rest, size=min(need, len(rest)), replace=False))
    return np.array(sorted(pick), dtype=np.int32)


# (workload, map format, QK-norm, indexer heads, rows checked: "all" or a
# minimum, exact spans: None for the workload's own)
FULL_CASES = [
    ("tiny", "bf16", False, 0, "all", None),
    ("8b", "bf16", False, 0, "all", None),
    ("27b", "bf16", False, 0, 4096, None),
    ("27b_120k", "bf16", False, 0, 4096, None),
    ("8b_ragged_host", "bf16", False, 0, "all", None),
    ("27b_120k", "q8", False, 0, 4096, None),
    ("8b_ragged_host", "q8", False, 0, "all", None),
    ("27b", "bf16", True, 0, 4096, None),
    ("27b_120k", "bf16", False, 1, 4096, None),
    # 30% of the prefix kept exact in 1,113 scattered spans, as the pages'
    # 27B runs keep 28-31%: 83,168 fill rows, so the last 256-row tile holds
    # 224 rows and the last tall indexer tile covers one row tile
    ("27b_120k", "bf16", False, 1, 4096, 1113),
]


def _check_layers(name, w, caches, rows, idx: bool, rescale=None):
    """Oracle layer by layer on `rows` against the caches; returns the worst errors."""
    s = w.spec
    chk = U.ValueCheck(s.head_dim)
    for l in range(s.n_late):
        if rescale is None:
            k, v = oracle.fill_workload(w, rows=rows, layers=[l])[l]
        else:
            scales, g_of_row = rescale
            k, v = oracle.fill_workload_rescaled(w, scales, g_of_row, rows, layers=[l])[l]
        ref = {"K": k, "V": v}
        if idx:
            ref["I"] = oracle.fill_indexer_workload(w, rows=rows, layers=[l])[l]
        chk.add(caches, {l: ref}, rows)
        if l % 8 == 7 or l == s.n_late - 1:
            _say(f"[full] {name}: layers 0..{l} checked on {len(rows)} rows")
    return chk.finish()


def _record(label, checked, n_fill, n_late, worst):
    line = (f"{label}: {checked} of {n_fill} fill rows ({100.0 * checked / n_fill:.1f}%) x {n_late} layers, "
            f"worst Frobenius {worst['fro']:.2e}, floored max {worst['maxel']:.2e}")
    U.RECORDS.append(line)
    _say(f"[full] {line}")


@pytest.mark.parametrize("name,fmt,qk,idx,checked,spans", FULL_CASES,
                         ids=[f"{n}-{f}{'-qk' if q else ''}{'-idx' if i else ''}{f'-spans{sp}' if sp else ''}"
                              for n, f, q, i, _, sp in FULL_CASES])
def test_full_size(name, fmt, qk, idx, checked, spans):
    over = {} if spans is None else {"n_spans": spans}
    s = workloads.spec(name, map_format=fmt, qk_norm=qk, idx_heads=idx, **over)
    _say(f"[full] {name} ({fmt} maps{', QK-norm' if qk else ''}{', indexer keys' if idx else ''}"
         f"{f', {spans} exact spans' if spans else ''}): generating inputs")
    w = workloads.make(s)
    di = U.DeviceInputs(w)
    plan = B.Plan.for_spec(s)
    _say(f"[full] {name}: rf_fill_rows + rf_fill on the GPU")
    rows, n = U.gpu_fill_rows(plan, di)
    f = rows.cpu().numpy()
    assert np.array_equal(f, oracle.fill_row_set(s.n_rows, w.exact_rows))
    out = U.gpu_fill(plan, di, rows, n, layers_per_launch=BENCH_GROUP[name])
    kc, vc = out[:2]
    ic = out[2] if idx else None
    _say(f"[full] {name}: placement over {s.n_late} layers x {s.n_rows} slots")
    U.check_placement(kc, vc, f, s.n_rows, ic=ic)
    rs = f if checked == "all" else sample_rows(f, w.exact_rows, w.positions, n_min=checked)
    _say(f"[full] {name}: oracle on {len(rs)} rows x {s.n_late} layers")
    caches = {"K": kc, "V": vc}
    if idx:
        caches["I"] = ic
    worst = _check_layers(name, w, caches, rs, bool(idx))
    _record(f"{name} {fmt}{' qk-norm' if qk else ''}{' indexer' if idx else ''}{f' {spans} spans' if spans else ''}",
            len(rs), len(f), s.n_late, worst)


def test_full_size_deployed_27b_q8_value_rescale():
    """The 27B deployment of the pages at the 120K size: int8 maps, the value
    rescale measured on the first c = 512 tail rows inside the fill (RidgeFill
    sections 2.3 and 4.2).  Scales against the oracle's to a relative 1e-3;
    the rescaled caches against the oracle's rescaled fill (computed with the
    oracle's scales) to the fill tolerance; placement on every row."""
    name, c = "27b_120k", 512
    s = workloads.spec(name, map_format="q8")
    _say(f"[full] {name} deployed (q8 maps, value rescale c={c}): generating inputs")
    w = workloads.make(s)
    c_rows, c_grp = workloads.calibration_row_list(s, c)
    truth = workloads.make_layer_truth(s, len(c_rows), outliers=w.outlier_channels)
    di = U.DeviceInputs(w)
    plan = B.Plan.for_spec(s)
    rows, n = U.gpu_fill_rows(plan, di)
    f = rows.cpu().numpy()
    ng = len(s.prompt_lens)
    g_of_row = workloads.prompt_of_row(s)
    sc = torch.full((s.n_late, ng, s.n_kv), -7.0, dtype=torch.float32, device="cuda:0")
    g = BENCH_GROUP[name]
    mws = torch.empty(plan.value_scales_workspace_bytes(len(c_rows), g), dtype=torch.uint8, device="cuda:0")
    measure = ([U.t16(t).cuda() for t in truth], U.i32(c_rows).cuda(), U.i32(c_grp).cuda(),
               U.i32(g_of_row).cuda(), ng, sc, mws)
    _say(f"[full] {name} deployed: rf_fill_q8 with the in-fill measurement")
    kc, vc = U.gpu_fill(plan, di, rows, n, layers_per_launch=g, measure=measure)
    U.check_placement(kc, vc, f, s.n_rows)
    ref_scales = oracle.value_scales(w, truth, c_rows, c_grp, ng)
    got = sc.cpu().numpy().astype(np.float64)
    for l in range(s.n_late):
        err = np.max(np.abs(got[l] - ref_scales[l]) / np.abs(ref_scales[l]))
        assert err <= SCALE_RTOL, f"layer {l}: scale relative error {err:.2e}"
    spread = max(float(np.max(np.abs(ref_scales[l] - 1.0))) for l in ref_scales)
    _say(f"[full] {name} deployed: scales within {SCALE_RTOL} of the oracle; max |scale - 1| = {spread:.3f}")
    rs = sample_rows(f, w.exact_rows, w.positions, n_min=4096, seed=1)
    worst = _check_layers(f"{name} deployed", w, {"K": kc, "V": vc}, rs, False, rescale=(ref_scales, g_of_row))
    _record(f"{name} q8 + value rescale c={c} (measured in the fill)", len(rs), len(f), s.n_late, worst)


def test_full_size_bitwise_rerun_grouping_and_row_split():
    """The 27B-shaped 120K fill in the benchmark's configuration, bitwise: a
    second identical call, one layer per launch instead of six, and the fill
    rows split in two halves that interleave 64-row runs (so every 256-row
    tile holds other rows than before) all give the same caches."""
    name = "27b_120k"
    s = workloads.spec(name)
    _say(f"[full] {name}: bitwise rerun, grouping and row split")
    w = workloads.make(s)
    di = U.DeviceInputs(w)
    plan = B.Plan.for_spec(s)
    rows, n = U.gpu_fill_rows(plan, di)
    g = BENCH_GROUP[name]
    ref = U.gpu_fill(plan, di, rows, n, layers_per_launch=g)

    def same(out, what):
        for l in range(s.n_late):
            assert torch.equal(ref[0][l], out[0][l]) and torch.equal(ref[1][l], out[1][l]), f"{what}: layer {l}"
        _say(f"[full] {name}: {what} bitwise equal")

    same(U.gpu_fill(plan, di, rows, n, layers_per_launch=g), "second call")
    same(U.gpu_fill(plan, di, rows, n, layers_per_launch=1), "one layer per launch")
    f = rows.cpu().numpy()
    run = (np.arange(len(f)) // 64) % 2 == 0
    a = torch.from_numpy(f[run].copy()).cuda()
    b = torch.from_numpy(f[~run].copy()).cuda()
    caches = di.caches()
    U.gpu_fill(plan, di, a, a.numel(), caches=caches, layers_per_launch=g)
    same(U.gpu_fill(plan, di, b, b.numel(), caches=caches, layers_per_launch=g), "two interleaved halves")
