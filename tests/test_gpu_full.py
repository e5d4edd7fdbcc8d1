"""GPU parity at the full sizes of the five workloads, in the launch
configuration the benchmark times (all late layers, widest layer grouping the
benchmark's workspace allows).

Placement is checked bit-exactly on every row and layer.  Values are checked
against the fp64 oracle on sampled rows: the first and last fill rows, the rows
on both sides of every exact span and prompt boundary, the largest positions
and a seeded random sample.
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


def sample_rows(fill: np.ndarray, exact: np.ndarray, positions: np.ndarray, n: int = 96, seed: int = 0):
    fset = set(fill.tolist())
    pick = {int(fill[0]), int(fill[-1])}
    ex = np.asarray(exact)
    # neighbours of exact runs and of prompt starts
    edges = set()
    for r in ex:
        edges.update((int(r) - 1, int(r) + 1))
    edges.update(np.flatnonzero(positions == 0).tolist())
    edges.update((np.flatnonzero(positions == 0) - 1).tolist())
    pick.update(r for r in edges if r in fset)
    # largest positions among fill rows
    order = np.argsort(positions[fill])
    pick.update(int(r) for r in fill[order[-4:]])
    g = np.random.default_rng(seed)
    pick.update(int(r) for r in g.choice(fill, size=min(n, len(fill)), replace=False))
    return np.array(sorted(pick), dtype=np.int32)


FULL_CASES = [(n, "bf16", False, 0) for n in workloads.CONFIG_ORDER] + \
    [("27b_120k", "q8", False, 0), ("8b_ragged_host", "q8", False, 0), ("27b", "bf16", True, 0),
     ("27b_120k", "bf16", False, 1)]


@pytest.mark.parametrize("name,fmt,qk,idx", FULL_CASES,
                         ids=[f"{n}-{f}{'-qk' if q else ''}{'-idx' if i else ''}" for n, f, q, i in FULL_CASES])
def test_full_size(name, fmt, qk, idx):
    s = workloads.spec(name, map_format=fmt, qk_norm=qk, idx_heads=idx)
    print(f"[full] {name} ({fmt} maps{', QK-norm' if qk else ''}{', indexer keys' if idx else ''}): "
          "generating inputs", flush=True)
    w = workloads.make(s)
    di = U.DeviceInputs(w)
    plan = B.Plan.for_spec(s)
    print(f"[full] {name}: rf_fill_rows + rf_fill on the GPU", flush=True)
    rows, n = U.gpu_fill_rows(plan, di)
    f = rows.cpu().numpy()
    assert np.array_equal(f, oracle.fill_row_set(s.n_rows, w.exact_rows))
    out = U.gpu_fill(plan, di, rows, n, layers_per_launch=BENCH_GROUP[name])
    kc, vc = out[:2]
    ic = out[2] if idx else None
    print(f"[full] {name}: placement over {s.n_late} layers x {s.n_rows} slots", flush=True)
    U.check_placement(kc, vc, f, s.n_rows, ic=ic)
    rs = sample_rows(f, w.exact_rows, w.positions)
    print(f"[full] {name}: oracle on {len(rs)} sampled rows x {s.n_late} layers", flush=True)
    ref = oracle.fill_workload(w, rows=rs)
    worst = U.check_values(kc, vc, ref, rs, s.head_dim)
    print(f"[full] {name}: worst {worst}", flush=True)
    if idx:
        wi = U.check_indexer_values(ic, oracle.fill_indexer_workload(w, rows=rs), rs, s.head_dim)
        print(f"[full] {name}: indexer worst {wi}", flush=True)
