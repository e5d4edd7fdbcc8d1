"""GPU parity at the edges of the shapes the library accepts.

The map contraction runs ceil(d_in / 64) stages of 64 columns, with separate
code for one, two and three stages; the tiles have 256 rows, so fills of 1,
255, 256 and 257 rows sit on and around a tile edge; d_in and d_out may
differ (the map is d_out x d_in).  Values against the fp64 oracle to the
fill's tolerance, placement bit-exact.  The last case turns every option of
the fill on at once.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from late_layer_kv_amd import binding as B
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _check(s, tag):
    print(f"[edges] {tag}: d_in={s.d_in} d_out={s.d_out} rows={s.n_rows} tail={s.tail}", flush=True)
    w = workloads.make(s)
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    rows, n = U.gpu_fill_rows(plan, di)
    f = rows.cpu().numpy()
    assert n == s.n_rows - len(np.unique(w.exact_rows))
    kc, vc = U.gpu_fill(plan, di, rows, n)
    U.check_placement(kc, vc, f, s.n_rows)
    worst = U.check_values(kc, vc, oracle.fill_workload(w, rows=f), f, s.head_dim)
    print(f"[edges] {tag}: worst {worst}", flush=True)


@pytest.mark.parametrize("d_in", [64, 128, 192, 320, 448])
def test_map_depths(d_in):
    """1, 2, 3, 5 and 7 stages of the map's main loop (d_in != d_out)."""
    _check(workloads.spec("tiny", d_in=d_in, n_late=2, prompt_lens=(300,), tail=40, seed=80 + d_in // 64),
           f"depth {d_in // 64}")


def test_wider_output_than_input():
    """d_out = 512 > d_in = 256: the identity on the leading diagonal of the map,
    two feature tiles per row in the key/value contraction's input."""
    _check(workloads.spec("tiny", d_in=256, d_out=512, n_late=2, prompt_lens=(300,), tail=40, seed=90),
           "d_out > d_in")


@pytest.mark.parametrize("n_fill", [1, 255, 256, 257])
def test_fills_around_a_tile_edge(n_fill):
    """One row, and fills that end one row before, on and after a 256-row tile."""
    _check(workloads.spec("tiny", n_late=2, prompt_lens=(n_fill + 64,), tail=64, seed=100 + n_fill),
           f"{n_fill} rows")


@pytest.mark.parametrize("d_in", [128, 384])
def test_int8_map_depths(d_in):
    """Int8 maps at one and three 128-column scale blocks (2 and 6 stages)."""
    _check(workloads.spec("tiny", d_in=d_in, n_late=2, prompt_lens=(300,), tail=40, map_format="q8",
                          seed=95 + d_in // 128), f"q8 depth {d_in // 64}")


def test_every_option_in_one_call():
    """Streamed int8 maps, QK-norm, one indexer head, the value measurement
    inside the fill, a slot mapping and a table from rf_rope_table, all in one
    fill of a ragged four-request batch: scales against the oracle's to 1e-3,
    K (normalised per head), rescaled V and the indexer keys against the
    oracle to the fill's tolerance, placement bit-exact at the mapped slots."""
    s = workloads.spec("8b_ragged_host", n_late=2, prompt_lens=(300, 257, 129, 64), tail=50,
                       map_format="q8", qk_norm=True, idx_heads=1, seed=70)
    c = 32
    print(f"[edges] all options: host={s.maps_on_host} fmt={s.map_format} c={c}", flush=True)
    w = workloads.make(s)
    rows_c, grp_c = workloads.calibration_row_list(s, c)
    truth = workloads.make_layer_truth(s, len(rows_c), outliers=w.outlier_channels)
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    fr, n = U.gpu_fill_rows(plan, di)
    f = fr.cpu().numpy()
    slots = np.random.default_rng(9).permutation(s.n_rows).astype(np.int32)
    table = torch.empty((s.max_pos, s.head_dim // 2, 2), dtype=torch.float32, device="cuda:0")
    B.rope_table(plan, table)
    ng = len(s.prompt_lens)
    g_of_row = workloads.prompt_of_row(s)
    sc = torch.full((s.n_late, ng, s.n_kv), -7.0, dtype=torch.float32, device="cuda:0")
    mws = torch.empty(plan.value_scales_workspace_bytes(len(rows_c), s.n_late), dtype=torch.uint8, device="cuda:0")
    measure = ([U.t16(t).cuda() for t in truth], U.i32(rows_c).cuda(), U.i32(grp_c).cuda(),
               U.i32(g_of_row).cuda(), ng, sc, mws)
    kc, vc, ic = U.gpu_fill(plan, di, fr, n, slots=U.i32(slots).cuda(), rope=table, measure=measure)
    U.check_placement(kc, vc, f, s.n_rows, slots=slots, ic=ic)
    ref_scales = oracle.value_scales(w, truth, rows_c, grp_c, ng)
    got = sc.cpu().numpy().astype(np.float64)
    for l in range(s.n_late):
        err = np.max(np.abs(got[l] - ref_scales[l]) / np.abs(ref_scales[l]))
        assert err <= 1e-3, f"layer {l}: scale relative error {err:.2e}"
    U.check_values(kc, vc, oracle.fill_workload_rescaled(w, ref_scales, g_of_row, f), f, s.head_dim, slots=slots)
    worst = U.check_indexer_values(ic, oracle.fill_indexer_workload(w, rows=f), f, s.head_dim, slots=slots)
    print(f"[edges] all options: indexer worst {worst}", flush=True)


def test_dense_scattered_exact_spans():
    """About 30% of the prefix kept exact as scattered 32-row spans (the
    density of the pages' 27B runs): the fill gathers the remaining rows
    across many short runs."""
    s = workloads.spec("27b_120k", n_late=2, prompt_lens=(1300,), tail=100, n_spans=12, seed=110)
    _check(s, "30% scattered exact rows")


def test_widest_launch_group():
    """33 late layers with a workspace for all of them: one launch of the
    library's maximum of 32 layers, then one of a single layer."""
    s = workloads.spec("tiny", n_late=33, prompt_lens=(300,), tail=40, seed=120)
    print(f"[edges] widest group: L={s.n_late}", flush=True)
    w = workloads.make(s)
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    rows, n = U.gpu_fill_rows(plan, di)
    assert plan.fill_workspace_bytes(n, 33) == plan.fill_workspace_bytes(n, 32)
    kc, vc = U.gpu_fill(plan, di, rows, n, layers_per_launch=33)
    f = rows.cpu().numpy()
    U.check_placement(kc, vc, f, s.n_rows)
    U.check_values(kc, vc, oracle.fill_workload(w, rows=f), f, s.head_dim)
    k1, v1 = U.gpu_fill(plan, di, rows, n, layers_per_launch=1)
    for l in range(s.n_late):
        assert torch.equal(kc[l], k1[l]) and torch.equal(vc[l], v1[l]), f"layer {l}"


def test_prompt_that_is_all_exact():
    """A ragged batch whose second prompt is shorter than the tail: all its
    rows are exact, none is filled, its slots stay untouched."""
    _check(workloads.spec("8b_ragged_host", n_late=2, prompt_lens=(300, 40, 129), tail=50, seed=130),
           "a prompt with no filled rows")


def test_cache_larger_than_the_batch():
    """n_slots = 3 x n_rows, rows scattered to distinct slots anywhere in the
    cache: only those slots are written, with the oracle's values."""
    s = workloads.spec("tiny", n_late=2, prompt_lens=(300,), tail=40, seed=140)
    print(f"[edges] cache of {3 * s.n_rows} slots for {s.n_rows} rows", flush=True)
    w = workloads.make(s)
    di = U.DeviceInputs(w)
    n_slots = 3 * s.n_rows
    plan = B.Plan(s.d_in, s.d_out, s.n_late, s.n_kv, s.head_dim, s.rms_eps, s.rope_theta, s.n_rows, n_slots,
                  s.max_pos)
    rows, n = U.gpu_fill_rows(plan, di)
    slots = np.random.default_rng(7).choice(n_slots, s.n_rows, replace=False).astype(np.int32)
    mk = lambda: [torch.full((n_slots, s.kv_width), U.CANARY, dtype=torch.int16, device="cuda:0")
                  for _ in range(s.n_late)]
    kc, vc = U.gpu_fill(plan, di, rows, n, caches=(mk(), mk()), slots=U.i32(slots).cuda())
    f = rows.cpu().numpy()
    U.check_placement(kc, vc, f, n_slots, slots=slots)
    U.check_values(kc, vc, oracle.fill_workload(w, rows=f), f, s.head_dim, slots=slots)


def test_no_exact_rows():
    """An empty exact set (no tail, no spans): every row of a ragged batch is
    filled, each at its own prompt's positions (RidgeFill section 2.1 with a
    zero tail; rf_fill_rows given no exact rows)."""
    _check(workloads.spec("8b_ragged_host", n_late=2, prompt_lens=(300, 257, 129), tail=0, seed=150),
           "no exact rows")
