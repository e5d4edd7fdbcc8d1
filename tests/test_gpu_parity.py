"""GPU parity: librf against the fp64 oracle, element by element.

Sizes here keep the oracle to seconds while spanning several 256-row tiles,
every feature tile and a ragged last tile.  Full-size workloads are in
test_gpu_full.py.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from late_layer_kv_amd import binding as B
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

# Parity-sized cases with the shapes and value distributions of the five
# workloads (fewer rows and layers), plus the tiny-distribution reading of the
# larger shapes.
CASES = {
    "tiny": workloads.spec("tiny"),
    "tiny_8b_values": workloads.spec("tiny", map_sigma=0.01, n_outliers=4, seed=10),
    "8b_mid": workloads.spec("8b", n_late=3, prompt_lens=(700,), tail=60, seed=11),
    "27b_mid_spans": workloads.spec("27b_120k", n_late=2, prompt_lens=(1300,), tail=100, n_spans=4, seed=12),
    "27b_mid_tiny_values": workloads.spec("27b", n_late=2, prompt_lens=(600,), tail=64, map_sigma=0.02,
                                          n_outliers=0, seed=13),
    "ragged_mid": workloads.spec("8b_ragged_host", n_late=2, prompt_lens=(300, 257, 129, 64), tail=50, seed=14),
}

_cache = {}


def _workload(name):
    if name not in _cache:
        _cache[name] = workloads.make(CASES[name])
    return _cache[name]


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("name", list(CASES))
def test_fill_rows_match_oracle(name):
    w = _workload(name)
    s = w.spec
    _say(f"[fill_rows] {name} n_rows={s.n_rows} n_exact={len(w.exact_rows)}")
    di = U.DeviceInputs(w, maps_on_host=False)
    plan = U.plan_for(w, maps_on_host=False)
    rows, n = U.gpu_fill_rows(plan, di)
    ref = oracle.fill_row_set(s.n_rows, w.exact_rows)
    assert n == len(ref)
    assert np.array_equal(rows.cpu().numpy(), ref)


@pytest.mark.parametrize("name", ["27b_120k", "8b_ragged_host"])
def test_fill_rows_full_size_exact_sets(name):
    """The full-size exact sets (tail of each prompt, 64 scattered spans), given
    shuffled and with duplicates; only row indices, so no data is drawn."""
    s = workloads.spec(name)
    e = workloads.exact_row_list(s)
    g = np.random.default_rng(5)
    shuffled = np.concatenate([e, e[: len(e) // 3]])
    g.shuffle(shuffled)
    _say(f"[fill_rows full] {name} n_rows={s.n_rows} n_exact_given={len(shuffled)}")
    plan = B.Plan.for_spec(s, maps_on_host=False)
    out = torch.full((s.n_rows,), -7, dtype=torch.int32, device="cuda:0")
    nf = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    ws = torch.empty(B.fill_rows_workspace_bytes(s.n_rows), dtype=torch.uint8, device="cuda:0")
    B.fill_rows(plan, U.i32(shuffled).cuda(), out, nf, ws)
    torch.cuda.synchronize()
    ref = oracle.fill_row_set(s.n_rows, e)
    assert int(nf.item()) == len(ref)
    assert np.array_equal(out[: len(ref)].cpu().numpy(), ref)
    assert torch.all(out[len(ref):] == -7)


@pytest.mark.parametrize("name", list(CASES))
def test_fill_matches_oracle(name):
    w = _workload(name)
    s = w.spec
    _say(f"[fill] {name} d_in={s.d_in} d_out={s.d_out} L={s.n_late} kv={s.n_kv}x{s.head_dim} rows={s.n_rows}")
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    rows, n = U.gpu_fill_rows(plan, di)
    kc, vc = U.gpu_fill(plan, di, rows, n)
    f = rows.cpu().numpy()
    U.check_placement(kc, vc, f, s.n_rows)
    ref = oracle.fill_workload(w, rows=f)
    worst = U.check_values(kc, vc, ref, f, s.head_dim)
    _say(f"[fill] {name} worst {worst}")


@pytest.mark.parametrize("name", ["tiny", "8b_mid"])
def test_identity_fill_equals_exact_projection(name):
    """Identity fill (A = I, b = 0; POP's fill) gives the same bytes as the
    exact layer write rf_kv_project from the same input, and both match the
    oracle's exact-layer K/V."""
    w = _workload(name)
    s = w.spec
    _say(f"[identity] {name}")
    di = U.DeviceInputs(w, maps_on_host=False)
    plan = U.plan_for(w, maps_on_host=False)
    rows, n = U.gpu_fill_rows(plan, di)
    a, b = U.identity_maps(di)
    kc1, vc1 = U.gpu_fill(plan, di, rows, n, map_a=a, map_b=b)
    kc2, vc2 = U.gpu_kv_project(plan, di, [di.x] * s.n_late, rows, n)
    for l in range(s.n_late):
        assert torch.equal(kc1[l], kc2[l]), f"K layer {l}"
        assert torch.equal(vc1[l], vc2[l]), f"V layer {l}"
    f = rows.cpu().numpy()
    ref = oracle.exact_kv_workload(w, w.x, f)
    U.check_values(kc2, vc2, ref, f, s.head_dim)


def _spread_rows(x: torch.Tensor, span: int) -> torch.Tensor:
    """x's rows copied into a strided view whose rows lie so far apart that
    n_rows * row stride covers about `span` bytes (row starts stay 16-byte
    aligned)."""
    n, d = x.shape
    ld = (span // (2 * n) + 64) // 8 * 8
    flat = torch.zeros((n - 1) * ld + d, dtype=x.dtype, device=x.device)
    v = torch.as_strided(flat, (n, d), (ld, 1))
    v.copy_(x)
    return v


WIDE_CASES = {
    "tiny": workloads.spec("tiny"),
    # one 128-wide indexer head over one kv head of 128: 384 K/V/indexer
    # columns, so compact inputs take tall tiles and the spread ones the
    # padded tile
    "tiny_idx": workloads.spec("tiny", n_kv=1, head_dim=128, idx_heads=1, seed=7),
}


@pytest.mark.parametrize("name,gib", [(n, g) for n in WIDE_CASES for g in (3, 4)])
def test_operands_spanning_4gib(name, gib):
    """An operand whose rows span 4 GiB or more is read through 64-bit
    pointers (the usual path reads through a buffer resource with 32-bit
    offsets, and tall indexer tiles are not used); one spanning 3 GiB stays
    on the usual path with a buffer size above 2^31 bytes.  Either way the
    fill with such a split-layer state, and rf_kv_project with such layer
    inputs, write the same bytes as with the compact layout."""
    w = workloads.make(WIDE_CASES[name])
    s = w.spec
    _say(f"[wide] {name}, rows spread over about {gib} GiB")
    di = U.DeviceInputs(w, maps_on_host=False)
    plan = U.plan_for(w, maps_on_host=False)
    rows, n = U.gpu_fill_rows(plan, di)
    fill1 = U.gpu_fill(plan, di, rows, n)
    proj1 = U.gpu_kv_project(plan, di, [di.x] * s.n_late, rows, n)
    compact = di.x
    di.x = _spread_rows(compact, gib << 30)
    span = di.x.stride(0) * s.n_rows * 2
    assert (span >= (1 << 32)) if gib >= 4 else ((1 << 31) < span < (1 << 32)), span
    fill2 = U.gpu_fill(plan, di, rows, n)
    proj2 = U.gpu_kv_project(plan, di, [di.x] * s.n_late, rows, n)
    di.x = None
    torch.cuda.empty_cache()
    for what, a, b in (("fill", fill1, fill2), ("rf_kv_project", proj1, proj2)):
        for cache, ca, cb in zip("KVI", a, b):
            for l in range(s.n_late):
                assert torch.equal(ca[l], cb[l]), f"{what}, {cache} cache, layer {l}"
    f = rows.cpu().numpy()
    U.check_values(fill1[0], fill1[1], oracle.fill_workload(w, rows=f), f, s.head_dim)


def test_streamed_maps_equal_resident():
    """Maps streamed from pinned host memory give the same bytes as resident maps."""
    w = _workload("ragged_mid")
    _say("[streamed] ragged_mid")
    res = U.DeviceInputs(w, maps_on_host=False)
    hst = U.DeviceInputs(w, maps_on_host=True)
    p_res = U.plan_for(w, maps_on_host=False)
    p_hst = U.plan_for(w, maps_on_host=True)
    rows, n = U.gpu_fill_rows(p_res, res)
    k1, v1 = U.gpu_fill(p_res, res, rows, n)
    k2, v2 = U.gpu_fill(p_hst, hst, rows, n)
    for l in range(w.spec.n_late):
        assert torch.equal(k1[l], k2[l]) and torch.equal(v1[l], v2[l]), f"layer {l}"


@pytest.mark.parametrize("fmt", ["bf16", "q8"])
def test_streamed_groups_equal_resident(fmt):
    """Six streamed layers go as groups of 1, RF_STREAM_GROUP and the rest
    (two device buffers of RF_STREAM_GROUP layers, used alternately, so the
    third group reuses the first buffer): the same bytes as resident maps in
    one launch and as one layer per launch, bf16 and int8; the workspace of a
    streamed plan stops growing at RF_STREAM_GROUP layers per launch."""
    assert B.RF_STREAM_GROUP < 5  # six layers make at least three groups
    s = workloads.spec("8b_ragged_host", n_late=6, prompt_lens=(300, 257, 129, 64), tail=50, map_format=fmt,
                       seed=15)
    _say(f"[streamed groups] {fmt} L={s.n_late}")
    w = workloads.make(s)
    res = U.DeviceInputs(w, maps_on_host=False)
    hst = U.DeviceInputs(w, maps_on_host=True)
    p_res = U.plan_for(w, maps_on_host=False)
    p_hst = U.plan_for(w, maps_on_host=True)
    rows, n = U.gpu_fill_rows(p_res, res)
    g = B.RF_STREAM_GROUP
    assert p_hst.fill_workspace_bytes(n, s.n_late) == p_hst.fill_workspace_bytes(n, g)
    assert p_hst.fill_workspace_bytes(n, g) > p_hst.fill_workspace_bytes(n, 1)
    k1, v1 = U.gpu_fill(p_res, res, rows, n)
    k2, v2 = U.gpu_fill(p_hst, hst, rows, n)
    k3, v3 = U.gpu_fill(p_hst, hst, rows, n, layers_per_launch=1)
    for l in range(s.n_late):
        assert torch.equal(k1[l], k2[l]) and torch.equal(v1[l], v2[l]), f"layer {l}"
        assert torch.equal(k1[l], k3[l]) and torch.equal(v1[l], v3[l]), f"layer {l} (one layer per launch)"


def test_layer_grouping_does_not_change_bytes():
    w = _workload("8b_mid")
    _say("[grouping] 8b_mid")
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    rows, n = U.gpu_fill_rows(plan, di)
    k1, v1 = U.gpu_fill(plan, di, rows, n, layers_per_launch=1)
    k3, v3 = U.gpu_fill(plan, di, rows, n, layers_per_launch=3)
    for l in range(w.spec.n_late):
        assert torch.equal(k1[l], k3[l]) and torch.equal(v1[l], v3[l])


def test_rerun_and_row_independence():
    """Two identical calls give identical caches, and filling A then B gives the
    same cache as filling A u B at once (a row's K/V depend on its own state only)."""
    w = _workload("tiny")
    _say("[determinism] tiny")
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    rows, n = U.gpu_fill_rows(plan, di)
    k1, v1 = U.gpu_fill(plan, di, rows, n)
    k2, v2 = U.gpu_fill(plan, di, rows, n)
    f = rows.cpu().numpy()
    a = torch.from_numpy(f[0::3].copy()).cuda()
    b = torch.from_numpy(np.setdiff1d(f, f[0::3]).astype(np.int32)).cuda()
    caches = di.caches()
    U.gpu_fill(plan, di, a, a.numel(), caches=caches)
    k3, v3 = U.gpu_fill(plan, di, b, b.numel(), caches=caches)
    for l in range(w.spec.n_late):
        assert torch.equal(k1[l], k2[l]) and torch.equal(v1[l], v2[l])
        assert torch.equal(k1[l], k3[l]) and torch.equal(v1[l], v3[l])


def test_empty_fill_leaves_cache_untouched():
    w = _workload("tiny")
    _say("[empty] tiny")
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    rows = torch.zeros(0, dtype=torch.int32, device="cuda:0")
    kc, vc = U.gpu_fill(plan, di, rows, 0)
    for c in kc + vc:
        assert torch.all(c == U.CANARY)


def test_slot_mapping_and_given_rope_table():
    """slot_of_row places each row's entry at its slot; a table from
    rf_rope_table gives the same bytes as the one rf_fill builds itself."""
    w = _workload("tiny")
    s = w.spec
    _say("[slots] tiny")
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    rows, n = U.gpu_fill_rows(plan, di)
    slots = np.random.default_rng(3).permutation(s.n_rows).astype(np.int32)
    sl = U.i32(slots).cuda()
    kc, vc = U.gpu_fill(plan, di, rows, n, slots=sl)
    f = rows.cpu().numpy()
    U.check_placement(kc, vc, f, s.n_rows, slots=slots)
    U.check_values(kc, vc, oracle.fill_workload(w, rows=f), f, s.head_dim, slots=slots)
    table = torch.empty((s.max_pos, s.head_dim // 2, 2), dtype=torch.float32, device="cuda:0")
    B.rope_table(plan, table)
    k2, v2 = U.gpu_fill(plan, di, rows, n, slots=sl, rope=table)
    for l in range(s.n_late):
        assert torch.equal(kc[l], k2[l]) and torch.equal(vc[l], v2[l])


def test_rope_table_matches_double_angles():
    s = workloads.spec("27b_120k")
    _say("[rope table] 27b_120k")
    plan = B.Plan.for_spec(s, maps_on_host=False)
    table = torch.empty((s.max_pos, s.head_dim // 2, 2), dtype=torch.float32, device="cuda:0")
    B.rope_table(plan, table)
    torch.cuda.synchronize()
    t = table.cpu().numpy().astype(np.float64)
    pos = np.array([0, 1, 2, 1000, 65535, 99999, s.max_pos - 1])
    ang = pos[:, None] * oracle.rope_inv_freq(s.head_dim, s.rope_theta)[None, :]
    assert np.max(np.abs(t[pos, :, 0] - np.cos(ang))) <= 6.0e-8
    assert np.max(np.abs(t[pos, :, 1] - np.sin(ang))) <= 6.0e-8


def test_validate_flag_reports_bad_rows():
    w = _workload("tiny")
    s = w.spec
    _say("[validate] tiny")
    di = U.DeviceInputs(w)
    plan = U.plan_for(w, validate=True)
    rows, n = U.gpu_fill_rows(plan, di)
    U.gpu_fill(plan, di, rows, n)  # valid rows pass
    bad = rows.flip(0).contiguous()
    with pytest.raises(B.RfError) as e:
        U.gpu_fill(plan, di, bad, n)
    assert e.value.status == -3
    oob = rows.clone()
    oob[5] = s.n_rows + 3
    with pytest.raises(B.RfError):
        U.gpu_fill(plan, di, oob, n)
