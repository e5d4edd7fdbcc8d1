"""GPU parity of the indexer keys (rf_fill_opts.w_idx / idx_cache).

In sparse-attention layers filled rows also write the indexer's keys
(RidgeFill section 2.1 and section 5.1: one 128-wide key head shared by the
indexer's query heads).  They are projected from the layer's normalised input
and rotated like the attention keys, without QK-norm.  Values against the
fp64 oracle to the fill's tolerance, placement bit-exact, and bitwise
identities: K/V do not change when indexer heads are added, an indexer head
with a key head's weights reproduces that key head, and an identity-map fill
equals the exact-row path.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from late_layer_kv_amd import binding as B
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

CASES = {
    # heads of 64: one indexer head is half of a 128-feature wave, the rest padding
    "tiny_idx": workloads.spec("tiny", idx_heads=1, seed=60),
    "tiny_idx3": workloads.spec("tiny", idx_heads=3, seed=61),
    "8b_mid_idx": workloads.spec("8b", n_late=3, prompt_lens=(700,), tail=60, idx_heads=1, seed=62),
    "27b_mid_q8_qk_idx": workloads.spec("27b_120k", n_late=2, prompt_lens=(1300,), tail=100, n_spans=4,
                                        map_format="q8", qk_norm=True, idx_heads=1, seed=63),
    "ragged_host_idx": workloads.spec("8b_ragged_host", n_late=2, prompt_lens=(300, 257, 129, 64), tail=50,
                                      idx_heads=2, seed=64),
    # the indexer columns end half way into a 256-feature tile: those 128
    # features go to the 512-row tall kernel (heads of 64: two heads; heads of
    # 128: a whole indexer tile plus the remainder, three tall tiles, the last
    # one ragged)
    "tiny_idx2_tall": workloads.spec("tiny", idx_heads=2, seed=65),
    "8b_mid_idx3_tall": workloads.spec("8b", n_late=2, prompt_lens=(1500,), tail=60, idx_heads=3, seed=66),
}

_cache = {}


def _workload(name):
    if name not in _cache:
        _cache[name] = workloads.make(CASES[name])
    return _cache[name]


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("name", list(CASES))
def test_indexer_fill_matches_oracle(name):
    w = _workload(name)
    s = w.spec
    _say(f"[idx fill] {name} hd={s.head_dim} heads={s.idx_heads} fmt={s.map_format} host={s.maps_on_host}")
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    rows, n = U.gpu_fill_rows(plan, di)
    kc, vc, ic = U.gpu_fill(plan, di, rows, n)
    f = rows.cpu().numpy()
    U.check_placement(kc, vc, f, s.n_rows, ic=ic)
    U.check_values(kc, vc, oracle.fill_workload(w, rows=f), f, s.head_dim)
    worst = U.check_indexer_values(ic, oracle.fill_indexer_workload(w, rows=f), f, s.head_dim)
    _say(f"[idx fill] {name} indexer worst {worst}")


@pytest.mark.parametrize("name", ["tiny_idx", "8b_mid_idx", "27b_mid_q8_qk_idx", "8b_mid_idx3_tall"])
def test_indexer_heads_leave_kv_unchanged(name):
    """The extra columns change nothing else: K and V are bitwise those of the
    same fill on a plan without indexer heads."""
    w = _workload(name)
    s = w.spec
    _say(f"[idx kv unchanged] {name}")
    di = U.DeviceInputs(w)
    rows, n = U.gpu_fill_rows(U.plan_for(w), di)
    k1, v1, _ = U.gpu_fill(U.plan_for(w), di, rows, n)
    plain = U.plan_for(w, n_idx=0)
    w_idx, di.w_idx = di.w_idx, None
    try:
        k2, v2 = U.gpu_fill(plain, di, rows, n)
    finally:
        di.w_idx = w_idx
    for l in range(s.n_late):
        assert torch.equal(k1[l], k2[l]) and torch.equal(v1[l], v2[l]), f"layer {l}"


@pytest.mark.parametrize("name", ["tiny_idx", "8b_mid_idx", "tiny_idx2_tall", "8b_mid_idx3_tall"])
def test_indexer_head_with_key_weights_equals_key_head(name):
    """An indexer head given the first key head's weights (layers without
    QK-norm) stores exactly that key head."""
    w = _workload(name)
    s = w.spec
    _say(f"[idx == key head] {name}")
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    rows, n = U.gpu_fill_rows(plan, di)
    hd = s.head_dim
    wi = [torch.cat([wk[:hd]] * s.idx_heads).contiguous() for wk in di.w_k]
    kc, vc, ic = U.gpu_fill(plan, di, rows, n, w_idx=wi)
    f = torch.from_numpy(rows.cpu().numpy().astype(np.int64)).to(kc[0].device)
    for l in range(s.n_late):
        k0 = kc[l].index_select(0, f)[:, :hd]
        for h in range(s.idx_heads):
            assert torch.equal(ic[l].index_select(0, f)[:, h * hd:(h + 1) * hd], k0), f"layer {l} head {h}"


@pytest.mark.parametrize("name", ["tiny_idx3", "8b_mid_idx", "tiny_idx2_tall", "8b_mid_idx3_tall"])
def test_indexer_identity_fill_equals_exact_projection(name):
    """Identity maps give the exact-row path's bytes, indexer keys included,
    and those match the oracle's exact indexer keys."""
    w = _workload(name)
    s = w.spec
    _say(f"[idx identity] {name}")
    di = U.DeviceInputs(w, maps_on_host=False)
    plan = U.plan_for(w, maps_on_host=False)
    rows, n = U.gpu_fill_rows(plan, di)
    a, b = U.identity_maps(di)
    k1, v1, i1 = U.gpu_fill(plan, di, rows, n, map_a=a, map_b=b)
    k2, v2, i2 = U.gpu_kv_project(plan, di, [di.x] * s.n_late, rows, n)
    for l in range(s.n_late):
        assert torch.equal(k1[l], k2[l]) and torch.equal(v1[l], v2[l]), f"layer {l}"
        assert torch.equal(i1[l], i2[l]), f"layer {l} indexer"
    f = rows.cpu().numpy()
    U.check_indexer_values(i2, oracle.exact_indexer_workload(w, w.x, f), f, s.head_dim)


@pytest.mark.parametrize("name", ["ragged_host_idx", "8b_mid_idx3_tall"])
def test_indexer_grouping_and_streaming_are_bitwise_neutral(name):
    """One layer per launch, all layers per launch and streamed maps give the
    same indexer bytes."""
    w = _workload(name)
    s = w.spec
    _say("[idx grouping]")
    dev = U.DeviceInputs(w, maps_on_host=False)
    plan = U.plan_for(w, maps_on_host=False)
    rows, n = U.gpu_fill_rows(plan, dev)
    _, _, i1 = U.gpu_fill(plan, dev, rows, n, layers_per_launch=1)
    _, _, i2 = U.gpu_fill(plan, dev, rows, n, layers_per_launch=s.n_late)
    host = U.DeviceInputs(w, maps_on_host=True)
    _, _, i3 = U.gpu_fill(U.plan_for(w, maps_on_host=True), host, rows, n)
    for l in range(s.n_late):
        assert torch.equal(i1[l], i2[l]) and torch.equal(i1[l], i3[l]), f"layer {l}"


def _tall_case(n_rows, tail, seed):
    # d = 512 keeps the oracle cheap; 8 kv heads of 128 and one indexer head
    # make 2176 columns: 8 regular feature tiles and a 128-wide remainder,
    # which takes the tall tiles of 512 rows
    return workloads.spec("8b", d_in=512, d_out=512, n_late=2, prompt_lens=(n_rows,), tail=tail, idx_heads=1,
                          seed=seed)


@pytest.mark.parametrize("n_fill", [1, 511, 512, 513])
def test_tall_tiles_around_their_512_row_edge(n_fill):
    """One row, and fills that end one row before, on and after a tall tile."""
    s = _tall_case(n_fill + 64, 64, 70 + n_fill % 97)
    w = workloads.make(s)
    _say(f"[tall edge] {n_fill} rows")
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    rows, n = U.gpu_fill_rows(plan, di)
    assert n == n_fill
    kc, vc, ic = U.gpu_fill(plan, di, rows, n)
    f = rows.cpu().numpy()
    U.check_placement(kc, vc, f, s.n_rows, ic=ic)
    U.check_values(kc, vc, oracle.fill_workload(w, rows=f), f, s.head_dim)
    U.check_indexer_values(ic, oracle.fill_indexer_workload(w, rows=f), f, s.head_dim)


def test_tall_tiles_with_a_slot_map_and_skipped_rows():
    """Tall tiles store at slot(row) under a scattered slot map into a cache
    of twice as many slots, and skip rows whose slot is out of range, like
    the regular tiles do."""
    s = _tall_case(1500, 60, 77)
    w = workloads.make(s)
    _say("[tall slots]")
    di = U.DeviceInputs(w)
    n_slots = 2 * s.n_rows
    plan = B.Plan(s.d_in, s.d_out, s.n_late, s.n_kv, s.head_dim, s.rms_eps, s.rope_theta, s.n_rows, n_slots,
                  s.max_pos, n_idx=s.idx_heads)
    rows, n = U.gpu_fill_rows(plan, di)
    f = rows.cpu().numpy()
    slots = np.random.default_rng(7).permutation(n_slots)[: s.n_rows].astype(np.int32)
    bad = f[::37]
    slots[bad] = n_slots + 5          # out of range: these rows are not stored
    mk = lambda width: [torch.full((n_slots, width), U.CANARY, dtype=torch.int16, device="cuda:0")
                        for _ in range(s.n_late)]
    kc, vc, ic = U.gpu_fill(plan, di, rows, n, caches=(mk(s.kv_width), mk(s.kv_width)),
                            idx_caches=mk(s.idx_heads * s.head_dim), slots=U.i32(slots).cuda())
    kept = np.setdiff1d(f, bad)
    U.check_placement(kc, vc, kept, n_slots, slots=slots, ic=ic)
    U.check_values(kc, vc, oracle.fill_workload(w, rows=kept), kept, s.head_dim, slots=slots)
    U.check_indexer_values(ic, oracle.fill_indexer_workload(w, rows=kept), kept, s.head_dim, slots=slots)
