"""GPU parity of the value rescale (rf_value_scales, rf_fill's rf_vscale).

RidgeFill, section 2.3 ("Value rescale"); on for the 27B with c = 512
(section 4.2).  Scales are checked against the fp64 oracle to a relative
1e-3: each side's value vectors carry the fill's bf16 roundings (relative
error about 3e-3 per element), but a head norm over head_dim values and the
mean over c rows average them down by more than an order of magnitude.  The
rescaled fill is held to the fill's own tolerance against the oracle's
rescaled fill (oracle scales), and to bitwise identities.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from late_layer_kv_amd import binding as B
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

SCALE_RTOL = 1e-3

CASES = {
    # name: (spec, c)
    "tiny_ragged": (workloads.spec("tiny", prompt_lens=(200, 130, 80), tail=40, seed=40), 16),
    "8b_mid_two": (workloads.spec("8b", n_late=3, prompt_lens=(500, 330), tail=96, seed=41), 64),
    "27b_mid": (workloads.spec("27b", n_late=2, prompt_lens=(900,), tail=300, seed=42), 256),
    "27b_mid_q8": (workloads.spec("27b", n_late=2, prompt_lens=(900,), tail=300, map_format="q8", seed=43), 256),
    "ragged_host": (workloads.spec("8b_ragged_host", n_late=2, prompt_lens=(300, 257, 129, 64), tail=50,
                                   seed=44), 32),
    # six streamed layers: launch groups of 1, RF_STREAM_GROUP and the rest
    "ragged_host6": (workloads.spec("8b_ragged_host", n_late=6, prompt_lens=(300, 257, 129, 64), tail=50,
                                    map_format="q8", seed=45), 32),
}

_cache = {}


def _case(name):
    if name not in _cache:
        s, c = CASES[name]
        w = workloads.make(s)
        rows, grp = workloads.calibration_row_list(s, c)
        truth = workloads.make_layer_truth(s, len(rows), outliers=w.outlier_channels)
        _cache[name] = (w, rows, grp, truth)
    return _cache[name]


def _say(*a):
    print(*a, flush=True)


def gpu_scales(plan, di, rows, grp, truth_dev, n_groups, layers_per_launch=None):
    s = di.w.spec
    g = s.n_late if layers_per_launch is None else layers_per_launch
    out = torch.full((s.n_late, n_groups, s.n_kv), -5.0, dtype=torch.float32, device="cuda:0")
    ws = torch.empty(max(plan.value_scales_workspace_bytes(len(rows), g), 256), dtype=torch.uint8, device="cuda:0")
    r = U.i32(rows).cuda()
    gr = U.i32(grp).cuda()
    if di.q8:
        B.value_scales(plan, di.x, truth_dev, r, gr, n_groups, di.map_q, di.map_b, di.gamma, di.w_v, out, ws,
                       map_scale=di.map_scale)
    else:
        B.value_scales(plan, di.x, truth_dev, r, gr, n_groups, di.map_a, di.map_b, di.gamma, di.w_v, out, ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_value_scales_match_oracle(name):
    w, rows, grp, truth = _case(name)
    s = w.spec
    ng = len(s.prompt_lens)
    _say(f"[scales] {name} rows={len(rows)} groups={ng} host={s.maps_on_host} fmt={s.map_format}")
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    td = [U.t16(t).cuda() for t in truth]
    got = gpu_scales(plan, di, rows, grp, td, ng).cpu().numpy().astype(np.float64)
    ref = oracle.value_scales(w, truth, rows, grp, ng)
    for l in range(s.n_late):
        err = np.max(np.abs(got[l] - ref[l]) / np.abs(ref[l]))
        assert err <= SCALE_RTOL, f"layer {l}: scale relative error {err:.2e}\n{got[l]}\n{ref[l]}"
    spread = max(float(np.max(np.abs(ref[l] - 1.0))) for l in ref)
    _say(f"[scales] {name} max |scale - 1| = {spread:.3f}")


@pytest.mark.parametrize("name", ["tiny_ragged", "8b_mid_two", "27b_mid_q8", "ragged_host"])
def test_rescaled_fill_matches_oracle(name):
    """GPU scales into the GPU fill, against the oracle's scales in the oracle's fill."""
    w, rows, grp, truth = _case(name)
    s = w.spec
    ng = len(s.prompt_lens)
    _say(f"[rescaled fill] {name}")
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    td = [U.t16(t).cuda() for t in truth]
    sc = gpu_scales(plan, di, rows, grp, td, ng)
    g_of_row = workloads.prompt_of_row(s)
    fr, n = U.gpu_fill_rows(plan, di)
    kc, vc = U.gpu_fill(plan, di, fr, n, vscale=(sc, U.i32(g_of_row).cuda(), ng))
    f = fr.cpu().numpy()
    U.check_placement(kc, vc, f, s.n_rows)
    ref_scales = oracle.value_scales(w, truth, rows, grp, ng)
    ref = oracle.fill_workload_rescaled(w, ref_scales, g_of_row, f)
    worst = U.check_values(kc, vc, ref, f, s.head_dim)
    _say(f"[rescaled fill] {name} worst {worst}")


def test_unit_scales_leave_the_fill_unchanged():
    """All scales 1: the rescaled fill writes exactly the plain fill's bytes."""
    w, rows, grp, truth = _case("8b_mid_two")
    s = w.spec
    _say("[unit scales] 8b_mid_two")
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    fr, n = U.gpu_fill_rows(plan, di)
    ones = torch.ones((s.n_late, 2, s.n_kv), dtype=torch.float32, device="cuda:0")
    g_of_row = U.i32(workloads.prompt_of_row(s)).cuda()
    k1, v1 = U.gpu_fill(plan, di, fr, n)
    k2, v2 = U.gpu_fill(plan, di, fr, n, vscale=(ones, g_of_row, 2))
    for l in range(s.n_late):
        assert torch.equal(k1[l], k2[l]) and torch.equal(v1[l], v2[l]), f"layer {l}"


@pytest.mark.parametrize("name", ["tiny_ragged", "8b_mid_two"])
def test_true_equals_predicted_gives_unit_scales(name):
    """With identity maps (A = I, b = 0) the prediction is the split state
    itself; passing it as the true input makes both value vectors the same
    bytes, so every scale is exactly 1."""
    w, rows, grp, truth = _case(name)
    s = w.spec
    _say(f"[identity scales] {name}")
    di = U.DeviceInputs(w, maps_on_host=False)
    plan = U.plan_for(w, maps_on_host=False)
    a, b = U.identity_maps(di)
    di.map_a, di.map_b = a, b
    xr = U.t16(w.x[rows]).cuda()
    sc = gpu_scales(plan, di, rows, grp, [xr] * s.n_late, len(s.prompt_lens))
    assert torch.all(sc == 1.0), sc


def test_rows_outside_the_groups_are_skipped_and_streamed_equals_resident():
    w, rows, grp, truth = _case("ragged_host")
    s = w.spec
    _say("[groups / streamed] ragged_host")
    res = U.DeviceInputs(w, maps_on_host=False)
    hst = U.DeviceInputs(w, maps_on_host=True)
    p_res = U.plan_for(w, maps_on_host=False)
    p_hst = U.plan_for(w, maps_on_host=True)
    td = [U.t16(t).cuda() for t in truth]
    ng = len(s.prompt_lens)
    s1 = gpu_scales(p_res, res, rows, grp, td, ng)
    s2 = gpu_scales(p_hst, hst, rows, grp, td, ng)
    s3 = gpu_scales(p_res, res, rows, grp, td, ng, layers_per_launch=1)
    assert torch.equal(s1, s2) and torch.equal(s1, s3)
    g = workloads.prompt_of_row(s).copy()
    g[g == 2] = ng + 5               # the third request's rows name no group
    fr, n = U.gpu_fill_rows(p_res, res)
    k1, v1 = U.gpu_fill(p_res, res, fr, n, vscale=(s1, U.i32(g).cuda(), ng))
    k2, v2 = U.gpu_fill(p_hst, hst, fr, n, vscale=(s1, U.i32(g).cuda(), ng))
    f = fr.cpu().numpy()
    kept = f[g[f] != ng + 5]
    U.check_placement(k1, v1, kept, s.n_rows)
    for l in range(s.n_late):
        assert torch.equal(k1[l], k2[l]) and torch.equal(v1[l], v2[l]), f"layer {l}"


@pytest.mark.parametrize("name,groups", [("tiny_ragged", None), ("8b_mid_two", 1), ("27b_mid_q8", None),
                                         ("ragged_host", None), ("ragged_host6", None), ("ragged_host6", 1)])
def test_measured_fill_equals_two_calls(name, groups):
    """The measurement run inside the fill (rf_fill_opts.measure, the maps
    loaded once per layer group) gives bitwise the scales of rf_value_scales
    and the caches of the fill that applies them, also when the measurement's
    workspace allows fewer layers per launch than the fill's."""
    w, rows, grp, truth = _case(name)
    s = w.spec
    ng = len(s.prompt_lens)
    _say(f"[measured fill] {name} groups={groups}")
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    td = [U.t16(t).cuda() for t in truth]
    g_of_row = U.i32(workloads.prompt_of_row(s)).cuda()
    sc = gpu_scales(plan, di, rows, grp, td, ng)
    fr, n = U.gpu_fill_rows(plan, di)
    k1, v1 = U.gpu_fill(plan, di, fr, n, vscale=(sc, g_of_row, ng))
    sc2 = torch.full_like(sc, -7.0)
    g = s.n_late if groups is None else groups
    mws = torch.empty(plan.value_scales_workspace_bytes(len(rows), g), dtype=torch.uint8, device="cuda:0")
    measure = (td, U.i32(rows).cuda(), U.i32(grp).cuda(), g_of_row, ng, sc2, mws)
    k2, v2 = U.gpu_fill(plan, di, fr, n, measure=measure)
    assert torch.equal(sc, sc2)
    for l in range(s.n_late):
        assert torch.equal(k1[l], k2[l]) and torch.equal(v1[l], v2[l]), f"layer {l}"
