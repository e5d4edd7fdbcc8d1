"""GPU parity of QK-norm on the filled keys (rf_fill_opts.k_norm).

Layers that normalise their keys (the Qwen layers; RidgeFill sections 6.6
and 7) get an RMSNorm over each key head with a per-dimension gain before the
rotation.  Values against the fp64 oracle to the fill's tolerance, placement
bit-exact, and bitwise identities with the exact-row path.
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
    "tiny_qk": workloads.spec("tiny", qk_norm=True, seed=50),
    "8b_mid_qk": workloads.spec("8b", n_late=3, prompt_lens=(700,), tail=60, qk_norm=True, seed=51),
    "27b_mid_q8_qk": workloads.spec("27b_120k", n_late=2, prompt_lens=(1300,), tail=100, n_spans=4,
                                    map_format="q8", qk_norm=True, seed=52),
    "ragged_host_qk": workloads.spec("8b_ragged_host", n_late=2, prompt_lens=(300, 257, 129, 64), tail=50,
                                     qk_norm=True, seed=53),
}

_cache = {}


def _workload(name):
    if name not in _cache:
        _cache[name] = workloads.make(CASES[name])
    return _cache[name]


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("name", list(CASES))
def test_qk_fill_matches_oracle(name):
    w = _workload(name)
    s = w.spec
    _say(f"[qk fill] {name} hd={s.head_dim} fmt={s.map_format} host={s.maps_on_host}")
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    rows, n = U.gpu_fill_rows(plan, di)
    kc, vc = U.gpu_fill(plan, di, rows, n)
    f = rows.cpu().numpy()
    U.check_placement(kc, vc, f, s.n_rows)
    worst = U.check_values(kc, vc, oracle.fill_workload(w, rows=f), f, s.head_dim)
    _say(f"[qk fill] {name} worst {worst}")


@pytest.mark.parametrize("name", ["tiny_qk", "8b_mid_qk"])
def test_qk_identity_fill_equals_exact_projection(name):
    """Identity maps with QK-norm give the exact-row path's bytes."""
    w = _workload(name)
    s = w.spec
    _say(f"[qk identity] {name}")
    di = U.DeviceInputs(w, maps_on_host=False)
    plan = U.plan_for(w, maps_on_host=False)
    rows, n = U.gpu_fill_rows(plan, di)
    a, b = U.identity_maps(di)
    k1, v1 = U.gpu_fill(plan, di, rows, n, map_a=a, map_b=b)
    k2, v2 = U.gpu_kv_project(plan, di, [di.x] * s.n_late, rows, n)
    for l in range(s.n_late):
        assert torch.equal(k1[l], k2[l]) and torch.equal(v1[l], v2[l]), f"layer {l}"
    f = rows.cpu().numpy()
    U.check_values(k2, v2, oracle.exact_kv_workload(w, w.x, f), f, s.head_dim)


@pytest.mark.parametrize("name", ["tiny_qk", "8b_mid_qk"])
def test_unit_gain_gives_unit_rms_keys(name):
    """With gain 1 every stored key head has RMS sqrt(ms / (ms + eps)) ~ 1
    (the rotation keeps each pair's norm); values are untouched by QK-norm."""
    w = _workload(name)
    s = w.spec
    _say(f"[qk unit gain] {name}")
    di = U.DeviceInputs(w)
    di.k_norm = [torch.full((s.head_dim,), U.BF16_ONE, dtype=torch.int16, device="cuda:0") for _ in range(s.n_late)]
    plan = U.plan_for(w)
    rows, n = U.gpu_fill_rows(plan, di)
    kc, vc = U.gpu_fill(plan, di, rows, n)
    f = rows.cpu().numpy()
    for l in range(s.n_late):
        k = U.bits_to_f64(kc[l][rows.long()]).reshape(n, s.n_kv, s.head_dim)
        rms = np.sqrt(np.mean(k * k, axis=2))
        assert np.max(np.abs(rms - 1.0)) < 4e-3, f"layer {l}: key head RMS off by {np.max(np.abs(rms - 1.0)):.2e}"
    plain = U.DeviceInputs(w)
    plain.k_norm = None
    kp, vp = U.gpu_fill(plan, plain, rows, n)
    for l in range(s.n_late):
        assert torch.equal(vc[l], vp[l]), f"layer {l}: values changed"


def test_qk_with_value_rescale():
    """QK-norm and the value rescale together (their combined kernel)."""
    w = _workload("8b_mid_qk")
    s = w.spec
    _say("[qk + rescale] 8b_mid_qk")
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    rows, n = U.gpu_fill_rows(plan, di)
    sc = np.array([[0.75, 1.25, 1.0, 0.5, 2.0, 1.5, 1.1, 0.9]] * s.n_late, dtype=np.float32)[:, None, :]
    g_of_row = workloads.prompt_of_row(s)
    kc, vc = U.gpu_fill(plan, di, rows, n, vscale=(torch.from_numpy(sc).cuda(), U.i32(g_of_row).cuda(), 1))
    f = rows.cpu().numpy()
    ref = oracle.fill_workload_rescaled(w, {l: sc[l].astype(np.float64) for l in range(s.n_late)}, g_of_row, f)
    U.check_values(kc, vc, ref, f, s.head_dim)
