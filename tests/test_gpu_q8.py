"""GPU parity of the int8 map path (rf_fill_q8, rf_map_dequantize_q8).

The format is the 27B deployment's (RidgeFill, section 2.2 "Size and cost",
section 4.2): int8 codes with one bf16 scale for each 128-weight block of a row.  The
oracle dequantizes exactly (fp64); the library rounds each q * s once to bf16
before its bf16 matrix instructions, so values are held to the fill's
tolerance, the expansion itself bit-exactly, and rf_fill_q8 bitwise to rf_fill
on the expanded map.
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
    "tiny_q8": workloads.spec("tiny", map_format="q8", seed=20),
    "8b_mid_q8": workloads.spec("8b", n_late=3, prompt_lens=(700,), tail=60, map_format="q8", seed=21),
    "27b_mid_spans_q8": workloads.spec("27b_120k", n_late=2, prompt_lens=(1300,), tail=100, n_spans=4,
                                       map_format="q8", seed=22),
    "ragged_mid_q8": workloads.spec("8b_ragged_host", n_late=2, prompt_lens=(300, 257, 129, 64), tail=50,
                                    map_format="q8", seed=23),
}

_cache = {}


def _workload(name):
    if name not in _cache:
        _cache[name] = workloads.make(CASES[name])
    return _cache[name]


def _say(*a):
    print(*a, flush=True)


def _dequant_gpu(q: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    qd = torch.from_numpy(np.ascontiguousarray(q)).cuda()
    sd = U.t16(s_bits).cuda()
    out = torch.full(q.shape, U.CANARY, dtype=torch.int16, device="cuda:0")
    B.map_dequantize_q8(qd, sd, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


def test_dequantize_is_bit_exact():
    """rf_map_dequantize_q8 equals RNE(q * s) computed from the exact product."""
    w = workloads.make(workloads.spec("8b", n_late=1, prompt_lens=(8,), tail=2, map_format="q8", seed=24))
    cases = [(w.map_q[0], w.map_scale[0])]
    g = np.random.default_rng(25)
    q = g.integers(-127, 128, size=(96, 640)).astype(np.int8)
    sc = np.exp(g.uniform(-80.0, 80.0, size=(96, 5))).astype(np.float32)
    sc[::7] *= -1.0                    # the kernel multiplies whatever scale it is given
    s_bits = workloads.f32_to_bf16_bits(sc)
    s_bits[3, 2] = 0                   # zero scale
    cases.append((q, s_bits))
    for q, s_bits in cases:
        _say(f"[dequant] {q.shape}")
        got = _dequant_gpu(q, s_bits)
        ref = oracle.dequantize_q8_bf16(q, s_bits)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("name", list(CASES))
def test_q8_fill_matches_oracle(name):
    w = _workload(name)
    s = w.spec
    _say(f"[q8 fill] {name} d={s.d_in} L={s.n_late} rows={s.n_rows} host={s.maps_on_host}")
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    rows, n = U.gpu_fill_rows(plan, di)
    kc, vc = U.gpu_fill(plan, di, rows, n)
    f = rows.cpu().numpy()
    U.check_placement(kc, vc, f, s.n_rows)
    worst = U.check_values(kc, vc, oracle.fill_workload(w, rows=f), f, s.head_dim)
    _say(f"[q8 fill] {name} worst {worst}")


@pytest.mark.parametrize("name", ["tiny_q8", "8b_mid_q8"])
def test_q8_fill_equals_bf16_fill_of_the_expanded_map(name):
    """rf_fill_q8 is rf_fill on bf16(q * s): the same bytes, for grouped and
    one-layer launches."""
    w = _workload(name)
    s = w.spec
    _say(f"[q8 == bf16 image] {name}")
    di = U.DeviceInputs(w, maps_on_host=False)
    p8 = U.plan_for(w, maps_on_host=False)
    pb = U.plan_for(w, maps_on_host=False, maps_q8=False)
    rows, n = U.gpu_fill_rows(p8, di)
    image = [U.t16(oracle.dequantize_q8_bf16(q, sc)).cuda() for q, sc in zip(w.map_q, w.map_scale)]
    for g in (1, s.n_late):
        k8, v8 = U.gpu_fill(p8, di, rows, n, layers_per_launch=g)
        kb, vb = U.gpu_fill(pb, di, rows, n, layers_per_launch=g, map_a=image)
        for l in range(s.n_late):
            assert torch.equal(k8[l], kb[l]) and torch.equal(v8[l], vb[l]), f"group {g} layer {l}"


def test_q8_power_of_two_scales_equal_integral_bf16_map():
    """With every scale 2^-7 the int8 map is exactly q / 128, so the int8 path
    equals the bf16 path given that map (built here from the codes alone)."""
    w = _workload("8b_mid_q8")
    s = w.spec
    _say("[q8 pow2] 8b_mid_q8")
    di = U.DeviceInputs(w, maps_on_host=False)
    di.map_scale = [torch.full((s.d_out, s.d_in // 128), 0x3C00, dtype=torch.int16, device="cuda:0")
                    for _ in range(s.n_late)]
    a = [U.t16(workloads.f32_to_bf16_bits(q.astype(np.float32) / 128.0)).cuda() for q in w.map_q]
    p8 = U.plan_for(w, maps_on_host=False)
    pb = U.plan_for(w, maps_on_host=False, maps_q8=False)
    rows, n = U.gpu_fill_rows(p8, di)
    k8, v8 = U.gpu_fill(p8, di, rows, n)
    kb, vb = U.gpu_fill(pb, di, rows, n, map_a=a)
    for l in range(s.n_late):
        assert torch.equal(k8[l], kb[l]) and torch.equal(v8[l], vb[l]), f"layer {l}"


def test_q8_streamed_equals_resident():
    """int8 maps streamed from pinned host memory give the resident path's bytes."""
    w = _workload("ragged_mid_q8")
    _say("[q8 streamed] ragged_mid_q8")
    res = U.DeviceInputs(w, maps_on_host=False)
    hst = U.DeviceInputs(w, maps_on_host=True)
    p_res = U.plan_for(w, maps_on_host=False)
    p_hst = U.plan_for(w, maps_on_host=True)
    s = w.spec
    image = s.d_out * s.d_in * 2
    p_bf = U.plan_for(w, maps_on_host=True, maps_q8=False)
    # a streamed launch holds each of its layers' bf16 images on top of the
    # bf16 plan's needs, for at most RF_STREAM_GROUP layers
    g = min(s.n_late, B.RF_STREAM_GROUP)
    assert p_hst.fill_workspace_bytes(100, s.n_late) == p_hst.fill_workspace_bytes(100, g)
    for k in range(1, g + 1):
        assert p_hst.fill_workspace_bytes(100, k) == p_bf.fill_workspace_bytes(100, k) + k * image
    p_bf.close()
    rows, n = U.gpu_fill_rows(p_res, res)
    k1, v1 = U.gpu_fill(p_res, res, rows, n)
    k2, v2 = U.gpu_fill(p_hst, hst, rows, n)
    for l in range(s.n_late):
        assert torch.equal(k1[l], k2[l]) and torch.equal(v1[l], v2[l]), f"layer {l}"
