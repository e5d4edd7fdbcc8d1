"""rf_fill and rf_fill_q8 under HIP graph capture.

With maps resident in device memory the fill keeps no state between calls
(the workspace is the caller's, the RoPE table is either given or rebuilt in
the workspace) and issues only kernel launches on the caller's stream: no
memory sets, no allocation, no synchronisation.  A captured fill therefore
replays to the same bytes as the eager call.  Each replay below is checked
against the eager result, with other eager work of the program and
synchronisations between the replays.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from late_layer_kv_amd import binding as B
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,given_table", [("bf16", False), ("bf16", True), ("q8", False)])
def test_captured_fill_replays_to_the_eager_bytes(fmt, given_table):
    s = workloads.spec("8b", n_late=3, prompt_lens=(700,), tail=60, qk_norm=True, idx_heads=1, map_format=fmt,
                       seed=120)
    print(f"[graph] {fmt} maps, given_table={given_table}", flush=True)
    w = workloads.make(s)
    di = U.DeviceInputs(w, maps_on_host=False)
    plan = U.plan_for(w, maps_on_host=False)
    fr, n = U.gpu_fill_rows(plan, di)
    f = fr.cpu().numpy()
    slots = U.i32(np.random.default_rng(121).permutation(s.n_rows)).cuda()
    table = None
    if given_table:
        table = torch.empty((s.max_pos, s.head_dim // 2, 2), dtype=torch.float32, device="cuda:0")
        B.rope_table(plan, table)
    g = 2  # two launch groups of the three layers
    ws = torch.empty(plan.fill_workspace_bytes(n, g), dtype=torch.uint8, device="cuda:0")

    def run(kc, vc, ic):
        if di.q8:
            B.fill_q8(plan, di.x, fr, n, di.positions, slots, di.map_q, di.map_scale, di.map_b, di.gamma, di.w_k,
                      di.w_v, table, kc, vc, ws, k_norm=di.k_norm, w_idx=di.w_idx, idx_cache=ic)
        else:
            B.fill(plan, di.x, fr, n, di.positions, slots, di.map_a, di.map_b, di.gamma, di.w_k, di.w_v, table,
                   kc, vc, ws, k_norm=di.k_norm, w_idx=di.w_idx, idx_cache=ic)

    ref_k, ref_v = di.caches()
    ref_i = di.idx_caches()
    run(ref_k, ref_v, ref_i)
    torch.cuda.synchronize()

    kc, vc = di.caches()
    ic = di.idx_caches()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream, as torch's capture expects
        run(kc, vc, ic)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(kc, vc, ic)
    torch.cuda.synchronize()

    other_k, other_v = di.caches()
    other_i = di.idx_caches()
    for rep in range(3):
        for c in kc + vc + ic:
            c.fill_(U.CANARY)
        run(other_k, other_v, other_i)  # eager work of the program between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l in range(s.n_late):
            assert torch.equal(kc[l], ref_k[l]), f"replay {rep}: K layer {l}"
            assert torch.equal(vc[l], ref_v[l]), f"replay {rep}: V layer {l}"
            assert torch.equal(ic[l], ref_i[l]), f"replay {rep}: indexer keys layer {l}"
            assert torch.equal(other_k[l], ref_k[l]) and torch.equal(other_v[l], ref_v[l])
    sl = slots.cpu().numpy()
    U.check_placement(kc, vc, f, s.n_rows, slots=sl, ic=ic)
    U.check_values(kc, vc, oracle.fill_workload(w, rows=f), f, s.head_dim, slots=sl)
    print(f"[graph] {fmt} maps, given_table={given_table}: 3 replays bitwise equal to the eager fill", flush=True)
