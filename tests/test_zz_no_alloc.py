"""rf_fill_rows_noalloc against rf_fill_rows, through the C ABI (GPU).

The no-allocation entry point keeps its scratch in a device array the library
owns; every call on the GPU reuses it.  Two calls in a row, the second on a
smaller batch, must each give exactly the rows (and count) of rf_fill_rows
with a caller workspace, and the fill-row set of the oracle (RidgeFill
section 2.1: all rows minus the exact set).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from late_layer_kv_amd import binding as B

pytestmark = pytest.mark.gpu


def _exact_shuffled(s, seed):
    e = workloads.exact_row_list(s)
    g = np.random.default_rng(seed)
    given = np.concatenate([e, e[: len(e) // 3]])   # duplicates, any order
    g.shuffle(given)
    return e, torch.from_numpy(given.astype(np.int32)).cuda()


def _both(s, seed):
    e, given = _exact_shuffled(s, seed)
    plan = B.Plan.for_spec(s, maps_on_host=False)
    ref = oracle.fill_row_set(s.n_rows, e)
    print(f"[no-alloc] {s.name}: n_rows={s.n_rows} exact={len(e)} fill={len(ref)}", flush=True)
    out_ws = torch.full((s.n_rows,), -7, dtype=torch.int32, device="cuda:0")
    nf_ws = torch.full((1,), -7, dtype=torch.int32, device="cuda:0")
    ws = torch.empty(B.fill_rows_workspace_bytes(s.n_rows), dtype=torch.uint8, device="cuda:0")
    B.fill_rows(plan, given, out_ws, nf_ws, ws)
    out = torch.full((s.n_rows,), -7, dtype=torch.int32, device="cuda:0")
    nf = torch.full((1,), -7, dtype=torch.int32, device="cuda:0")
    B.fill_rows_noalloc(plan, given, out, nf)
    torch.cuda.synchronize()
    n = int(nf.item())
    assert n == int(nf_ws.item()) == len(ref)
    assert torch.equal(out, out_ws), "no-alloc rows differ from the workspace entry point"
    assert np.array_equal(out[:n].cpu().numpy(), ref)
    assert torch.all(out[n:] == -7), "rows past n_fill were written"


def test_no_alloc_two_calls_second_smaller():
    # the ragged four-request batch, then a 120K-row prompt's worth less: a
    # smaller batch whose mask is shorter than what the first call left behind
    _both(workloads.spec("8b_ragged_host"), seed=1)
    _both(workloads.spec("tiny", prompt_lens=(5000, 700, 33), tail=64), seed=2)


def test_no_alloc_at_its_row_limit_then_tiny():
    _both(workloads.spec("tiny", prompt_lens=(B.RF_NOALLOC_MAX_ROWS - 1000, 1000), tail=2048), seed=3)
    _both(workloads.spec("tiny", prompt_lens=(3,), tail=2), seed=4)


def test_no_alloc_refuses_a_batch_over_the_limit():
    s = workloads.spec("tiny", prompt_lens=(B.RF_NOALLOC_MAX_ROWS + 1,), tail=64)
    plan = B.Plan.for_spec(s, maps_on_host=False)
    out = torch.empty(s.n_rows, dtype=torch.int32, device="cuda:0")
    nf = torch.empty(1, dtype=torch.int32, device="cuda:0")
    with pytest.raises(B.RfError) as e:
        B.fill_rows_noalloc(plan, None, out, nf)
    assert e.value.status == -2
