"""GPU parity over a seeded sweep of mixed configurations.

Each case draws, from its own fixed seed, a shape the library accepts and a
mix of options that the other parity files mostly exercise one or two at a
time: d_in (a multiple of 64, or of 128 for int8 maps) and d_out (a multiple
of 256), not always equal; head_dim 64 or 128 with kv-head counts that fill
128-wide feature blocks; one to three late layers in launch groups of any
size; one to three prompts with their tails and scattered exact spans; int8
maps, QK-norm, indexer key heads (a whole 256-wide feature tile, a 128-wide
remainder for the tall tiles, or a 64-wide one), maps streamed from pinned
host memory, a scattered slot map and either value distribution of the
workloads.  K, V and indexer keys against the fp64 oracle at the fill's
tolerance; placement bit-exact at the mapped slots.
"""
import random

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

N_CASES = 16


def _draw(i: int):
    """Case i: (spec, layers per launch, use a slot map)."""
    r = random.Random(7000 + i)
    hd = r.choice([64, 128])
    n_kv = r.choice([1, 2, 3, 4]) if hd == 128 else r.choice([2, 4, 6])
    q8 = r.random() < 0.3
    d_in = 128 * r.randint(1, 6) if q8 else 64 * r.randint(1, 12)
    d_out = 256 * r.randint(1, 3)
    n_late = r.randint(1, 3)
    n_prompts = r.randint(1, 3)
    lens = tuple(r.randint(90, 900) for _ in range(n_prompts))
    tail = r.randint(1, min(80, min(lens) - 1))
    spans = r.randint(1, 3) if lens[0] - tail >= 400 else 0
    tiny_values = r.random() < 0.5
    s = workloads.spec(
        "tiny", d_in=d_in, d_out=d_out, n_late=n_late, n_kv=n_kv, head_dim=hd, prompt_lens=lens, tail=tail,
        n_spans=spans, rope_theta=r.choice([1.0e4, 5.0e5]),
        map_sigma=0.02 if tiny_values else 0.01, n_outliers=0 if tiny_values else 4,
        maps_on_host=r.random() < 0.25, map_format="q8" if q8 else "bf16", qk_norm=r.random() < 0.3,
        idx_heads=r.choice([0, 0, 1, 2]), seed=7000 + i)
    return s, r.randint(1, n_late), r.random() < 0.5


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_case_matches_oracle(i):
    s, g, use_slots = _draw(i)
    print(f"[sweep {i}] d_in={s.d_in} d_out={s.d_out} L={s.n_late} (groups of {g}) kv={s.n_kv}x{s.head_dim} "
          f"idx={s.idx_heads} prompts={s.prompt_lens} tail={s.tail} spans={s.n_spans} fmt={s.map_format} "
          f"qk={s.qk_norm} host={s.maps_on_host} slots={use_slots}", flush=True)
    w = workloads.make(s)
    di = U.DeviceInputs(w)
    plan = U.plan_for(w)
    fr, n = U.gpu_fill_rows(plan, di)
    f = fr.cpu().numpy()
    assert np.array_equal(f, oracle.fill_row_set(s.n_rows, w.exact_rows))
    slots = np.random.default_rng(7000 + i).permutation(s.n_rows).astype(np.int32) if use_slots else None
    out = U.gpu_fill(plan, di, fr, n, layers_per_launch=g, slots=None if slots is None else U.i32(slots).cuda())
    kc, vc = out[0], out[1]
    ic = out[2] if s.idx_heads else None
    U.check_placement(kc, vc, f, s.n_rows, slots=slots, ic=ic)
    worst = U.check_values(kc, vc, oracle.fill_workload(w, rows=f), f, s.head_dim, slots=slots)
    if ic is not None:
        wi = U.check_indexer_values(ic, oracle.fill_indexer_workload(w, rows=f), f, s.head_dim, slots=slots)
        worst = {k: max(worst[k], wi[k]) for k in worst}
    print(f"[sweep {i}] rows={n} worst {worst}", flush=True)
    torch.cuda.synchronize()
