"""GPU parity at the edges of the shapes the library accepts.

The map contraction runs ceil(d_in / 64) stages of 64 columns, with separate
code for one, two and three stages; the tiles have 256 rows, so fills of 1,
255, 256 and 257 rows sit on and around a tile edge; d_in and d_out may
differ (the map is d_out x d_in).  Values against the fp64 oracle to the
fill's tolerance, placement bit-exact.
"""
import numpy as np
import pytest

import oracle
import workloads
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
