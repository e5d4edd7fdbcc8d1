"""fp64 oracle of the value rescale.

Test infrastructure only (see ``oracle/__init__.py``).

"RidgeFill: Training-Free Late-Layer Cache Fill for Faster Prefill", section
2.3 ("Value rescale"), and section 4.2 (on for the 27B, c = 512): in each late
layer, the first c rows of a request's tail are projected to values twice,
from their true input and from the map's prediction; per key-value head, the
exact-to-predicted ratio of value norms averaged over those rows scales the
values of the request's filled rows.  Readings taken here:

* "the first c tail rows" are the c lowest rows of each request's tail (all of
  the tail when it is shorter than c);
* the scale is the mean over the c rows of the per-row ratio
  ||v_exact||_2 / ||v_pred||_2 of the head's value vector (a mean of ratios,
  not a ratio of mean norms); rows whose predicted head norm is zero are left
  out, and a head with no rows left keeps scale 1;
* each request has its own scales (the pages measure them per request from the
  request's own tokens), one per late layer and key-value head;
* the scale multiplies the filled rows' value vectors before they are stored;
  keys are not touched.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from .fill import bf16_bits_to_f64, fill_workload, map_matrix, predicted_input, project, rms_norm


def calibration_rows(prompt_lens: Sequence[int], tail: int, c: int) -> Tuple[np.ndarray, np.ndarray]:
    """Rows measured for the value scale and the request each belongs to.

    Request p's tail is its last ``tail`` rows; its calibration rows are the
    first min(c, tail) of them.  Returns (rows int32, request int32), ascending.
    """
    rows, grp = [], []
    start = 0
    for p, n in enumerate(prompt_lens):
        t = min(tail, n)
        first = start + n - t
        k = min(c, t)
        rows.extend(range(first, first + k))
        grp.extend([p] * k)
        start += n
    return np.array(rows, dtype=np.int32), np.array(grp, dtype=np.int32)


def head_norms(v: np.ndarray, head_dim: int) -> np.ndarray:
    """Euclidean norm of every head of every row: [n][n_heads]."""
    n, width = v.shape
    return np.linalg.norm(v.reshape(n, width // head_dim, head_dim), axis=2)


def scales_from_values(v_exact: np.ndarray, v_pred: np.ndarray, group: np.ndarray, n_groups: int,
                       head_dim: int) -> np.ndarray:
    """Per request and head: mean over the request's rows of ||v_exact|| / ||v_pred||."""
    ne = head_norms(v_exact, head_dim)
    npr = head_norms(v_pred, head_dim)
    n_heads = ne.shape[1]
    out = np.ones((n_groups, n_heads))
    for g in range(n_groups):
        sel = np.asarray(group) == g
        for h in range(n_heads):
            ok = sel & (npr[:, h] > 0)
            if ok.any():
                out[g, h] = np.mean(ne[ok, h] / npr[ok, h])
    return out


def value_scales(w, layer_true: List[np.ndarray], calib_rows: np.ndarray, calib_group: np.ndarray,
                 n_groups: int, layers: Optional[List[int]] = None) -> Dict[int, np.ndarray]:
    """{layer: scales [n_groups][n_kv]} for a workload.

    ``layer_true[l]`` holds bf16 bits [len(calib_rows)][d_out]: the true input of
    layer l for each calibration row, in calibration order.
    """
    s = w.spec
    r = np.asarray(calib_rows)
    xs = bf16_bits_to_f64(w.x[r])
    out = {}
    for l in (range(s.n_late) if layers is None else layers):
        g = bf16_bits_to_f64(w.gamma[l])
        wv = bf16_bits_to_f64(w.w_v[l])
        y_pred = predicted_input(xs, map_matrix(w, l), bf16_bits_to_f64(w.map_b[l]))
        v_pred = project(rms_norm(y_pred, g, s.rms_eps), wv)
        v_exact = project(rms_norm(bf16_bits_to_f64(layer_true[l]), g, s.rms_eps), wv)
        out[l] = scales_from_values(v_exact, v_pred, calib_group, n_groups, s.head_dim)
    return out


def rescale_values(v: np.ndarray, scale: np.ndarray, group_of_rows: np.ndarray, head_dim: int) -> np.ndarray:
    """Filled value vectors times their request's per-head scale.

    v: [n][n_kv*head_dim]; scale: [n_groups][n_kv]; group_of_rows: [n].
    """
    n, width = v.shape
    f = np.repeat(scale[np.asarray(group_of_rows)], head_dim, axis=1)
    return v * f


def fill_workload_rescaled(w, scales: Dict[int, np.ndarray], group_of_row: np.ndarray,
                           rows: np.ndarray, layers: Optional[List[int]] = None):
    """The fill of ``rows`` with each layer's values rescaled per request.

    Returns {layer: (K, V)}: K as the plain fill, V times the scale of the
    row's request and head.
    """
    base = fill_workload(w, rows=rows, layers=layers)
    g = np.asarray(group_of_row)[np.asarray(rows)]
    return {l: (k, rescale_values(v, scales[l], g, w.spec.head_dim)) for l, (k, v) in base.items()}
