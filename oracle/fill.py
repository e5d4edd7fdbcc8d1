"""fp64 oracle of the fill: rows, map, norm, projections, rotary embedding.

Test infrastructure only (see ``oracle/__init__.py``).

Citations name sections of "RidgeFill: Training-Free Late-Layer Cache Fill for
Faster Prefill" (arXiv 2611.09709).  Readings the pages leave open are stated
where they are taken:

* maps act on row vectors: the paper's column form x_hat = A x_S + b becomes
  x_hat = x_S A^T + b with A stored [d_out][d_in] exactly as the paper sizes
  it (d_out rows, d_in columns, section 2.2 "Size and cost");
* the layer's normalization, which the pages name without writing out, is
  RMSNorm gamma * y / sqrt(mean(y^2) + eps) with a multiplicative gain and eps
  inside the root;
* projections are stored [out][in] and applied as h W^T;
* the rotary embedding, applied to the keys in the usual way, is the
  rotate-half form: within every head,
  dimension j < hd/2 is paired with j + hd/2 and the pair is turned by the
  angle pos * theta^(-2j/hd), with no frequency scaling;
* QK-norm (layers that normalise their keys) is an RMSNorm over each key head
  with a per-dimension gain shared by the heads and the layer's eps, applied
  after the key projection and before the rotation;
* the sparse-attention indexer's keys that filled rows also write (section 2.1,
  section 5.1: one 128-wide key head shared by the indexer's query heads) are
  projected from the same normalised input as the layer's keys and values and
  rotated the same way; no key norm applies to them (the pages give the
  indexer no normalization of its own).
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Tuple

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fill_row_set(n_rows: int, exact_rows: Iterable[int]) -> np.ndarray:
    """Rows whose late-layer cache entries come from the fill, ascending.

    Section 2.1 ("Split, tail and prefix"): the tail runs every layer exactly,
    and prefix rows are split between exact computation and the fill, so the
    filled rows are all rows minus the exact set (tail plus chosen rows,
    section 2.4).
    """
    return np.setdiff1d(np.arange(n_rows, dtype=np.int64),
                        np.asarray(list(exact_rows) if not isinstance(exact_rows, np.ndarray)
                                   else exact_rows, dtype=np.int64)).astype(np.int32)


def predicted_input(x_s: np.ndarray, a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Section 2.2, the map equation x_hat_l = A_l x_S + b_l, for a stack of rows.

    x_s: [n][d_in]; a: [d_out][d_in]; b: [d_out]  ->  [n][d_out].
    """
    return x_s @ a.T + b


def rms_norm(y: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """Section 2.2: the prediction is normalised by the layer's unchanged norm,
    like a true input; here that norm is RMSNorm over the last axis."""
    return gamma * y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)


def project(h: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Sections 2.1-2.2: the layer's own key or value projection, w stored [out][in]."""
    return h @ w.T


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Angular frequency of pair j: theta^(-2j/head_dim), j < head_dim/2."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * j / head_dim)


def rope(k: np.ndarray, positions: np.ndarray, theta: float, head_dim: int) -> np.ndarray:
    """Section 2.2 (predicted keys are rotated the standard way) and section 6.6
    (each key takes the rotation of its own row's position).

    k: [n][n_heads * head_dim]; positions: [n].  Angles in float64.
    """
    n, width = k.shape
    half = head_dim // 2
    kh = k.reshape(n, width // head_dim, head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * rope_inv_freq(head_dim, theta)[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    lo = kh[..., :half]
    hi = kh[..., half:]
    out = np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)
    return out.reshape(n, width)


def qk_norm(k: np.ndarray, k_gamma: np.ndarray, eps: float, head_dim: int) -> np.ndarray:
    """QK-norm on keys (section 6.6 and section 7: in the Qwen models both
    queries and keys are normalised per head ahead of attention): every head of every row is scaled to
    unit RMS, RMSNorm over its head_dim values with eps inside the root, then
    multiplied by the per-dimension gain k_gamma [head_dim] shared by the heads.

    k: [n][n_heads * head_dim].
    """
    n, width = k.shape
    kh = k.reshape(n, width // head_dim, head_dim)
    ms = np.mean(kh * kh, axis=2, keepdims=True)
    return (kh / np.sqrt(ms + eps) * k_gamma).reshape(n, width)


def layer_kv(h_in: np.ndarray, gamma: np.ndarray, w_k: np.ndarray, w_v: np.ndarray,
             positions: np.ndarray, theta: float, head_dim: int, eps: float,
             k_gamma: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """The cache entries a late attention layer stores for one input row.

    Section 2.1: for such a row a late layer produces only the keys and values
    later tokens attend to; section 2.2: the input is normalised and projected
    by the layer's unchanged weights, and the keys are rotated.
    With ``k_gamma`` the layer normalises its keys (QK-norm) before the
    rotation, as the Qwen layers do.
    """
    h = rms_norm(h_in, gamma, eps)
    k = project(h, w_k)
    if k_gamma is not None:
        k = qk_norm(k, k_gamma, eps, head_dim)
    k = rope(k, positions, theta, head_dim)
    v = project(h, w_v)
    return k, v


def indexer_keys(h_in: np.ndarray, gamma: np.ndarray, w_idx: np.ndarray, positions: np.ndarray,
                 theta: float, head_dim: int, eps: float) -> np.ndarray:
    """The indexer keys a late sparse-attention layer writes from an input row.

    Section 2.1 (filled rows also write the indexer's keys, section 5.1): the
    layer's normalised input times the indexer key projection W_idx
    [heads * head_dim][d], each head rotated like the attention keys.
    """
    return rope(project(rms_norm(h_in, gamma, eps), w_idx), positions, theta, head_dim)


def fill_layer(x_s, a, b, gamma, w_k, w_v, positions, theta, head_dim, eps, k_gamma=None):
    """One late layer's filled K/V: the map's prediction through layer_kv."""
    return layer_kv(predicted_input(x_s, a, b), gamma, w_k, w_v, positions,
                    theta, head_dim, eps, k_gamma)


def _k_gamma(w, l):
    kn = getattr(w, "k_norm", None)
    return None if kn is None else bf16_bits_to_f64(kn[l])


def _rows(w, rows: Optional[np.ndarray]) -> np.ndarray:
    return fill_row_set(w.spec.n_rows, w.exact_rows) if rows is None else np.asarray(rows)


def map_matrix(w, l: int) -> np.ndarray:
    """Layer l's map A_l [d_out][d_in] in float64, from bf16 or int8 storage.

    int8 maps (section 2.2 "Size and cost", section 4.2) are dequantized
    exactly: code times the bf16 scale of its 128-weight block.
    """
    if w.map_q is not None:
        from .quant import dequantize_q8
        return dequantize_q8(w.map_q[l], w.map_scale[l])
    return bf16_bits_to_f64(w.map_a[l])


def fill_workload(w, rows: Optional[np.ndarray] = None,
                  layers: Optional[List[int]] = None) -> Dict[int, Tuple[np.ndarray, np.ndarray]]:
    """fp64 K and V of every late layer for the given rows of a workload.

    ``w`` is a ``workloads.Workload``; ``rows`` defaults to the whole fill set.
    Returns {layer: (K [len(rows)][n_kv*hd], V [...])}, unrounded.
    """
    s = w.spec
    r = _rows(w, rows)
    xs = bf16_bits_to_f64(w.x[r])
    pos = w.positions[r]
    out = {}
    for l in (range(s.n_late) if layers is None else layers):
        out[l] = fill_layer(xs, map_matrix(w, l), bf16_bits_to_f64(w.map_b[l]),
                            bf16_bits_to_f64(w.gamma[l]), bf16_bits_to_f64(w.w_k[l]),
                            bf16_bits_to_f64(w.w_v[l]), pos, s.rope_theta, s.head_dim,
                            s.rms_eps, _k_gamma(w, l))
    return out


def exact_kv_workload(w, layer_inputs: np.ndarray, rows: np.ndarray,
                      layers: Optional[List[int]] = None) -> Dict[int, Tuple[np.ndarray, np.ndarray]]:
    """fp64 K and V that each late layer writes from the given true inputs.

    The exact path of section 2.1 applied to the layer's own cache write only
    (no map): ``layer_inputs`` is a bf16 bit array [n_rows][d_out] used as the
    input of every layer listed.
    """
    s = w.spec
    r = np.asarray(rows)
    h = bf16_bits_to_f64(layer_inputs[r])
    pos = w.positions[r]
    out = {}
    for l in (range(s.n_late) if layers is None else layers):
        out[l] = layer_kv(h, bf16_bits_to_f64(w.gamma[l]), bf16_bits_to_f64(w.w_k[l]),
                          bf16_bits_to_f64(w.w_v[l]), pos, s.rope_theta, s.head_dim, s.rms_eps,
                          _k_gamma(w, l))
    return out


def fill_indexer_workload(w, rows: Optional[np.ndarray] = None,
                          layers: Optional[List[int]] = None) -> Dict[int, np.ndarray]:
    """fp64 indexer keys of every late layer for the given (filled) rows:
    {layer: [len(rows)][idx_heads * head_dim]}, unrounded."""
    s = w.spec
    r = _rows(w, rows)
    xs = bf16_bits_to_f64(w.x[r])
    pos = w.positions[r]
    out = {}
    for l in (range(s.n_late) if layers is None else layers):
        y = predicted_input(xs, map_matrix(w, l), bf16_bits_to_f64(w.map_b[l]))
        out[l] = indexer_keys(y, bf16_bits_to_f64(w.gamma[l]), bf16_bits_to_f64(w.w_idx[l]), pos,
                              s.rope_theta, s.head_dim, s.rms_eps)
    return out


def exact_indexer_workload(w, layer_inputs: np.ndarray, rows: np.ndarray,
                           layers: Optional[List[int]] = None) -> Dict[int, np.ndarray]:
    """fp64 indexer keys each late layer writes from the given true inputs."""
    s = w.spec
    r = np.asarray(rows)
    h = bf16_bits_to_f64(layer_inputs[r])
    pos = w.positions[r]
    return {l: indexer_keys(h, bf16_bits_to_f64(w.gamma[l]), bf16_bits_to_f64(w.w_idx[l]), pos,
                            s.rope_theta, s.head_dim, s.rms_eps)
            for l in (range(s.n_late) if layers is None else layers)}
