"""Seeded synthetic inputs for the late-layer cache fill.

This module only draws numbers.  It holds none of the fill's arithmetic: no
map product, no normalisation, no projection, no rotary embedding and no
row-set logic.  Both the CPU oracle (``oracle/``) and the GPU library's tests
and benchmark take their inputs from here, so the two sides see the very same
bf16 bit patterns.

Recipe (RidgeFill, "2 Method": a split state x_S per row, one map pair
(A_l, b_l) per late layer, and each late layer's own RMSNorm gain and key /
value projections):

* every value is drawn in fp32 from numpy's PCG64 and then cast to bf16 with
  round-to-nearest-even on the bit pattern;
* every array has its own seed sequence ``SeedSequence([seed, kind, i, j])``,
  so any array (one layer's map, one block of rows) can be regenerated alone
  and arrays can be drawn in parallel threads;
* x_S ~ N(0, 1) per element; ``n_outliers`` channels, drawn once without
  replacement, are multiplied by ``outlier_scale`` in fp32 before the cast;
* A_l = I + N(0, map_sigma^2) stored [d_out][d_in] (row n is output feature n;
  the identity is placed on the leading diagonal when d_in != d_out);
* b_l ~ N(0, bias_sigma^2), gamma_l ~ 1 + N(0, gamma_sigma^2);
* W_k, W_v ~ N(0, 1/d_out), stored [n_kv * head_dim][d_out];
* int8 maps (``map_format="q8"``, the 27B deployment's format: int8 codes
  and one bf16 scale for each 128-weight block of a row) are drawn directly in that
  format with the same value distribution: a block holding the identity's
  diagonal gets scale ~ (1 + N(0, map_sigma^2)) / 127 and diagonal code 127,
  any other block scale ~ map_sigma * (2.8 + 0.4 |N(0, 1)|) / 127; the other
  codes are N(0, map_sigma^2) / scale rounded to integers and clipped to
  [-127, 127];
* layers that normalise their keys (``qk_norm=True``) get a key-norm gain
  k_gamma_l ~ 1 + N(0, gamma_sigma^2) of length head_dim;
* layers with a sparse-attention indexer (``idx_heads > 0``) get its key
  projection W_idx ~ N(0, 1/d_out), stored [idx_heads * head_dim][d_out];
* positions restart at 0 for every prompt of a batch;
* the exact set is the last ``tail`` rows of every prompt plus ``n_spans``
  disjoint spans of ``span_len`` rows drawn uniformly inside the first
  prompt's prefix (redrawn on overlap).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import List, Optional, Tuple

import numpy as np

__all__ = [
    "Spec", "Workload", "SPECS", "CONFIG_ORDER", "spec", "make",
    "f32_to_bf16_bits", "exact_row_list", "prompt_of_row", "calibration_row_list", "make_layer_truth",
]

# seed-sequence "kind" tags
_K_X, _K_OUTLIER, _K_LAYER, _K_SPANS, _K_TRUTH = 1, 2, 3, 4, 5
_L_MAP, _L_BIAS, _L_GAMMA, _L_WK, _L_WV, _L_QSCALE, _L_KNORM, _L_WIDX = 0, 1, 2, 3, 4, 5, 6, 7
Q8_BLOCK = 128  # weights per bf16 scale along each row of an int8 map
_X_BLOCK = 8192  # rows per independently seeded block of x_S


@dataclass(frozen=True)
class Spec:
    """Shape and value distribution of one synthetic workload."""
    name: str
    d_in: int
    d_out: int
    n_late: int
    n_kv: int
    head_dim: int
    prompt_lens: Tuple[int, ...]
    tail: int
    n_spans: int = 0
    span_len: int = 32
    rope_theta: float = 5.0e5
    rms_eps: float = 1.0e-5
    map_sigma: float = 0.01
    bias_sigma: float = 0.01
    gamma_sigma: float = 0.1
    n_outliers: int = 4
    outlier_scale: float = 20.0
    maps_on_host: bool = False
    map_format: str = "bf16"   # "bf16" or "q8"
    qk_norm: bool = False      # keys normalised per head before RoPE
    idx_heads: int = 0         # indexer key heads per late layer (head_dim wide each)
    seed: int = 0

    @property
    def n_rows(self) -> int:
        return int(sum(self.prompt_lens))

    @property
    def kv_width(self) -> int:
        return self.n_kv * self.head_dim

    @property
    def max_pos(self) -> int:
        return int(max(self.prompt_lens))


# The five workloads: a tiny model, a Llama-3.1-8B-shaped one, a 27B-dense-shaped
# one at 64K and 120K rows, and a ragged batch of four 8B-shaped prompts whose
# maps live in pinned host memory.  Configurations 2-4 share the 8B value
# distributions (outlier channels, map noise 0.01).
SPECS = {
    "tiny": Spec("tiny", 256, 256, 4, 2, 64, (512,), 64, rope_theta=1.0e4,
                 map_sigma=0.02, n_outliers=0, seed=0),
    "8b": Spec("8b", 4096, 4096, 22, 8, 128, (16384,), 2048, seed=1),
    "27b": Spec("27b", 5120, 5120, 42, 8, 128, (65536,), 4096, seed=2),
    "27b_120k": Spec("27b_120k", 5120, 5120, 42, 8, 128, (122880,), 4096,
                     n_spans=64, seed=3),
    "8b_ragged_host": Spec("8b_ragged_host", 4096, 4096, 22, 8, 128,
                           (32768, 24576, 16384, 9216), 2048,
                           maps_on_host=True, seed=4),
}
CONFIG_ORDER = ["tiny", "8b", "27b", "27b_120k", "8b_ragged_host"]


def spec(name: str, **overrides) -> Spec:
    """A named spec, optionally with fields replaced (smaller parity cases)."""
    return replace(SPECS[name], **overrides)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Cast finite fp32 values to bf16 bit patterns, round-to-nearest-even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = u >> 16
    r &= 1
    r += u
    r += 0x7FFF
    r >>= 16
    return r.astype(np.uint16)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _normal(key, shape, sigma=1.0, mean=0.0) -> np.ndarray:
    z = _rng(*key).standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        z *= np.float32(sigma)
    if mean != 0.0:
        z += np.float32(mean)
    return z


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


@dataclass
class Workload:
    """bf16 bit patterns (uint16) for every input of one fill call."""
    spec: Spec
    x: np.ndarray                 # [n_rows][d_in]
    map_a: List[Optional[np.ndarray]]  # n_late x [d_out][d_in] (None for q8 maps)
    map_b: List[np.ndarray]       # n_late x [d_out]
    gamma: List[np.ndarray]       # n_late x [d_out]
    w_k: List[np.ndarray]         # n_late x [n_kv*head_dim][d_out]
    w_v: List[np.ndarray]         # n_late x [n_kv*head_dim][d_out]
    positions: np.ndarray         # int32 [n_rows]
    exact_rows: np.ndarray        # int32, ascending, unique
    outlier_channels: np.ndarray  # int64 [n_outliers]
    map_q: Optional[List[np.ndarray]] = None      # q8 only: n_late x int8 [d_out][d_in]
    map_scale: Optional[List[np.ndarray]] = None  # q8 only: n_late x bf16 [d_out][d_in/128]
    k_norm: Optional[List[np.ndarray]] = None     # qk_norm only: n_late x bf16 [head_dim]
    w_idx: Optional[List[np.ndarray]] = None      # idx_heads only: n_late x bf16 [idx_heads*hd][d_out]
    extra: dict = field(default_factory=dict)


def exact_row_list(s: Spec) -> np.ndarray:
    """The exact set: each prompt's last ``tail`` rows plus the seeded spans."""
    rows = []
    start = 0
    for n in s.prompt_lens:
        t = min(s.tail, n)
        rows.extend(range(start + n - t, start + n))
        start += n
    if s.n_spans:
        first = s.prompt_lens[0]
        hi = first - min(s.tail, first) - s.span_len  # last legal span start
        if hi < 0 or s.n_spans * s.span_len > hi + s.span_len:
            raise ValueError("spans do not fit in the first prompt's prefix")
        g = _rng(s.seed, _K_SPANS)
        taken: List[Tuple[int, int]] = []
        while len(taken) < s.n_spans:
            a = int(g.integers(0, hi + 1))
            b = a + s.span_len
            if any(a < e and s0 < b for s0, e in taken):
                continue
            taken.append((a, b))
        for a, b in taken:
            rows.extend(range(a, b))
    return np.array(sorted(set(rows)), dtype=np.int32)


def prompt_of_row(s: Spec) -> np.ndarray:
    """Index of the prompt (request) each row belongs to, int32 [n_rows]."""
    return np.concatenate([np.full(n, p, dtype=np.int32) for p, n in enumerate(s.prompt_lens)])


def calibration_row_list(s: Spec, c: int):
    """The first min(c, tail) rows of every prompt's tail and their prompt
    index: the rows a value rescale measures (int32 arrays, ascending)."""
    rows, grp = [], []
    start = 0
    for p, n in enumerate(s.prompt_lens):
        t = min(s.tail, n)
        k = min(c, t)
        rows.extend(range(start + n - t, start + n - t + k))
        grp.extend([p] * k)
        start += n
    return np.array(rows, dtype=np.int32), np.array(grp, dtype=np.int32)


def make_layer_truth(s: Spec, n: int, layers: Optional[List[int]] = None,
                     outliers: Optional[np.ndarray] = None) -> List[np.ndarray]:
    """Stand-ins for the true inputs of the late layers on n rows (bf16 bits
    [n][d_out] per layer): drawn like x_S, N(0, 1) with the outlier channels
    scaled, independently per layer."""
    out = []
    for l in (range(s.n_late) if layers is None else layers):
        v = _normal((s.seed, _K_TRUTH, l), (n, s.d_out))
        if outliers is not None and len(outliers):
            v[:, outliers[outliers < s.d_out]] *= np.float32(s.outlier_scale)
        out.append(f32_to_bf16_bits(v))
    return out


def _positions(s: Spec) -> np.ndarray:
    return np.concatenate([np.arange(n, dtype=np.int32) for n in s.prompt_lens])


def _gen_x_block(s: Spec, x: np.ndarray, blk: int, outliers: np.ndarray) -> None:
    r0 = blk * _X_BLOCK
    r1 = min(s.n_rows, r0 + _X_BLOCK)
    v = _normal((s.seed, _K_X, blk), (r1 - r0, s.d_in))
    if len(outliers):
        v[:, outliers] *= np.float32(s.outlier_scale)
    x[r0:r1] = f32_to_bf16_bits(v)


def _gen_q8_map(s: Spec, l: int):
    if s.d_in % Q8_BLOCK:
        raise ValueError(f"d_in={s.d_in} is not a multiple of {Q8_BLOCK}")
    nb = s.d_in // Q8_BLOCK
    k = min(s.d_in, s.d_out)
    z = _normal((s.seed, _K_LAYER, l, _L_QSCALE), (s.d_out, nb))
    scale = np.float32(s.map_sigma) * (np.float32(2.8) + np.float32(0.4) * np.abs(z))
    diag_rows = np.arange(k)
    scale[diag_rows, diag_rows // Q8_BLOCK] = np.float32(1.0) + np.float32(s.map_sigma) * z[diag_rows, diag_rows // Q8_BLOCK]
    scale /= np.float32(127.0)
    s_bits = f32_to_bf16_bits(scale)
    s_val = (s_bits.astype(np.uint32) << 16).view(np.float32)
    q = _normal((s.seed, _K_LAYER, l, _L_MAP), (s.d_out, s.d_in), s.map_sigma)
    q /= np.repeat(s_val, Q8_BLOCK, axis=1)
    np.rint(q, out=q)
    np.clip(q, -127, 127, out=q)
    q = q.astype(np.int8)
    q[diag_rows, diag_rows] = 127
    return q, s_bits


def _gen_layer(s: Spec, l: int):
    if s.map_format == "q8":
        a = None
    else:
        a = _normal((s.seed, _K_LAYER, l, _L_MAP), (s.d_out, s.d_in), s.map_sigma)
        k = min(s.d_in, s.d_out)
        a[np.arange(k), np.arange(k)] += np.float32(1.0)
    b = _normal((s.seed, _K_LAYER, l, _L_BIAS), (s.d_out,), s.bias_sigma)
    g = _normal((s.seed, _K_LAYER, l, _L_GAMMA), (s.d_out,), s.gamma_sigma, 1.0)
    wsig = 1.0 / np.sqrt(s.d_out)
    wk = _normal((s.seed, _K_LAYER, l, _L_WK), (s.kv_width, s.d_out), wsig)
    wv = _normal((s.seed, _K_LAYER, l, _L_WV), (s.kv_width, s.d_out), wsig)
    out = tuple(None if t is None else f32_to_bf16_bits(t) for t in (a, b, g, wk, wv))
    if s.map_format == "q8":
        out += _gen_q8_map(s, l)
    else:
        out += (None, None)
    if s.qk_norm:
        out += (f32_to_bf16_bits(_normal((s.seed, _K_LAYER, l, _L_KNORM), (s.head_dim,), s.gamma_sigma, 1.0)),)
    else:
        out += (None,)
    if s.idx_heads:
        out += (f32_to_bf16_bits(_normal((s.seed, _K_LAYER, l, _L_WIDX), (s.idx_heads * s.head_dim, s.d_out), wsig)),)
    else:
        out += (None,)
    return out


def make(s: Spec, layers: Optional[List[int]] = None) -> Workload:
    """Draw every input of ``s`` (all late layers unless ``layers`` is given)."""
    outliers = np.sort(_rng(s.seed, _K_OUTLIER).choice(s.d_in, s.n_outliers, replace=False)) \
        if s.n_outliers else np.zeros(0, dtype=np.int64)
    x = np.empty((s.n_rows, s.d_in), dtype=np.uint16)
    n_blk = (s.n_rows + _X_BLOCK - 1) // _X_BLOCK
    layer_ids = list(range(s.n_late)) if layers is None else list(layers)
    with ThreadPoolExecutor(_threads()) as ex:
        futs = [ex.submit(_gen_x_block, s, x, i, outliers) for i in range(n_blk)]
        lay = list(ex.map(lambda l: _gen_layer(s, l), layer_ids))
        for f in futs:
            f.result()
    return Workload(
        spec=s, x=x,
        map_a=[t[0] for t in lay], map_b=[t[1] for t in lay], gamma=[t[2] for t in lay],
        w_k=[t[3] for t in lay], w_v=[t[4] for t in lay],
        positions=_positions(s), exact_rows=exact_row_list(s),
        outlier_channels=outliers,
        map_q=[t[5] for t in lay] if s.map_format == "q8" else None,
        map_scale=[t[6] for t in lay] if s.map_format == "q8" else None,
        k_norm=[t[7] for t in lay] if s.qk_norm else None,
        w_idx=[t[8] for t in lay] if s.idx_heads else None)
