"""Helpers for the GPU tests: upload a workload, run the library, compare.

Inputs come from ``workloads``; expected values come from ``oracle``; the
device results come from librf through ``late_layer_kv_amd.binding``.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from late_layer_kv_amd import binding as B

CANARY = 0x7FC1          # a bf16 NaN pattern the fill never produces
FRO_TOL = 5e-3           # Frobenius relative error bound per layer, K and V separately
MAXEL_TOL = 3e-2         # max element error, floored by the reference head vector's RMS
BF16_ONE = 0x3F80


def t16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16))


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32)))


def bits_to_f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_bits_to_f64(t.cpu().numpy().view(np.uint16))


class DeviceInputs:
    """A workload's inputs in device memory (maps in pinned host memory if asked)."""

    def __init__(self, w, maps_on_host: bool = None, device: str = "cuda:0"):
        s = w.spec
        self.w = w
        self.device = device
        host = s.maps_on_host if maps_on_host is None else maps_on_host
        self.maps_on_host = host
        self.x = t16(w.x).to(device)
        place = (lambda t: t.pin_memory()) if host else (lambda t: t.to(device))
        self.q8 = w.map_q is not None
        if self.q8:
            self.map_a = None
            self.map_q = [place(torch.from_numpy(np.ascontiguousarray(q))) for q in w.map_q]
            self.map_scale = [place(t16(sc)) for sc in w.map_scale]
        else:
            self.map_a = [place(t16(a)) for a in w.map_a]
        self.map_b = [place(t16(b)) for b in w.map_b]
        self.gamma = [t16(g).to(device) for g in w.gamma]
        self.w_k = [t16(a).to(device) for a in w.w_k]
        self.w_v = [t16(a).to(device) for a in w.w_v]
        self.positions = i32(w.positions).to(device)
        self.exact = i32(w.exact_rows).to(device)
        self.k_norm = None if w.k_norm is None else [t16(g).to(device) for g in w.k_norm]
        self.w_idx = None if w.w_idx is None else [t16(a).to(device) for a in w.w_idx]

    def caches(self):
        s = self.w.spec
        mk = lambda: [torch.full((s.n_rows, s.kv_width), CANARY, dtype=torch.int16, device=self.device)
                      for _ in range(s.n_late)]
        return mk(), mk()

    def idx_caches(self):
        s = self.w.spec
        return [torch.full((s.n_rows, s.idx_heads * s.head_dim), CANARY, dtype=torch.int16, device=self.device)
                for _ in range(s.n_late)]


def plan_for(w, **kw) -> B.Plan:
    return B.Plan.for_spec(w.spec, **kw)


def gpu_fill_rows(plan, di: DeviceInputs, exact: torch.Tensor = None):
    s = di.w.spec
    ex = di.exact if exact is None else exact
    out = torch.full((max(s.n_rows, 1),), -7, dtype=torch.int32, device=di.device)
    nf = torch.zeros(1, dtype=torch.int32, device=di.device)
    ws = torch.empty(B.fill_rows_workspace_bytes(s.n_rows), dtype=torch.uint8, device=di.device)
    B.fill_rows(plan, ex, out, nf, ws)
    torch.cuda.synchronize()
    n = int(nf.item())
    return out[:n].clone(), n


def gpu_fill(plan, di: DeviceInputs, rows: torch.Tensor, n_fill: int, caches=None, layers_per_launch=None,
             map_a=None, map_b=None, rope=None, slots=None, vscale=None, idx_caches=None, w_idx=None, measure=None):
    """(K caches, V caches), plus the indexer-key caches when the workload has
    indexer heads."""
    s = di.w.spec
    kc, vc = di.caches() if caches is None else caches
    ic = None
    if di.w_idx is not None:
        ic = di.idx_caches() if idx_caches is None else idx_caches
    wi = di.w_idx if w_idx is None else w_idx
    g = s.n_late if layers_per_launch is None else layers_per_launch
    ws = torch.empty(max(plan.fill_workspace_bytes(n_fill, g), 256), dtype=torch.uint8, device=di.device)
    if di.q8 and map_a is None:
        B.fill_q8(plan, di.x, rows, n_fill, di.positions, slots, di.map_q, di.map_scale,
                  di.map_b if map_b is None else map_b, di.gamma, di.w_k, di.w_v, rope, kc, vc, ws, vscale=vscale,
                  k_norm=di.k_norm, w_idx=wi, idx_cache=ic, measure=measure)
    else:
        B.fill(plan, di.x, rows, n_fill, di.positions, slots, di.map_a if map_a is None else map_a,
               di.map_b if map_b is None else map_b, di.gamma, di.w_k, di.w_v, rope, kc, vc, ws, vscale=vscale,
               k_norm=di.k_norm, w_idx=wi, idx_cache=ic, measure=measure)
    torch.cuda.synchronize()
    return (kc, vc) if ic is None else (kc, vc, ic)


def gpu_kv_project(plan, di: DeviceInputs, layer_in, rows: torch.Tensor, n: int, caches=None, slots=None):
    s = di.w.spec
    kc, vc = di.caches() if caches is None else caches
    ic = None if di.w_idx is None else di.idx_caches()
    ws = torch.empty(plan.kv_project_workspace_bytes(s.n_late), dtype=torch.uint8, device=di.device)
    B.kv_project(plan, layer_in, rows, n, di.positions, slots, di.gamma, di.w_k, di.w_v, None, kc, vc, ws,
                 k_norm=di.k_norm, w_idx=di.w_idx, idx_cache=ic)
    torch.cuda.synchronize()
    return (kc, vc) if ic is None else (kc, vc, ic)


def kv_errors(got: np.ndarray, ref: np.ndarray, head_dim: int):
    """(Frobenius relative, max floored element, inf-norm ratio) of got vs ref."""
    n, width = ref.shape
    d = got - ref
    fro = np.linalg.norm(d) / np.linalg.norm(ref)
    rh = ref.reshape(n, width // head_dim, head_dim)
    rms = np.sqrt(np.mean(rh * rh, axis=2, keepdims=True))
    floor = np.maximum(np.abs(rh), rms)
    maxel = float(np.max(np.abs(d.reshape(rh.shape)) / floor))
    inf = float(np.max(np.abs(d)) / np.max(np.abs(ref)))
    return float(fro), maxel, inf


# Checked-row counts of the full-size parity runs, printed at the end of the
# test session (tests/conftest.py), so they show under pytest -q as well.
RECORDS = []


class ValueCheck:
    """The fill's value tolerance over rows given in chunks: per layer and for
    K and V separately, the Frobenius relative error over every row checked
    (squared norms accumulated across chunks), the floored max element error
    and the inf-norm ratio."""

    def __init__(self, head_dim: int):
        self.hd = head_dim
        self.acc = {}   # (layer, name) -> [sum d^2, sum r^2, max floored, max |d|, max |r|]
        self.rows = 0

    def add(self, caches: dict, ref: dict, rows: np.ndarray, slots: np.ndarray = None):
        """caches: {"K": list, "V": list, ...}; ref: {layer: {name: array [len(rows)][width]}}."""
        sl = rows if slots is None else slots[rows]
        idx = torch.from_numpy(np.asarray(sl, dtype=np.int64)).to(next(iter(caches.values()))[0].device)
        for l, per in ref.items():
            for name, r in per.items():
                got = bits_to_f64(caches[name][l].index_select(0, idx))
                d = got - r
                n, width = r.shape
                rh = r.reshape(n, width // self.hd, self.hd)
                floor = np.maximum(np.abs(rh), np.sqrt(np.mean(rh * rh, axis=2, keepdims=True)))
                a = self.acc.setdefault((l, name), [0.0, 0.0, 0.0, 0.0, 0.0])
                a[0] += float(np.sum(d * d))
                a[1] += float(np.sum(r * r))
                a[2] = max(a[2], float(np.max(np.abs(d.reshape(rh.shape)) / floor)))
                a[3] = max(a[3], float(np.max(np.abs(d))))
                a[4] = max(a[4], float(np.max(np.abs(r))))
        self.rows += len(rows)
        return self

    def finish(self):
        worst = {"fro": 0.0, "maxel": 0.0, "inf": 0.0}
        for (l, name), (d2, r2, maxel, md, mr) in sorted(self.acc.items()):
            fro = float(np.sqrt(d2 / r2))
            worst["fro"] = max(worst["fro"], fro)
            worst["maxel"] = max(worst["maxel"], maxel)
            worst["inf"] = max(worst["inf"], md / mr)
            assert fro <= FRO_TOL, f"layer {l} {name}: Frobenius relative error {fro:.3e}"
            assert maxel <= MAXEL_TOL, f"layer {l} {name}: max element error {maxel:.3e}"
        return worst


def check_values(kc, vc, ref: dict, rows: np.ndarray, head_dim: int, slots: np.ndarray = None):
    """Compare cache rows at slot(rows) with the oracle, per layer, K and V."""
    chk = ValueCheck(head_dim)
    chk.add({"K": kc, "V": vc}, {l: {"K": rk, "V": rv} for l, (rk, rv) in ref.items()}, rows, slots)
    return chk.finish()


def check_placement(kc, vc, fill_rows: np.ndarray, n_slots: int, slots: np.ndarray = None, ic=None):
    """Bit-exact placement: written slots are exactly slot(fill rows); every
    other slot still holds the canary in every byte (K, V and, if given, the
    indexer keys)."""
    filled = np.zeros(n_slots, dtype=bool)
    filled[fill_rows if slots is None else slots[fill_rows]] = True
    want = torch.from_numpy(filled).to(kc[0].device)
    for l in range(len(kc)):
        for name, cache in (("K", kc), ("V", vc)) + ((("I", ic),) if ic is not None else ()):
            eq = cache[l] == CANARY
            untouched = eq.all(dim=1)
            anyc = eq.any(dim=1)
            assert torch.equal(untouched, ~want), f"layer {l} {name}: slots outside the fill set were written"
            assert not torch.any(anyc & want), f"layer {l} {name}: a filled slot still holds canary bytes"


def identity_maps(di: DeviceInputs):
    """A = I, b = 0 for every late layer, on the device."""
    s = di.w.spec
    eye = torch.zeros((s.d_out, s.d_in), dtype=torch.int16)
    k = min(s.d_in, s.d_out)
    eye[torch.arange(k), torch.arange(k)] = BF16_ONE
    a = [eye.to(di.device) for _ in range(s.n_late)]
    b = [torch.zeros(s.d_out, dtype=torch.int16, device=di.device) for _ in range(s.n_late)]
    return a, b


def check_indexer_values(ic, ref: dict, rows: np.ndarray, head_dim: int, slots: np.ndarray = None):
    """Compare indexer-key cache rows at slot(rows) with the oracle, per layer."""
    sl = rows if slots is None else slots[rows]
    idx = torch.from_numpy(np.asarray(sl, dtype=np.int64)).to(ic[0].device)
    worst = {"fro": 0.0, "maxel": 0.0, "inf": 0.0}
    for l, r in ref.items():
        got = bits_to_f64(ic[l].index_select(0, idx))
        fro, maxel, inf = kv_errors(got, r, head_dim)
        worst = {k: max(worst[k], v) for k, v in (("fro", fro), ("maxel", maxel), ("inf", inf))}
        assert fro <= FRO_TOL, f"layer {l} indexer keys: Frobenius relative error {fro:.3e}"
        assert maxel <= MAXEL_TOL, f"layer {l} indexer keys: max element error {maxel:.3e}"
    return worst
