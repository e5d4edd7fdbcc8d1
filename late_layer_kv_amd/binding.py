"""ctypes binding of librf.so (include/rf.h).

Argument marshalling only: every step of the fill runs in the HIP kernels of
the library.  Tensors are torch tensors (device memory, or pinned host memory
for streamed maps); bf16 data may be given as torch.bfloat16 or as int16 /
uint16 bit patterns.  Work goes on torch's current HIP stream unless a stream
is passed.  If the library is not built this module raises on first use; there
is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import List, Optional, Sequence

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librf.so")

RF_MAPS_HOST = 1
RF_VALIDATE = 2
RF_MAPS_Q8 = 4
RF_RIDGE_RAW = 1
RF_STREAM_GROUP = 4  # most layers per launch with streamed maps (include/rf.h)
RF_NOALLOC_MAX_ROWS = 1 << 20  # rows rf_fill_rows_noalloc takes (include/rf.h)
Q8_BLOCK = 128

STATUS = {0: "RF_OK", -1: "RF_E_ARG", -2: "RF_E_SHAPE", -3: "RF_E_ROWS", -4: "RF_E_WORKSPACE",
          -5: "RF_E_HIP", -6: "RF_E_LINALG"}

# Every symbol include/rf.h declares.
EXPORTS = [
    "rf_plan_create", "rf_plan_destroy", "rf_fill_workspace_bytes", "rf_kv_project_workspace_bytes",
    "rf_rope_table", "rf_fill_rows_workspace_bytes", "rf_fill_rows", "rf_fill", "rf_kv_project",
    "rf_ridge_acc_create", "rf_ridge_acc_add", "rf_ridge_solve", "rf_ridge_acc_destroy", "rf_ridge_fit",
    "rf_plan_profile", "rf_plan_profile_read", "rf_last_error",
    "rf_fill_q8", "rf_map_dequantize_q8", "rf_map_quantize_q8",
    "rf_value_scales_workspace_bytes", "rf_value_scales", "rf_value_scales_q8",
    "rf_ridge_dev_create", "rf_ridge_dev_add", "rf_ridge_dev_merge", "rf_ridge_dev_destroy", "rf_ridge_acc_sums",
    "rf_ridge_dev_solve_workspace_bytes", "rf_ridge_dev_solve", "rf_fill_rows_noalloc",
]

KERNEL_KINDS = ["map", "kv", "prep", "rope", "rows", "copy", "dequant", "scale", "norm"]


class RfError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {msg}")
        self.status = status


class Shape(C.Structure):
    _fields_ = [("d_in", C.c_int32), ("d_out", C.c_int32), ("n_late", C.c_int32), ("n_kv", C.c_int32),
                ("head_dim", C.c_int32), ("rms_eps", C.c_float), ("rope_theta", C.c_double),
                ("n_rows", C.c_int32), ("n_slots", C.c_int32), ("max_pos", C.c_int32), ("n_idx", C.c_int32)]


class Profile(C.Structure):
    _fields_ = [("ms", C.c_double * len(KERNEL_KINDS)), ("launches", C.c_int64 * len(KERNEL_KINDS))]


class VScale(C.Structure):
    """rf_vscale: per-request value scales applied by the fill."""
    _fields_ = [("scale", C.c_void_p), ("group_of_row", C.c_void_p), ("n_groups", C.c_int32)]


class VMeasure(C.Structure):
    """rf_vmeasure: the value-scale measurement run inside a fill."""
    _fields_ = [("layer_in", C.POINTER(C.c_void_p)), ("ld_in", C.c_int64), ("calib_rows", C.c_void_p),
                ("calib_group", C.c_void_p), ("n_calib", C.c_int32), ("group_of_row", C.c_void_p),
                ("n_groups", C.c_int32), ("scale", C.c_void_p), ("workspace", C.c_void_p), ("ws_bytes", C.c_size_t)]


class FillOpts(C.Structure):
    """rf_fill_opts: value rescale, QK-norm, indexer keys and in-fill measurement of a fill."""
    _fields_ = [("vscale", C.POINTER(VScale)), ("k_norm", C.POINTER(C.c_void_p)),
                ("w_idx", C.POINTER(C.c_void_p)), ("idx_cache", C.POINTER(C.c_void_p)),
                ("measure", C.POINTER(VMeasure))]


_lib = None
P = C.c_void_p
PP = C.POINTER(C.c_void_p)


def lib():
    """Load librf.so (built in-tree by late_layer_kv_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m late_layer_kv_amd.build`")
    L = C.CDLL(LIB_PATH)
    i32, i64, sz, dbl = C.c_int32, C.c_int64, C.c_size_t, C.c_double
    sig = {
        "rf_plan_create": (i32, [C.POINTER(Shape), i32, C.POINTER(P)]),
        "rf_plan_destroy": (None, [P]),
        "rf_fill_workspace_bytes": (sz, [P, i32, i32]),
        "rf_kv_project_workspace_bytes": (sz, [P, i32]),
        "rf_rope_table": (i32, [P, P, P]),
        "rf_fill_rows_workspace_bytes": (sz, [i32]),
        "rf_fill_rows": (i32, [P, P, i32, P, P, P, sz, P]),
        "rf_fill_rows_noalloc": (i32, [P, P, i32, P, P, P]),
        "rf_fill": (i32, [P, P, i64, P, i32, P, P, PP, PP, PP, PP, PP, P, PP, PP, P, P, sz, P]),
        "rf_kv_project": (i32, [P, PP, i64, P, i32, P, P, PP, PP, PP, P, PP, PP, P, P, sz, P]),
        "rf_ridge_acc_create": (i32, [i32, i32, C.POINTER(P)]),
        "rf_ridge_acc_add": (i32, [P, P, P, i64]),
        "rf_ridge_solve": (i32, [P, dbl, i32, P, P]),
        "rf_ridge_acc_destroy": (None, [P]),
        "rf_ridge_fit": (i32, [P, P, i64, i32, i32, dbl, i32, P, P]),
        "rf_plan_profile": (i32, [P, i32]),
        "rf_plan_profile_read": (i32, [P, C.POINTER(Profile)]),
        "rf_last_error": (C.c_char_p, []),
        "rf_fill_q8": (i32, [P, P, i64, P, i32, P, P, PP, PP, PP, PP, PP, PP, P, PP, PP, P, P, sz, P]),
        "rf_value_scales_workspace_bytes": (sz, [P, i32, i32]),
        "rf_ridge_dev_create": (i32, [i32, i32, C.POINTER(P)]),
        "rf_ridge_dev_add": (i32, [P, P, i64, P, i64, i64, P]),
        "rf_ridge_dev_merge": (i32, [P, P, P]),
        "rf_ridge_dev_destroy": (None, [P]),
        "rf_ridge_acc_sums": (i32, [P, P, P, P, P, P]),
        "rf_ridge_dev_solve_workspace_bytes": (sz, [P]),
        "rf_ridge_dev_solve": (i32, [P, dbl, i32, P, P, P, sz, P]),
        "rf_value_scales": (i32, [P, P, i64, PP, i64, P, P, i32, i32, PP, PP, PP, PP, P, P, sz, P]),
        "rf_value_scales_q8": (i32, [P, P, i64, PP, i64, P, P, i32, i32, PP, PP, PP, PP, PP, P, P, sz, P]),
        "rf_map_dequantize_q8": (i32, [P, P, i32, i32, P, P]),
        "rf_map_quantize_q8": (i32, [P, i32, i32, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def last_error() -> str:
    return lib().rf_last_error().decode()


def _check(fn: str, st: int) -> None:
    if st != 0:
        raise RfError(fn, st, last_error())


def _ptr(t) -> Optional[int]:
    """Data pointer of a tensor (None passes NULL)."""
    if t is None:
        return None
    return t.data_ptr()


def _ptr_array(ts: Sequence) -> C.Array:
    arr = (C.c_void_p * len(ts))()
    for i, t in enumerate(ts):
        arr[i] = t if isinstance(t, int) else t.data_ptr()
    return arr


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---- host-side argument checks ---------------------------------------------
# The library receives bare pointers, so it cannot see a tensor that is too
# small, of the wrong type or in the wrong memory; the kernels would then read
# or write past its end.  Every tensor argument is checked here, before
# anything is enqueued, against the sizes the plan fixes.  A failed check
# raises ValueError.

DEVICE_TYPE = "cuda"   # where device arguments must live (torch's name for HIP devices)
_BF16 = ("int16", "uint16", "bfloat16")


def _dtype(t) -> str:
    return str(t.dtype).replace("torch.", "")


def _arg(fn: str, name: str, t, dtypes, numel: int = 0, where: str = "device", optional: bool = False):
    """t must be a tensor of one of `dtypes` holding at least `numel` elements,
    with unit stride along its last axis, in device memory (where="device") or
    pinned host memory (where="pinned")."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{fn}: {name} is required")
    if not hasattr(t, "data_ptr") or not hasattr(t, "dtype"):
        raise ValueError(f"{fn}: {name} must be a tensor, got {type(t).__name__}")
    if _dtype(t) not in dtypes:
        raise ValueError(f"{fn}: {name} has dtype {_dtype(t)}, expected one of {', '.join(dtypes)}")
    if where == "device" and t.device.type != DEVICE_TYPE:
        raise ValueError(f"{fn}: {name} must be in device memory, not on {t.device}")
    if where == "pinned" and (t.device.type != "cpu" or not t.is_pinned()):
        raise ValueError(f"{fn}: {name} must be in pinned host memory (the plan streams its maps)")
    if t.dim() > 0 and t.numel() > 0 and t.stride(-1) != 1:   # an empty tensor has no layout to check
        raise ValueError(f"{fn}: {name} must have unit stride along its last axis")
    if t.numel() < numel:
        raise ValueError(f"{fn}: {name} holds {t.numel()} elements, at least {numel} needed")


def _rows_arg(fn: str, name: str, t, rows: int, cols: int, ld: Optional[int], where: str = "device"):
    """A row-major bf16 matrix of `rows` rows of which the first `cols`
    columns are read, rows `ld` elements apart (default: its row stride)."""
    _arg(fn, name, t, _BF16, 0, where)
    if t.dim() != 2:
        raise ValueError(f"{fn}: {name} must be 2-D [rows][columns]")
    ld = t.stride(0) if ld is None else ld
    if ld < cols:
        raise ValueError(f"{fn}: {name} rows are {ld} elements apart, fewer than the {cols} read")
    need = (rows - 1) * ld + cols if rows > 0 else 0
    span = (t.shape[0] - 1) * t.stride(0) + t.shape[1] if t.numel() else 0
    if span < need:
        raise ValueError(f"{fn}: {name} covers {span} elements, {need} needed for {rows} rows of {cols}")


def _layers(fn: str, name: str, ts, n_late: int, dtypes, numel: int, where: str = "device", shape=None):
    """One tensor per late layer; with `shape`, a 2-D tensor must have exactly
    that shape and be contiguous (maps: [d_out][d_in], so a transposed map is
    refused rather than read the wrong way round)."""
    if ts is None or len(ts) != n_late:
        raise ValueError(f"{fn}: {name} must hold one tensor per late layer ({n_late})")
    for i, t in enumerate(ts):
        _arg(fn, f"{name}[{i}]", t, dtypes, numel, where)
        if shape is not None and t.dim() == 2 and (tuple(t.shape) != tuple(shape) or not t.is_contiguous()):
            raise ValueError(f"{fn}: {name}[{i}] is {tuple(t.shape)}"
                             f"{'' if t.is_contiguous() else ' (not contiguous)'}, expected contiguous "
                             f"{tuple(shape)} = [d_out][d_in]")


def _workspace(fn: str, ws):
    _arg(fn, "workspace", ws, ("uint8", "int8", "int16", "int32", "float32", "float16", "bfloat16", "float64",
                                "int64", "uint16", "uint32"), 0)


def _check_fill(fn: str, plan: "Plan", x, ld_x, fill_rows_t, n_fill, positions, slot_of_row, maps, map_b, gamma,
                w_k, w_v, rope, k_cache, v_cache, workspace, vscale, k_norm, w_idx, idx_cache, measure):
    sh = plan.shape
    L, d_in, d_out = sh.n_late, sh.d_in, sh.d_out
    mw = "pinned" if plan.maps_on_host else "device"
    if not 0 <= n_fill <= sh.n_rows:
        raise ValueError(f"{fn}: n_fill={n_fill} outside [0, n_rows={sh.n_rows}]")
    _rows_arg(fn, "x", x, sh.n_rows, d_in, ld_x)
    _arg(fn, "fill_rows", fill_rows_t, ("int32",), n_fill)
    _arg(fn, "positions", positions, ("int32",), sh.n_rows)
    _arg(fn, "slot_of_row", slot_of_row, ("int32",), sh.n_rows, optional=True)
    if plan.maps_q8:
        map_q, map_scale = maps
        _layers(fn, "map_q", map_q, L, ("int8",), d_out * d_in, mw, (d_out, d_in))
        _layers(fn, "map_scale", map_scale, L, _BF16, d_out * (d_in // Q8_BLOCK), mw, (d_out, d_in // Q8_BLOCK))
    else:
        _layers(fn, "map_a", maps, L, _BF16, d_out * d_in, mw, (d_out, d_in))
    _layers(fn, "map_b", map_b, L, _BF16, d_out, mw)
    _layers(fn, "gamma", gamma, L, _BF16, d_out)
    _layers(fn, "w_k", w_k, L, _BF16, plan.kv_width * d_out)
    _layers(fn, "w_v", w_v, L, _BF16, plan.kv_width * d_out)
    _arg(fn, "rope", rope, ("float32",), sh.max_pos * sh.head_dim, optional=True)
    _layers(fn, "k_cache", k_cache, L, _BF16, sh.n_slots * plan.kv_width)
    _layers(fn, "v_cache", v_cache, L, _BF16, sh.n_slots * plan.kv_width)
    _workspace(fn, workspace)
    if k_norm is not None:
        _layers(fn, "k_norm", k_norm, L, _BF16, sh.head_dim)
    if w_idx is not None:
        _layers(fn, "w_idx", w_idx, L, _BF16, plan.idx_width * d_out)
    if idx_cache is not None:
        _layers(fn, "idx_cache", idx_cache, L, _BF16, sh.n_slots * plan.idx_width)
    if vscale is not None:
        scale, group_of_row, n_groups = vscale
        _arg(fn, "vscale scale", scale, ("float32",), L * max(n_groups, 1) * sh.n_kv)
        _arg(fn, "vscale group_of_row", group_of_row, ("int32",), sh.n_rows)
    if measure is not None:
        layer_in, calib_rows, calib_group, group_of_row, n_groups, scale, ws = measure
        _check_measure(fn, plan, layer_in, None, calib_rows, calib_group, n_groups, scale)
        _arg(fn, "measure group_of_row", group_of_row, ("int32",), sh.n_rows)
        _workspace(fn, ws)


def _check_measure(fn, plan, layer_in, ld_in, calib_rows, calib_group, n_groups, scale):
    sh = plan.shape
    _arg(fn, "calib_rows", calib_rows, ("int32",), 0)
    n = calib_rows.numel()
    _arg(fn, "calib_group", calib_group, ("int32",), n)
    if layer_in is None or len(layer_in) != sh.n_late:
        raise ValueError(f"{fn}: layer_in must hold one tensor per late layer ({sh.n_late})")
    for i, t in enumerate(layer_in):
        _rows_arg(fn, f"layer_in[{i}]", t, n, sh.d_out, ld_in)
    _arg(fn, "scale", scale, ("float32",), sh.n_late * max(n_groups, 1) * sh.n_kv)


class Plan:
    """An rf_plan for one shape (see rf_plan_create)."""

    def __init__(self, d_in: int, d_out: int, n_late: int, n_kv: int, head_dim: int, rms_eps: float,
                 rope_theta: float, n_rows: int, n_slots: int, max_pos: int,
                 maps_on_host: bool = False, validate: bool = False, maps_q8: bool = False, n_idx: int = 0):
        self.shape = Shape(d_in, d_out, n_late, n_kv, head_dim, rms_eps, rope_theta, n_rows, n_slots, max_pos,
                           n_idx)
        self.flags = ((RF_MAPS_HOST if maps_on_host else 0) | (RF_VALIDATE if validate else 0)
                      | (RF_MAPS_Q8 if maps_q8 else 0))
        self.maps_on_host, self.maps_q8 = bool(maps_on_host), bool(maps_q8)
        self.kv_width, self.idx_width = n_kv * head_dim, n_idx * head_dim
        h = C.c_void_p()
        _check("rf_plan_create", lib().rf_plan_create(C.byref(self.shape), self.flags, C.byref(h)))
        self.handle = h

    @classmethod
    def for_spec(cls, s, **kw) -> "Plan":
        """Plan for a workloads.Spec."""
        kw.setdefault("maps_on_host", s.maps_on_host)
        kw.setdefault("maps_q8", s.map_format == "q8")
        kw.setdefault("n_idx", s.idx_heads)
        return cls(s.d_in, s.d_out, s.n_late, s.n_kv, s.head_dim, s.rms_eps, s.rope_theta,
                   s.n_rows, s.n_rows, s.max_pos, **kw)

    def close(self) -> None:
        if self.handle:
            lib().rf_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def fill_workspace_bytes(self, n_fill: int, layers_per_launch: int = 1) -> int:
        return int(lib().rf_fill_workspace_bytes(self.handle, n_fill, layers_per_launch))

    def value_scales_workspace_bytes(self, n_calib: int, layers_per_launch: int = 1) -> int:
        return int(lib().rf_value_scales_workspace_bytes(self.handle, n_calib, layers_per_launch))

    def kv_project_workspace_bytes(self, layers_per_launch: int = 1) -> int:
        return int(lib().rf_kv_project_workspace_bytes(self.handle, layers_per_launch))

    def profile(self, enable: bool) -> None:
        """Bracket every launch of this plan with HIP events (rf_plan_profile)."""
        _check("rf_plan_profile", lib().rf_plan_profile(self.handle, 1 if enable else 0))

    def profile_read(self) -> dict:
        """{kind: (milliseconds, launches)} since the last read (rf_plan_profile_read)."""
        pr = Profile()
        _check("rf_plan_profile_read", lib().rf_plan_profile_read(self.handle, C.byref(pr)))
        return {k: (pr.ms[i], int(pr.launches[i])) for i, k in enumerate(KERNEL_KINDS)}


def fill_rows_workspace_bytes(n_rows: int) -> int:
    return int(lib().rf_fill_rows_workspace_bytes(n_rows))


def rope_table(plan: Plan, table, stream=None) -> None:
    _arg("rf_rope_table", "table", table, ("float32",), plan.shape.max_pos * plan.shape.head_dim)
    _check("rf_rope_table", lib().rf_rope_table(plan.handle, _ptr(table), _stream(stream)))


def fill_rows(plan: Plan, exact_rows, fill_rows_out, n_fill_out, workspace, stream=None) -> None:
    n_exact = 0 if exact_rows is None else exact_rows.numel()
    _arg("rf_fill_rows", "exact_rows", exact_rows, ("int32",), 0, optional=True)
    _arg("rf_fill_rows", "fill_rows_out", fill_rows_out, ("int32",), plan.shape.n_rows)
    _arg("rf_fill_rows", "n_fill_out", n_fill_out, ("int32",), 1)
    _workspace("rf_fill_rows", workspace)
    _check("rf_fill_rows", lib().rf_fill_rows(plan.handle, _ptr(exact_rows), n_exact, _ptr(fill_rows_out),
                                              _ptr(n_fill_out), _ptr(workspace), workspace.numel() *
                                              workspace.element_size(), _stream(stream)))


def fill_rows_noalloc(plan: Plan, exact_rows, fill_rows_out, n_fill_out, stream=None) -> None:
    """rf_fill_rows_noalloc: rf_fill_rows with the library's own scratch array
    (no workspace; plans of at most RF_NOALLOC_MAX_ROWS rows)."""
    n_exact = 0 if exact_rows is None else exact_rows.numel()
    _arg("rf_fill_rows_noalloc", "exact_rows", exact_rows, ("int32",), 0, optional=True)
    _arg("rf_fill_rows_noalloc", "fill_rows_out", fill_rows_out, ("int32",), plan.shape.n_rows)
    _arg("rf_fill_rows_noalloc", "n_fill_out", n_fill_out, ("int32",), 1)
    _check("rf_fill_rows_noalloc", lib().rf_fill_rows_noalloc(plan.handle, _ptr(exact_rows), n_exact,
                                                              _ptr(fill_rows_out), _ptr(n_fill_out),
                                                              _stream(stream)))


class _Opts:
    """Keeps an rf_fill_opts and everything it points to alive for one call."""

    def __init__(self, vscale=None, k_norm=None, w_idx=None, idx_cache=None, measure=None):
        self.ref = None
        if vscale is None and k_norm is None and w_idx is None and idx_cache is None and measure is None:
            return
        self.opts = FillOpts()
        if vscale is not None:
            scale, group_of_row, n_groups = vscale
            self.vs = VScale(scale.data_ptr(), group_of_row.data_ptr(), n_groups)
            self.opts.vscale = C.pointer(self.vs)
        if k_norm is not None:
            self.kn = _ptr_array(k_norm)
            self.opts.k_norm = C.cast(self.kn, C.POINTER(C.c_void_p))
        if w_idx is not None:
            self.wi = _ptr_array(w_idx)
            self.opts.w_idx = C.cast(self.wi, C.POINTER(C.c_void_p))
        if idx_cache is not None:
            self.ic = _ptr_array(idx_cache)
            self.opts.idx_cache = C.cast(self.ic, C.POINTER(C.c_void_p))
        if measure is not None:
            # (layer_in list, calib_rows, calib_group, group_of_row, n_groups, scale out, workspace)
            layer_in, calib_rows, calib_group, group_of_row, n_groups, scale, ws = measure
            self.li = _ptr_array(layer_in)
            self.vm = VMeasure(C.cast(self.li, C.POINTER(C.c_void_p)), layer_in[0].stride(0), _ptr(calib_rows),
                               _ptr(calib_group), calib_rows.numel(), _ptr(group_of_row), n_groups, _ptr(scale),
                               _ptr(ws), ws.numel() * ws.element_size())
            self.opts.measure = C.pointer(self.vm)
        self.ref = C.byref(self.opts)


def fill(plan: Plan, x, fill_rows_t, n_fill: int, positions, slot_of_row, map_a: Sequence, map_b: Sequence,
         gamma: Sequence, w_k: Sequence, w_v: Sequence, rope, k_cache: Sequence, v_cache: Sequence,
         workspace, stream=None, ld_x: Optional[int] = None, vscale=None, k_norm: Sequence = None,
         w_idx: Sequence = None, idx_cache: Sequence = None, measure=None) -> None:
    """rf_fill.  map_a/map_b are device tensors, or pinned host tensors for a
    plan made with maps_on_host.  vscale = (scale [n_late][n_groups][n_kv] fp32,
    group_of_row [n_rows] int32, n_groups) applies a value rescale; k_norm (one
    bf16 [head_dim] gain per late layer) applies QK-norm to the keys; w_idx /
    idx_cache (per late layer) write the indexer keys of a plan with n_idx > 0;
    measure = (layer_in, calib_rows, calib_group, group_of_row, n_groups, scale,
    workspace) measures the value scales inside the fill and applies them.

    map_a[l] is A_l [d_out][d_in], the map in the paper's orientation
    (y = A_l x + b_l, RidgeFill section 2.2), which is W_l transposed for the
    row-vector form Y = X W_l + b_l; rf_ridge_fit returns A_l.  A caller
    holding W_l [d_in][d_out] passes W_l.T made contiguous."""
    _check_fill("rf_fill", plan, x, ld_x, fill_rows_t, n_fill, positions, slot_of_row, map_a, map_b, gamma, w_k,
                w_v, rope, k_cache, v_cache, workspace, vscale, k_norm, w_idx, idx_cache, measure)
    ld = x.stride(0) if ld_x is None else ld_x
    o = _Opts(vscale, k_norm, w_idx, idx_cache, measure)
    _check("rf_fill", lib().rf_fill(
        plan.handle, _ptr(x), ld, _ptr(fill_rows_t), n_fill, _ptr(positions), _ptr(slot_of_row),
        _ptr_array(map_a), _ptr_array(map_b), _ptr_array(gamma), _ptr_array(w_k), _ptr_array(w_v),
        _ptr(rope), _ptr_array(k_cache), _ptr_array(v_cache), o.ref, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def fill_q8(plan: Plan, x, fill_rows_t, n_fill: int, positions, slot_of_row, map_q: Sequence,
            map_scale: Sequence, map_b: Sequence, gamma: Sequence, w_k: Sequence, w_v: Sequence, rope,
            k_cache: Sequence, v_cache: Sequence, workspace, stream=None, ld_x: Optional[int] = None,
            vscale=None, k_norm: Sequence = None, w_idx: Sequence = None, idx_cache: Sequence = None,
            measure=None) -> None:
    """rf_fill_q8: the fill with int8 maps (codes + bf16 block scales) for a
    plan made with maps_q8; pinned host tensors for a plan with maps_on_host."""
    _check_fill("rf_fill_q8", plan, x, ld_x, fill_rows_t, n_fill, positions, slot_of_row, (map_q, map_scale), map_b,
                gamma, w_k, w_v, rope, k_cache, v_cache, workspace, vscale, k_norm, w_idx, idx_cache, measure)
    ld = x.stride(0) if ld_x is None else ld_x
    o = _Opts(vscale, k_norm, w_idx, idx_cache, measure)
    _check("rf_fill_q8", lib().rf_fill_q8(
        plan.handle, _ptr(x), ld, _ptr(fill_rows_t), n_fill, _ptr(positions), _ptr(slot_of_row),
        _ptr_array(map_q), _ptr_array(map_scale), _ptr_array(map_b), _ptr_array(gamma), _ptr_array(w_k),
        _ptr_array(w_v), _ptr(rope), _ptr_array(k_cache), _ptr_array(v_cache), o.ref, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def value_scales(plan: Plan, x, layer_in: Sequence, calib_rows, calib_group, n_groups: int, map_a: Sequence,
                 map_b: Sequence, gamma: Sequence, w_v: Sequence, scale_out, workspace, stream=None,
                 ld_x: Optional[int] = None, ld_in: Optional[int] = None, map_scale: Sequence = None) -> None:
    """rf_value_scales (bf16 maps) or rf_value_scales_q8 (map_a holds int8 codes
    and map_scale their bf16 block scales): per request, layer and kv head,
    the mean ratio of exact to predicted value norms over the calibration rows."""
    fn = "rf_value_scales" if map_scale is None else "rf_value_scales_q8"
    sh = plan.shape
    mw = "pinned" if plan.maps_on_host else "device"
    _rows_arg(fn, "x", x, sh.n_rows, sh.d_in, ld_x)
    _check_measure(fn, plan, layer_in, ld_in, calib_rows, calib_group, n_groups, scale_out)
    if map_scale is None:
        _layers(fn, "map_a", map_a, sh.n_late, _BF16, sh.d_out * sh.d_in, mw, (sh.d_out, sh.d_in))
    else:
        _layers(fn, "map_q", map_a, sh.n_late, ("int8",), sh.d_out * sh.d_in, mw, (sh.d_out, sh.d_in))
        _layers(fn, "map_scale", map_scale, sh.n_late, _BF16, sh.d_out * (sh.d_in // Q8_BLOCK), mw,
                (sh.d_out, sh.d_in // Q8_BLOCK))
    _layers(fn, "map_b", map_b, sh.n_late, _BF16, sh.d_out, mw)
    _layers(fn, "gamma", gamma, sh.n_late, _BF16, sh.d_out)
    _layers(fn, "w_v", w_v, sh.n_late, _BF16, plan.kv_width * sh.d_out)
    _workspace(fn, workspace)
    ld = x.stride(0) if ld_x is None else ld_x
    ldi = layer_in[0].stride(0) if ld_in is None else ld_in
    n = calib_rows.numel()
    common = (plan.handle, _ptr(x), ld, _ptr_array(layer_in), ldi, _ptr(calib_rows), _ptr(calib_group), n,
              n_groups)
    tail = (_ptr_array(gamma), _ptr_array(w_v), _ptr(scale_out), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    if map_scale is None:
        _check("rf_value_scales", lib().rf_value_scales(*common, _ptr_array(map_a), _ptr_array(map_b), *tail))
    else:
        _check("rf_value_scales_q8", lib().rf_value_scales_q8(*common, _ptr_array(map_a), _ptr_array(map_scale),
                                                              _ptr_array(map_b), *tail))


def map_dequantize_q8(q, scale, w_out, stream=None) -> None:
    """rf_map_dequantize_q8: w_out[o][k] = bf16(q[o][k] * scale[o][k // 128]) on the device."""
    _arg("rf_map_dequantize_q8", "q", q, ("int8",), 0)
    if q.dim() != 2 or not q.is_contiguous():
        raise ValueError("rf_map_dequantize_q8: q must be a contiguous [d_out][d_in] matrix")
    d_out, d_in = q.shape
    _arg("rf_map_dequantize_q8", "scale", scale, _BF16, d_out * (d_in // Q8_BLOCK))
    _arg("rf_map_dequantize_q8", "w_out", w_out, _BF16, d_out * d_in)
    _check("rf_map_dequantize_q8", lib().rf_map_dequantize_q8(_ptr(q), _ptr(scale), d_out, d_in, _ptr(w_out),
                                                              _stream(stream)))


def map_quantize_q8(a: np.ndarray):
    """rf_map_quantize_q8 on the host: (int8 codes [d_out][d_in], bf16 scale bits [d_out][d_in/128])."""
    a = _f32(a)
    d_out, d_in = a.shape
    q = np.empty((d_out, d_in), dtype=np.int8)
    s = np.empty((d_out, max(d_in // Q8_BLOCK, 1)), dtype=np.uint16)
    _check("rf_map_quantize_q8", lib().rf_map_quantize_q8(a.ctypes.data, d_out, d_in, q.ctypes.data, s.ctypes.data))
    return q, s


def kv_project(plan: Plan, layer_in: Sequence, rows, n: int, positions, slot_of_row, gamma: Sequence,
               w_k: Sequence, w_v: Sequence, rope, k_cache: Sequence, v_cache: Sequence, workspace,
               stream=None, ld_in: Optional[int] = None, k_norm: Sequence = None, w_idx: Sequence = None,
               idx_cache: Sequence = None) -> None:
    """rf_kv_project: the exact cache write of every late layer from given inputs."""
    fn, sh = "rf_kv_project", plan.shape
    if not 0 <= n <= sh.n_rows:
        raise ValueError(f"{fn}: n={n} outside [0, n_rows={sh.n_rows}]")
    if layer_in is None or len(layer_in) != sh.n_late:
        raise ValueError(f"{fn}: layer_in must hold one tensor per late layer ({sh.n_late})")
    for i, t in enumerate(layer_in):
        _rows_arg(fn, f"layer_in[{i}]", t, sh.n_rows, sh.d_out, ld_in)
    _arg(fn, "rows", rows, ("int32",), n)
    _arg(fn, "positions", positions, ("int32",), sh.n_rows)
    _arg(fn, "slot_of_row", slot_of_row, ("int32",), sh.n_rows, optional=True)
    _layers(fn, "gamma", gamma, sh.n_late, _BF16, sh.d_out)
    _layers(fn, "w_k", w_k, sh.n_late, _BF16, plan.kv_width * sh.d_out)
    _layers(fn, "w_v", w_v, sh.n_late, _BF16, plan.kv_width * sh.d_out)
    _arg(fn, "rope", rope, ("float32",), sh.max_pos * sh.head_dim, optional=True)
    _layers(fn, "k_cache", k_cache, sh.n_late, _BF16, sh.n_slots * plan.kv_width)
    _layers(fn, "v_cache", v_cache, sh.n_late, _BF16, sh.n_slots * plan.kv_width)
    if k_norm is not None:
        _layers(fn, "k_norm", k_norm, sh.n_late, _BF16, sh.head_dim)
    if w_idx is not None:
        _layers(fn, "w_idx", w_idx, sh.n_late, _BF16, plan.idx_width * sh.d_out)
    if idx_cache is not None:
        _layers(fn, "idx_cache", idx_cache, sh.n_late, _BF16, sh.n_slots * plan.idx_width)
    _workspace(fn, workspace)
    ld = layer_in[0].stride(0) if ld_in is None else ld_in
    o = _Opts(None, k_norm, w_idx, idx_cache)
    _check("rf_kv_project", lib().rf_kv_project(
        plan.handle, _ptr_array(layer_in), ld, _ptr(rows), n, _ptr(positions), _ptr(slot_of_row),
        _ptr_array(gamma), _ptr_array(w_k), _ptr_array(w_v), _ptr(rope), _ptr_array(k_cache),
        _ptr_array(v_cache), o.ref, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def _f32(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


class RidgeAccumulator:
    """rf_ridge_acc: running sums of a ridge fit on the host (float64 inside)."""

    def __init__(self, d_in: int, d_out: int):
        h = C.c_void_p()
        _check("rf_ridge_acc_create", lib().rf_ridge_acc_create(d_in, d_out, C.byref(h)))
        self.handle, self.d_in, self.d_out = h, d_in, d_out

    def add(self, x: np.ndarray, y: np.ndarray) -> None:
        x, y = _f32(x), _f32(y)
        if x.shape[1] != self.d_in or y.shape[1] != self.d_out or x.shape[0] != y.shape[0]:
            raise ValueError("shape mismatch")
        _check("rf_ridge_acc_add", lib().rf_ridge_acc_add(self.handle, x.ctypes.data, y.ctypes.data, x.shape[0]))

    def solve(self, lam: float, raw: bool = False):
        a = np.empty((self.d_out, self.d_in), dtype=np.float32)
        b = np.empty(self.d_out, dtype=np.float32)
        _check("rf_ridge_solve", lib().rf_ridge_solve(self.handle, lam, RF_RIDGE_RAW if raw else 0,
                                                      a.ctypes.data, b.ctypes.data))
        return a, b

    def sums(self):
        """(sxx [d_in][d_in], sxy [d_in][d_out], sx, sy, n) in float64."""
        sxx = np.empty((self.d_in, self.d_in))
        sxy = np.empty((self.d_in, self.d_out))
        sx = np.empty(self.d_in)
        sy = np.empty(self.d_out)
        n = C.c_int64()
        _check("rf_ridge_acc_sums", lib().rf_ridge_acc_sums(self.handle, sxx.ctypes.data, sxy.ctypes.data,
                                                            sx.ctypes.data, sy.ctypes.data, C.byref(n)))
        return sxx, sxy, sx, sy, int(n.value)

    def close(self):
        if self.handle:
            lib().rf_ridge_acc_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class RidgeDeviceSums:
    """rf_ridge_dev: fp64 running sums of a ridge fit formed on the GPU from
    device bf16 activations; merge() moves them into a RidgeAccumulator."""

    def __init__(self, d_in: int, d_out: int):
        h = C.c_void_p()
        _check("rf_ridge_dev_create", lib().rf_ridge_dev_create(d_in, d_out, C.byref(h)))
        self.handle, self.d_in, self.d_out = h, d_in, d_out

    def add(self, x, y, stream=None) -> None:
        """x: device bf16 [n][>= d_in], y: device bf16 [n][>= d_out] (row-major)."""
        if x.dim() != 2 or y.dim() != 2 or x.shape[0] != y.shape[0]:
            raise ValueError("x and y must be 2-D with the same number of rows")
        _rows_arg("rf_ridge_dev_add", "x", x, x.shape[0], self.d_in, None)
        _rows_arg("rf_ridge_dev_add", "y", y, y.shape[0], self.d_out, None)
        _check("rf_ridge_dev_add", lib().rf_ridge_dev_add(self.handle, _ptr(x), x.stride(0), _ptr(y), y.stride(0),
                                                          x.shape[0], _stream(stream)))

    def merge(self, acc: "RidgeAccumulator", stream=None) -> None:
        _check("rf_ridge_dev_merge", lib().rf_ridge_dev_merge(self.handle, acc.handle, _stream(stream)))

    def solve_workspace_bytes(self) -> int:
        return int(lib().rf_ridge_dev_solve_workspace_bytes(self.handle))

    def solve(self, lam: float, raw: bool = False, a=None, b=None, workspace=None, stream=None):
        """rf_ridge_dev_solve: A [d_out][d_in] and b [d_out] (device fp32) from
        the device sums; outputs and workspace are allocated when not given."""
        import torch
        dev = torch.device("cuda", torch.cuda.current_device())
        a = torch.empty((self.d_out, self.d_in), dtype=torch.float32, device=dev) if a is None else a
        b = torch.empty(self.d_out, dtype=torch.float32, device=dev) if b is None else b
        if workspace is None:
            workspace = torch.empty(self.solve_workspace_bytes(), dtype=torch.uint8, device=dev)
        _arg("rf_ridge_dev_solve", "a", a, ("float32",), self.d_out * self.d_in)
        _arg("rf_ridge_dev_solve", "b", b, ("float32",), self.d_out)
        _workspace("rf_ridge_dev_solve", workspace)
        _check("rf_ridge_dev_solve", lib().rf_ridge_dev_solve(
            self.handle, lam, RF_RIDGE_RAW if raw else 0, _ptr(a), _ptr(b), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream)))
        return a, b

    def close(self):
        if self.handle:
            lib().rf_ridge_dev_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def ridge_fit(x: np.ndarray, y: np.ndarray, lam: float, raw: bool = False):
    """rf_ridge_fit: A [d_out][d_in] and b [d_out] (float32) of the ridge map."""
    x, y = _f32(x), _f32(y)
    n, d_in = x.shape
    d_out = y.shape[1]
    a = np.empty((d_out, d_in), dtype=np.float32)
    b = np.empty(d_out, dtype=np.float32)
    _check("rf_ridge_fit", lib().rf_ridge_fit(x.ctypes.data, y.ctypes.data, n, d_in, d_out, lam,
                                              RF_RIDGE_RAW if raw else 0, a.ctypes.data, b.ctypes.data))
    return a, b
