"""C-ABI library checks that need no GPU: symbols, host-side errors, host ridge."""
import ctypes as C
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import oracle
from late_layer_kv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rf.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set(re.findall(r"\b(rf_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_header_and_binding_agree():
    assert sorted(B.EXPORTS) == _declared_functions()


def test_library_exports_every_declared_symbol():
    L = B.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


def _shape(**kw):
    base = dict(d_in=256, d_out=256, n_late=4, n_kv=2, head_dim=64, rms_eps=1e-5, rope_theta=1e4,
                n_rows=512, n_slots=512, max_pos=512, n_idx=0)
    base.update(kw)
    return base


@pytest.mark.parametrize("bad,status", [
    (dict(d_in=100), -2), (dict(d_out=320), -2), (dict(n_late=0), -2), (dict(head_dim=96), -2),
    (dict(n_kv=1), -2), (dict(rope_theta=1.0), -2), (dict(max_pos=0), -2), (dict(rms_eps=-1.0), -2),
    (dict(n_idx=-1), -2), (dict(n_idx=9), -2),
])
def test_plan_rejects_bad_shapes(bad, status):
    with pytest.raises(B.RfError) as e:
        B.Plan(**_shape(**bad))
    assert e.value.status == status
    assert B.last_error()


def test_plan_rejects_unknown_flags():
    L = B.lib()
    sh = B.Shape(*_shape().values())
    h = C.c_void_p()
    assert L.rf_plan_create(C.byref(sh), 8, C.byref(h)) == -1
    assert L.rf_plan_create(None, 0, C.byref(h)) == -1


def test_fill_argument_errors_before_any_device_work():
    """Every check here fails on the host, before a HIP call, so it runs without a GPU."""
    p = B.Plan(**_shape())
    L = B.lib()
    nl = 4
    fake = C.c_void_p(0x1000)  # never dereferenced: the call must fail first
    arr = (C.c_void_p * nl)(*([0x1000] * nl))
    null_arr = (C.c_void_p * nl)(*([0x1000] * (nl - 1) + [0]))
    ws = 1 << 40

    def call(x=fake, ld=256, rows=fake, n=10, pos=fake, maps=arr, gam=arr, ws_ptr=C.c_void_p(0x10000), ws_b=ws,
             vs=None):
        return L.rf_fill(p.handle, x, ld, rows, n, pos, None, maps, arr, gam, arr, arr, None, arr, arr,
                         vs, ws_ptr, ws_b, None)
    assert call(n=-1) == -1
    assert call(n=513) == -1
    assert call(x=None) == -1
    assert call(x=C.c_void_p(0x1008)) == -1       # misaligned
    assert call(ld=100) == -1
    assert call(ld=260) == -1                      # ld not a multiple of 8
    assert call(rows=None) == -1
    assert call(pos=None) == -1
    assert call(maps=null_arr) == -1
    assert call(gam=None) == -1
    assert call(ws_ptr=C.c_void_p(0x10010)) == -4  # workspace misaligned
    assert call(ws_b=16) == -4
    assert "workspace" in B.last_error()
    def opts(vs=None, kn=None):
        o = B.FillOpts()
        if vs is not None:
            o.vscale = C.pointer(vs)
        if kn is not None:
            o.k_norm = C.cast(kn, C.POINTER(C.c_void_p))
        return C.byref(o)
    assert call(vs=opts(B.VScale(None, 0x1000, 1))) == -1   # null scale
    assert call(vs=opts(B.VScale(0x1000, None, 1))) == -1   # null groups
    assert call(vs=opts(B.VScale(0x1000, 0x1000, 0))) == -1  # no groups
    assert call(vs=opts(B.VScale(0x1002, 0x1000, 1))) == -1  # misaligned scale
    assert call(vs=opts(kn=null_arr)) == -1                  # a layer without a key-norm gain
    assert call(vs=opts(kn=(C.c_void_p * nl)(*([0x1000] * (nl - 1) + [0x1008])))) == -1  # misaligned gain
    # exact rows take no value rescale
    ws_ptr = C.c_void_p(0x10000)
    assert L.rf_kv_project(p.handle, arr, 256, fake, 10, fake, None, arr, arr, arr, None, arr, arr,
                           opts(B.VScale(0x1000, 0x1000, 1)), ws_ptr, ws, None) == -1
    p.close()


def test_workspace_sizes():
    p = B.Plan(**_shape())
    assert p.fill_workspace_bytes(448, 1) > 0
    assert p.fill_workspace_bytes(448, 4) > p.fill_workspace_bytes(448, 1)
    assert p.fill_workspace_bytes(448, 5) == 0   # more layers than the plan has
    assert p.fill_workspace_bytes(-1, 1) == 0
    # rope table + flag + prepared weights + Y + per-tile row sums of squares
    # + per-row norm factors, each rounded to 256 bytes
    rope = 512 * 32 * 8
    prep = 2 * 128 * 256 * 2
    y = 448 * 256 * 2
    ssq = 448 * (256 // 256) * 4
    rs = 448 * 4
    assert p.fill_workspace_bytes(448, 1) == rope + 256 + prep + y + ssq + rs
    assert p.fill_workspace_bytes(448, 2) == rope + 256 + 2 * (prep + y + ssq + rs)
    assert p.kv_project_workspace_bytes(2) == rope + 256 + 2 * prep + 2 * 512 * 4  # + norm factor per plan row
    # row mask padded to whole 4,096-row blocks, then two 256-byte-rounded
    # arrays of per-block counts and offsets
    assert B.fill_rows_workspace_bytes(1000) == 4096 + 2 * 256
    assert B.fill_rows_workspace_bytes(122880) == 122880 + 2 * 256
    assert B.fill_rows_workspace_bytes(0) == 4096 + 2 * 256
    assert B.fill_rows_workspace_bytes(-1) == 0
    p.close()


def test_stream_group_constant_matches_header():
    hdr = open(os.path.join(ROOT, "include", "rf.h")).read()
    m = re.search(r"#define RF_STREAM_GROUP (\d+)", hdr)
    assert m and int(m.group(1)) == B.RF_STREAM_GROUP


# ---- host ridge (float64 inside the library) against the fp64 oracle


def _data(seed, n, d_in, d_out, noise=0.3):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((n, d_in)) * g.uniform(0.5, 2.0, d_in) + g.standard_normal(d_in)).astype(np.float32)
    m = g.standard_normal((d_out, d_in))
    y = (x @ m.T + g.standard_normal(d_out) + noise * g.standard_normal((n, d_out))).astype(np.float32)
    return x, y


@pytest.mark.parametrize("lam", [0.03, 1e-3, 1.0])
def test_ridge_fit_matches_oracle(lam):
    x, y = _data(1, 400, 24, 16)
    a, b = B.ridge_fit(x, y, lam)
    ar, br = oracle.ridge_fit(x.astype(np.float64), y.astype(np.float64), lam)
    assert np.allclose(a, ar, rtol=1e-5, atol=1e-6)
    assert np.allclose(b, br, rtol=1e-5, atol=1e-5)


def test_ridge_raw_matches_oracle():
    x, y = _data(2, 300, 20, 8)
    a, b = B.ridge_fit(x, y, 2.5, raw=True)
    ar, br = oracle.ridge_fit_raw(x.astype(np.float64), y.astype(np.float64), 2.5)
    assert np.allclose(a, ar, rtol=1e-5, atol=1e-6)
    assert np.array_equal(b, np.zeros_like(b))


def test_ridge_running_sums_and_new_lambda():
    x, y = _data(3, 500, 16, 12)
    acc = B.RidgeAccumulator(16, 12)
    for a0, a1 in ((0, 1), (1, 200), (200, 500)):
        acc.add(x[a0:a1], y[a0:a1])
    for lam in (0.03, 0.3):
        a1, b1 = acc.solve(lam)
        a2, b2 = B.ridge_fit(x, y, lam)
        assert np.allclose(a1, a2, rtol=1e-6, atol=1e-7)
        assert np.allclose(b1, b2, rtol=1e-6, atol=1e-6)
    acc.close()


def test_ridge_recovers_map_as_lambda_vanishes():
    x, y = _data(4, 300, 12, 6, noise=0.0)
    ar, br = oracle.ridge_fit(x.astype(np.float64), y.astype(np.float64), 1e-12)
    a, b = B.ridge_fit(x, y, 1e-12)
    assert np.allclose(a, ar, rtol=1e-4, atol=1e-5)


def test_ridge_errors():
    with pytest.raises(B.RfError) as e:
        B.RidgeAccumulator(0, 3)
    assert e.value.status == -1
    acc = B.RidgeAccumulator(4, 2)
    with pytest.raises(B.RfError):
        acc.solve(0.1)   # nothing accumulated
    acc.add(np.zeros((3, 4), np.float32), np.zeros((3, 2), np.float32))
    with pytest.raises(B.RfError) as e:
        acc.solve(0.0)   # singular without a penalty
    assert e.value.status == -6
    with pytest.raises(B.RfError):
        acc.solve(-1.0)


# ---- int8 maps: host checks and the host quantizer


def test_q8_plan_needs_d_in_multiple_of_128():
    with pytest.raises(B.RfError) as e:
        B.Plan(**_shape(d_in=192), maps_q8=True)
    assert e.value.status == -2
    B.Plan(**_shape(d_in=192)).close()   # fine for bf16 maps


def test_q8_flag_must_match_the_call():
    L = B.lib()
    nl = 4
    fake = C.c_void_p(0x1000)
    arr = (C.c_void_p * nl)(*([0x1000] * nl))
    ws, ws_b = C.c_void_p(0x10000), 1 << 40
    p8 = B.Plan(**_shape(), maps_q8=True)
    pb = B.Plan(**_shape())
    # bf16 entry point on an int8 plan, and the reverse
    assert L.rf_fill(p8.handle, fake, 256, fake, 10, fake, None, arr, arr, arr, arr, arr, None, arr, arr,
                     None, ws, ws_b, None) == -1
    assert "RF_MAPS_Q8" in B.last_error()
    assert L.rf_fill_q8(pb.handle, fake, 256, fake, 10, fake, None, arr, arr, arr, arr, arr, arr, None, arr,
                        arr, None, ws, ws_b, None) == -1
    null_arr = (C.c_void_p * nl)(*([0x1000] * (nl - 1) + [0]))
    mis_arr = (C.c_void_p * nl)(*([0x1000] * (nl - 1) + [0x1004]))

    def call8(q=arr, s=arr, b=arr, ws_b=ws_b):
        return L.rf_fill_q8(p8.handle, fake, 256, fake, 10, fake, None, q, s, b, arr, arr, arr, None, arr, arr,
                            None, ws, ws_b, None)
    assert call8(q=None) == -1
    assert call8(s=None) == -1
    assert call8(q=null_arr) == -1
    assert call8(s=null_arr) == -1
    assert call8(q=mis_arr) == -1        # codes must be 16-byte aligned
    assert call8(b=null_arr) == -1
    assert call8(ws_b=16) == -4
    p8.close()
    pb.close()


def test_q8_workspace_adds_the_bf16_image():
    p8 = B.Plan(**_shape(), maps_q8=True)
    pb = B.Plan(**_shape())
    image = 256 * 256 * 2
    for g in (1, 2, 4):
        assert p8.fill_workspace_bytes(448, g) == pb.fill_workspace_bytes(448, g) + g * image
    assert p8.kv_project_workspace_bytes(2) == pb.kv_project_workspace_bytes(2)
    for p in (p8, pb):
        p.close()


def test_dequantize_argument_errors_before_any_device_work():
    L = B.lib()
    f = C.c_void_p(0x1000)
    assert L.rf_map_dequantize_q8(None, f, 4, 128, f, None) == -1
    assert L.rf_map_dequantize_q8(f, None, 4, 128, f, None) == -1
    assert L.rf_map_dequantize_q8(f, f, 4, 128, None, None) == -1
    assert L.rf_map_dequantize_q8(C.c_void_p(0x1001), f, 4, 128, f, None) == -1
    assert L.rf_map_dequantize_q8(f, f, 4, 128, C.c_void_p(0x1002), None) == -1
    assert L.rf_map_dequantize_q8(f, f, 4, 100, f, None) == -2
    assert L.rf_map_dequantize_q8(f, f, 0, 128, f, None) == -2


def _quant_inputs():
    import workloads
    w = workloads.make(workloads.spec("tiny"), layers=[0])
    g = np.random.default_rng(21)
    a_map = oracle.bf16_bits_to_f64(w.map_a[0]).astype(np.float32)          # an I + noise map
    heavy = (g.standard_t(2, size=(64, 384)) * np.exp(g.uniform(-30, 30, size=(64, 1)))).astype(np.float32)
    heavy[3, 128:256] = 0.0                                                   # all-zero block
    heavy[5, :128] = 0.0
    heavy[5, :4] = [63.5, 1.25, 1.75, -0.75]                                  # exact ties at scale 0.5
    tiny = (g.standard_normal((8, 128)) * 1e-38).astype(np.float32)           # subnormal range
    return [a_map, heavy, tiny]


@pytest.mark.parametrize("case", range(3))
def test_host_quantizer_matches_oracle_bitwise(case):
    a = _quant_inputs()[case]
    q, s = B.map_quantize_q8(a)
    qr, sr = oracle.quantize_q8(a)
    assert np.array_equal(s, sr) and np.array_equal(q, qr)


def test_host_quantizer_errors():
    with pytest.raises(B.RfError) as e:
        B.map_quantize_q8(np.ones((2, 100), np.float32))
    assert e.value.status == -2
    a = np.ones((2, 128), np.float32)
    a[1, 7] = np.nan
    with pytest.raises(B.RfError) as e:
        B.map_quantize_q8(a)
    assert e.value.status == -1


# ---- value rescale: host checks


def test_value_scales_argument_errors_and_workspace():
    p = B.Plan(**_shape())
    L = B.lib()
    nl = 4
    f = C.c_void_p(0x1000)
    arr = (C.c_void_p * nl)(*([0x1000] * nl))
    ws, ws_b = C.c_void_p(0x10000), 1 << 40

    def call(n=16, groups=2, x=f, ld_in=256, rows=f, grp=f, scale=f, lay=arr, ws_b=ws_b):
        return L.rf_value_scales(p.handle, x, 256, lay, ld_in, rows, grp, n, groups, arr, arr, arr, arr, scale,
                                 ws, ws_b, None)
    assert call(n=-1) == -1
    assert call(n=513) == -1
    assert call(groups=0) == -1
    assert call(x=None) == -1
    assert call(ld_in=100) == -1
    assert call(rows=None) == -1
    assert call(grp=None) == -1
    assert call(scale=None) == -1
    assert call(scale=C.c_void_p(0x1002)) == -1
    assert call(lay=None) == -1
    assert call(ws_b=16) == -4
    # int8 entry point on a bf16 plan
    assert L.rf_value_scales_q8(p.handle, f, 256, arr, 256, f, f, 16, 2, arr, arr, arr, arr, arr, f, ws, ws_b,
                                None) == -1
    # workspace: flag + prepared weights + Y + two value buffers + ratios + zero positions
    # + per-tile row sums of squares + per-row norm factors
    n, w, d = 40, 128, 256
    up = lambda v: (v + 255) // 256 * 256
    want = (256 + 2 * w * d * 2 + up(n * d * 2) + 2 * up(n * w * 2) + up(4 * n * 2 * 4) + up(n * 4)
            + up(n * (d // 256) * 4) + up(n * 4))
    assert p.value_scales_workspace_bytes(n, 1) == want
    assert p.value_scales_workspace_bytes(n, 5) == 0
    p.close()


def test_ridge_device_sums_argument_errors():
    L = B.lib()
    h = C.c_void_p()
    assert L.rf_ridge_dev_create(100, 128, C.byref(h)) == -2
    assert L.rf_ridge_dev_create(128, 0, C.byref(h)) == -2
    assert L.rf_ridge_dev_create(128, 128, None) == -1
    assert L.rf_ridge_dev_add(None, None, 128, None, 128, 4, None) == -1
    assert L.rf_ridge_dev_merge(None, None, None) == -1


def test_ridge_acc_sums_round_trip():
    x, y = _data(5, 50, 6, 4)
    acc = B.RidgeAccumulator(6, 4)
    acc.add(x, y)
    sxx, sxy, sx, sy, n = acc.sums()
    ref = oracle.RidgeSums(6, 4)
    ref.add(x.astype(np.float64), y.astype(np.float64))
    assert n == 50
    for a, b in ((sxx, ref.sxx), (sxy, ref.sxy), (sx, ref.sx), (sy, ref.sy)):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-9)
    assert np.array_equal(sxx, sxx.T)


def test_indexer_key_options():
    """Indexer keys are required exactly when the plan has indexer heads; the
    prepared weights grow by the indexer rows, padded to a 256-row tile."""
    L = B.lib()
    nl = 4
    fake = C.c_void_p(0x1000)
    arr = (C.c_void_p * nl)(*([0x1000] * nl))
    null_arr = (C.c_void_p * nl)(*([0x1000] * (nl - 1) + [0]))
    ws = 1 << 40

    def opts(wi=None, ic=None):
        o = B.FillOpts()
        if wi is not None:
            o.w_idx = C.cast(wi, C.POINTER(C.c_void_p))
        if ic is not None:
            o.idx_cache = C.cast(ic, C.POINTER(C.c_void_p))
        return o

    def fill(p, o):
        return L.rf_fill(p.handle, fake, 256, fake, 10, fake, None, arr, arr, arr, arr, arr, None, arr, arr,
                         None if o is None else C.byref(o), C.c_void_p(0x10000), ws, None)

    def project(p, o):
        return L.rf_kv_project(p.handle, arr, 256, fake, 10, fake, None, arr, arr, arr, None, arr, arr,
                               None if o is None else C.byref(o), C.c_void_p(0x10000), ws, None)
    p0 = B.Plan(**_shape())
    assert fill(p0, opts(wi=arr, ic=arr)) == -1        # the plan has no indexer heads
    assert "n_idx" in B.last_error()
    assert project(p0, opts(ic=arr)) == -1
    p1 = B.Plan(**_shape(n_idx=1))
    for call in (fill, project):
        assert call(p1, None) == -1                    # indexer keys required
        assert call(p1, opts(wi=arr)) == -1
        assert call(p1, opts(ic=arr)) == -1
        assert call(p1, opts(wi=null_arr, ic=arr)) == -1
        assert call(p1, opts(wi=arr, ic=null_arr)) == -1
    # prepared rows per layer: 2w + n_idx*hd = 256 + 64, padded to 512
    up = lambda v: (v + 255) // 256 * 256
    rope, d = 512 * 32 * 8, 256
    assert p1.kv_project_workspace_bytes(1) == rope + 256 + 512 * d * 2 + 512 * 4
    assert p0.kv_project_workspace_bytes(1) == rope + 256 + 256 * d * 2 + 512 * 4
    assert (p1.fill_workspace_bytes(448, 2) - p0.fill_workspace_bytes(448, 2)) == 2 * 256 * d * 2
    p0.close()
    p1.close()


def test_in_fill_measurement_argument_errors():
    """rf_fill_opts.measure: checked on the host before any device work."""
    L = B.lib()
    p = B.Plan(**_shape())
    nl = 4
    fake = C.c_void_p(0x1000)
    arr = (C.c_void_p * nl)(*([0x1000] * nl))
    ws = 1 << 40
    need = p.value_scales_workspace_bytes(16, 1)

    def call(vs=None, **kw):
        m = dict(layer_in=C.cast(arr, C.POINTER(C.c_void_p)), ld_in=256, calib_rows=0x1000, calib_group=0x1000,
                 n_calib=16, group_of_row=0x1000, n_groups=2, scale=0x1000, workspace=0x10000, ws_bytes=need)
        m.update(kw)
        vm = B.VMeasure(**m)
        o = B.FillOpts()
        o.measure = C.pointer(vm)
        if vs is not None:
            o.vscale = C.pointer(vs)
        return L.rf_fill(p.handle, fake, 256, fake, 10, fake, None, arr, arr, arr, arr, arr, None, arr, arr,
                         C.byref(o), C.c_void_p(0x10000), ws, None)
    assert call(vs=B.VScale(0x1000, 0x1000, 1)) == -1       # vscale and measure together
    assert call(n_calib=-1) == -1
    assert call(n_groups=0) == -1
    assert call(ld_in=100) == -1
    assert call(calib_rows=None) == -1
    assert call(layer_in=None) == -1
    assert call(scale=None) == -1                            # nowhere to put the scales
    assert call(group_of_row=None) == -1
    assert call(ws_bytes=need - 1) == -4
    assert call(workspace=0x10010) == -4
    p.close()


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and says why,
    before touching the GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_binding_fails_loudly_without_the_library():
    """With librf.so absent the binding raises on first use; nothing falls
    back to another implementation (run in a child so the loaded library of
    this session is untouched)."""
    code = (
        "import sys\n"
        "from late_layer_kv_amd import binding as B\n"
        "B.LIB_PATH = B.LIB_PATH + '.absent'\n"
        "try:\n"
        "    B.Plan(256, 256, 1, 1, 128, 1e-6, 1e4, 256, 256, 256)\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "    sys.exit(0)\n"
        "sys.exit(1)\n"
    )
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "is not built" in r.stdout


def test_traffic_summary_scales_counters_by_the_copy(tmp_path):
    """bench.py's traffic figure: per-launch FETCH_SIZE and WRITE_SIZE (KiB) of
    the map kernel, each scaled by bytes / counter of a device copy of known size."""
    import bench

    def write(path, counter, rows):
        with open(path, "w") as f:
            f.write("Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n")
            for name, grid, v in rows:
                f.write(f'"{name}",{grid},{counter},{v}\n')   # names hold commas; rocprofv3 quotes them

    calib = 4 << 30
    fetch, write_ = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # two map launches, one K/V launch and the calibration copy (which reads half what it moves)
    kv = "void rf::kv_gemm_kernel<128, false, false>(rf::KvParams)"
    torch_fill = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<short>>(int, ...)"
    write(fetch, "FETCH_SIZE", [("rf::map_gemm_kernel(rf::MapParams)", 256, 1000.0),
                                ("rf::map_gemm_kernel(rf::MapParams)", 256, 3000.0),
                                (kv, 256, 500.0), (kv, 256, 500.0),
                                ("rf::rope_table_kernel(float2*, int, int, double)", 64, 90.0),
                                (torch_fill, 4096, 77.0),
                                ("__amd_rocclr_copyBuffer", 1 << 20, calib / 1024 / 2)])
    write(write_, "WRITE_SIZE", [("rf::map_gemm_kernel(rf::MapParams)", 256, 400.0),
                                 ("rf::map_gemm_kernel(rf::MapParams)", 256, 400.0),
                                 (kv, 256, 100.0), (kv, 256, 100.0),
                                 ("rf::rope_table_kernel(float2*, int, int, double)", 64, 900.0),
                                 (torch_fill, 4096, 7777.0),
                                 ("__amd_rocclr_copyBuffer", 1 << 20, calib / 1024)])
    t = bench.summarize_pmc(str(fetch), str(write_), "27b_120k", calib, steps=2)
    assert t["copy_calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert t["copy_calibration"]["write_factor"] == pytest.approx(1.0)
    m = t["kernels"]["map_gemm"]
    assert m["fetch_kib_per_launch"] == pytest.approx(2000.0) and m["write_kib_per_launch"] == pytest.approx(400.0)
    assert t["traffic_bytes_per_launch"] == pytest.approx((2000.0 * 2 + 400.0) * 1024)
    assert t["kernels"]["kv_gemm"]["bytes_per_launch"] == pytest.approx((500.0 * 2 + 100.0) * 1024)
    # per step: the library kernels launched every step, over the two profiled
    # steps; the copy, the once-per-plan RoPE table and torch's kernels left out
    per_step = ((1000.0 + 3000.0) * 2 + 800.0 + (500.0 * 2 + 100.0) * 2) * 1024 / 2
    assert t["bytes_per_step"] == pytest.approx(per_step)
    assert set(t["kernels"]) == {"map_gemm", "kv_gemm", "rope_table", "vectorized_elementwise"}
    assert t["counted_per_step"] == ["kv_gemm", "map_gemm"]
    assert t["kernel_source_sha256"] == bench.kernel_source_hash()


# ---- the binding's own checks of tensor arguments (sizes, types, memory) -----

class _CpuAsDevice:
    """Run the binding's checks with CPU tensors standing in for device ones."""

    def __enter__(self):
        self.old, B.DEVICE_TYPE = B.DEVICE_TYPE, "cpu"

    def __exit__(self, *a):
        B.DEVICE_TYPE = self.old


def _fill_args(d_in=320, d_out=256, n_late=2, n_kv=2, hd=64, n_rows=300, n_fill=200):
    import torch
    i16, i32 = torch.int16, torch.int32
    plan = B.Plan(**_shape(d_in=d_in, d_out=d_out, n_late=n_late, n_kv=n_kv, head_dim=hd, n_rows=n_rows,
                           n_slots=n_rows, max_pos=n_rows))
    w = n_kv * hd
    args = dict(
        x=torch.zeros((n_rows, d_in), dtype=i16), fill_rows_t=torch.zeros(n_fill, dtype=i32), n_fill=n_fill,
        positions=torch.zeros(n_rows, dtype=i32), slot_of_row=None,
        map_a=[torch.zeros((d_out, d_in), dtype=i16) for _ in range(n_late)],
        map_b=[torch.zeros(d_out, dtype=i16) for _ in range(n_late)],
        gamma=[torch.zeros(d_out, dtype=i16) for _ in range(n_late)],
        w_k=[torch.zeros((w, d_out), dtype=i16) for _ in range(n_late)],
        w_v=[torch.zeros((w, d_out), dtype=i16) for _ in range(n_late)], rope=None,
        k_cache=[torch.zeros((n_rows, w), dtype=i16) for _ in range(n_late)],
        v_cache=[torch.zeros((n_rows, w), dtype=i16) for _ in range(n_late)],
        workspace=torch.zeros(256, dtype=torch.uint8),   # too small: the library refuses it
        stream=0)
    return plan, args


def _bad_fill_cases():
    import torch
    i16, i32 = torch.int16, torch.int32
    return {
        "x_too_few_rows": lambda a: a.update(x=a["x"][:299]),
        "x_float32": lambda a: a.update(x=a["x"].float()),
        "x_strided_columns": lambda a: a.update(x=torch.zeros((300, 640), dtype=i16)[:, ::2]),
        "x_narrow_rows": lambda a: a.update(x=torch.zeros((300, 256), dtype=i16)),
        "fill_rows_short": lambda a: a.update(fill_rows_t=a["fill_rows_t"][:199]),
        "fill_rows_int64": lambda a: a.update(fill_rows_t=a["fill_rows_t"].long()),
        "n_fill_above_rows": lambda a: a.update(n_fill=301),
        "positions_short": lambda a: a.update(positions=a["positions"][:299]),
        "positions_int16": lambda a: a.update(positions=a["positions"].short()),
        "slots_short": lambda a: a.update(slot_of_row=torch.zeros(299, dtype=i32)),
        "map_transposed": lambda a: a.update(map_a=[m.t().contiguous() for m in a["map_a"]]),
        "map_transposed_view": lambda a: a.update(map_a=[torch.zeros((320, 256), dtype=i16).t()] * 2),
        "map_short": lambda a: a.update(map_a=[m.flatten()[:-1] for m in a["map_a"]]),
        "map_one_layer_missing": lambda a: a.update(map_a=a["map_a"][:1]),
        "bias_short": lambda a: a.update(map_b=[b[:255] for b in a["map_b"]]),
        "gamma_short": lambda a: a.update(gamma=[g[:255] for g in a["gamma"]]),
        "w_k_short": lambda a: a.update(w_k=[w[:127] for w in a["w_k"]]),
        "w_v_float": lambda a: a.update(w_v=[w.float() for w in a["w_v"]]),
        "rope_short": lambda a: a.update(rope=torch.zeros(300 * 64 - 1, dtype=torch.float32)),
        "k_cache_short": lambda a: a.update(k_cache=[c[:299] for c in a["k_cache"]]),
        "v_cache_short": lambda a: a.update(v_cache=[c[:299] for c in a["v_cache"]]),
        "workspace_not_tensor": lambda a: a.update(workspace=1234),
    }


@pytest.mark.parametrize("case", sorted(_bad_fill_cases()))
def test_binding_rejects_bad_fill_tensors_before_any_call(case):
    plan, args = _fill_args()
    _bad_fill_cases()[case](args)
    with _CpuAsDevice():
        with pytest.raises(ValueError):
            B.fill(plan, **args)


def test_binding_passes_good_fill_tensors_to_the_library():
    plan, args = _fill_args()
    with _CpuAsDevice():
        with pytest.raises(B.RfError) as e:   # the binding's checks pass; librf refuses the workspace
            B.fill(plan, **args)
    assert e.value.status == -4


def test_binding_wants_pinned_host_maps_for_a_streaming_plan():
    import torch
    plan, args = _fill_args()
    plan.maps_on_host = True   # (a streaming plan itself needs a GPU for its map buffers)
    with _CpuAsDevice():
        with pytest.raises(ValueError, match="pinned"):
            B.fill(plan, **args)


def test_binding_rejects_device_data_on_the_host():
    plan, args = _fill_args()
    with pytest.raises(ValueError, match="device memory"):   # CPU tensors where device ones are needed
        B.fill(plan, **args)


def test_binding_rejects_bad_kv_project_and_fill_rows_tensors():
    import torch
    plan, args = _fill_args()
    with _CpuAsDevice():
        lay = [torch.zeros((300, 256), dtype=torch.int16)] * 2
        common = dict(positions=args["positions"], slot_of_row=None, gamma=args["gamma"], w_k=args["w_k"],
                      w_v=args["w_v"], rope=None, k_cache=args["k_cache"], v_cache=args["v_cache"],
                      workspace=args["workspace"], stream=0)
        with pytest.raises(ValueError, match="layer_in"):
            B.kv_project(plan, [t[:299] for t in lay], torch.zeros(10, dtype=torch.int32), 10, **common)
        with pytest.raises(ValueError, match="rows"):
            B.kv_project(plan, lay, torch.zeros(9, dtype=torch.int32), 10, **common)
        with pytest.raises(B.RfError):
            B.kv_project(plan, lay, torch.zeros(10, dtype=torch.int32), 10, **common)
        ws = torch.zeros(4096, dtype=torch.uint8)
        with pytest.raises(ValueError, match="fill_rows_out"):
            B.fill_rows(plan, torch.zeros(5, dtype=torch.int32), torch.zeros(299, dtype=torch.int32),
                        torch.zeros(1, dtype=torch.int32), ws, stream=0)
        with pytest.raises(ValueError, match="exact_rows"):
            B.fill_rows(plan, torch.zeros(5, dtype=torch.int64), torch.zeros(300, dtype=torch.int32),
                        torch.zeros(1, dtype=torch.int32), ws, stream=0)


def test_ridge_fit_output_is_the_map_the_fill_takes():
    """rf_ridge_fit returns A_l [d_out][d_in], the paper's orientation
    (RidgeFill section 2.2, y = A x + b): rounded to bf16 it passes the fill's
    map contract as it is, while W_l = A_l^T (the row-vector form Y = X W + b)
    is refused; on a known map the fit recovers A, not its transpose."""
    import torch
    d_in, d_out = 320, 256
    g = np.random.default_rng(5)
    a_true = g.standard_normal((d_out, d_in)) / np.sqrt(d_in)
    x = g.standard_normal((1000, d_in))
    y = x @ a_true.T
    a, b = B.ridge_fit(x, y, 1e-9)
    assert a.shape == (d_out, d_in)
    assert np.max(np.abs(a - a_true)) < 1e-3
    plan, args = _fill_args(d_in=d_in, d_out=d_out)
    bf = lambda m: torch.from_numpy(oracle.f64_to_bf16_bits(m.astype(np.float64)).view(np.int16).copy())
    args["map_a"] = [bf(a)] * 2
    with _CpuAsDevice():
        with pytest.raises(B.RfError):    # reaches the library (too small a workspace)
            B.fill(plan, **args)
        args["map_a"] = [bf(a.T)] * 2
        with pytest.raises(ValueError, match=r"\[d_out\]\[d_in\]"):
            B.fill(plan, **args)


def test_fill_rows_noalloc_limit_and_header_constant():
    """rf_fill_rows_noalloc refuses a plan over RF_NOALLOC_MAX_ROWS rows on the
    host, before anything is enqueued (no GPU needed to see it)."""
    hdr = open(os.path.join(ROOT, "include", "rf.h")).read()
    m = re.search(r"#define RF_NOALLOC_MAX_ROWS \(1 << (\d+)\)", hdr)
    assert m and (1 << int(m.group(1))) == B.RF_NOALLOC_MAX_ROWS
    L = B.lib()
    n = B.RF_NOALLOC_MAX_ROWS + 1
    p = B.Plan(**_shape(n_rows=n, n_slots=n, max_pos=n))
    st = L.rf_fill_rows_noalloc(p.handle, None, 0, C.c_void_p(0x10000), C.c_void_p(0x20000), None)
    assert st == -2 and "at most" in B.last_error()
    assert L.rf_fill_rows_noalloc(None, None, 0, C.c_void_p(0x10000), C.c_void_p(0x20000), None) == -1
    q = B.Plan(**_shape())
    assert L.rf_fill_rows_noalloc(q.handle, None, -1, C.c_void_p(0x10000), C.c_void_p(0x20000), None) == -1
    assert L.rf_fill_rows_noalloc(q.handle, None, 0, None, C.c_void_p(0x20000), None) == -1


def test_binding_takes_an_empty_exact_row_set():
    """No exact rows at all (a zero tail): an empty tensor passes the
    binding's checks whatever its stride, and reaches the library."""
    import torch
    plan, args = _fill_args()
    empty = torch.from_numpy(np.zeros(0, dtype=np.int32))
    with _CpuAsDevice():
        with pytest.raises(B.RfError) as e:   # the binding passes it on; librf refuses the workspace
            B.fill_rows(plan, empty, torch.zeros(300, dtype=torch.int32), torch.zeros(1, dtype=torch.int32),
                        torch.zeros(16, dtype=torch.uint8), stream=0)
    assert e.value.status == -4
