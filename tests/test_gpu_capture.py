"""GPU capture of the ridge sums and the solve from them (rf_ridge_dev_*),
RidgeFill section 2.2 "Fitting".

The device sums are merged into the host accumulator and solved there, and
solved on the GPU (rf_ridge_dev_solve); the results are compared with the
fp64 oracle on the same bf16 values and with the host accumulator fed the
same rows (only the order of the exact products' fp64 additions differs).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from late_layer_kv_amd import binding as B
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _data(seed, n, d_in, d_out):
    g = np.random.default_rng(seed)
    x = g.standard_normal((n, d_in)).astype(np.float32) * g.uniform(0.5, 2.0, d_in).astype(np.float32) \
        + g.standard_normal(d_in).astype(np.float32)
    m = (np.eye(d_in, d_out) + 0.05 * g.standard_normal((d_in, d_out))).astype(np.float32)
    y = x @ m + 0.1 * g.standard_normal((n, d_out)).astype(np.float32) + g.standard_normal(d_out).astype(np.float32)
    return workloads.f32_to_bf16_bits(x), workloads.f32_to_bf16_bits(y)


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("d_in,d_out,chunks", [(256, 384, (1, 31, 32, 33, 700)), (512, 256, (2048,))])
def test_device_sums_match_host_and_oracle(d_in, d_out, chunks):
    _say(f"[capture] d_in={d_in} d_out={d_out} chunks={chunks}")
    n = sum(chunks)
    xb, yb = _data(60 + d_in, n, d_in, d_out)
    dev = B.RidgeDeviceSums(d_in, d_out)
    host = B.RidgeAccumulator(d_in, d_out)
    ref = oracle.RidgeSums(d_in, d_out)
    r0 = 0
    for c in chunks:
        xs, ys = xb[r0:r0 + c], yb[r0:r0 + c]
        dev.add(U.t16(xs).cuda(), U.t16(ys).cuda())
        xf, yf = oracle.bf16_bits_to_f64(xs), oracle.bf16_bits_to_f64(ys)
        host.add(xf.astype(np.float32), yf.astype(np.float32))
        ref.add(xf, yf)
        r0 += c
    merged = B.RidgeAccumulator(d_in, d_out)
    dev.merge(merged)
    got = merged.sums()
    for g_, w_ in zip(got[:4], (ref.sxx, ref.sxy, ref.sx, ref.sy)):
        assert np.allclose(g_, w_, rtol=1e-13, atol=1e-13 * np.max(np.abs(w_)))
    assert got[4] == n
    for lam in (0.03, 1.0):
        a_d, b_d = merged.solve(lam)
        a_h, b_h = host.solve(lam)
        a_r, b_r = ref.solve(lam)
        assert np.allclose(a_d, a_h, rtol=1e-6, atol=1e-7) and np.allclose(b_d, b_h, rtol=1e-6, atol=1e-6)
        assert np.allclose(a_d, a_r, rtol=1e-5, atol=1e-6) and np.allclose(b_d, b_r, rtol=1e-5, atol=1e-5)
    # merging cleared the device sums
    empty = B.RidgeAccumulator(d_in, d_out)
    dev.merge(empty)
    with pytest.raises(B.RfError):
        empty.solve(0.1)


def test_device_sums_exact_on_small_integers():
    """Small integer data: every product and partial sum is an exact fp64
    integer, so the device and host sums agree bit for bit and the solves
    are identical."""
    d_in, d_out, n = 128, 128, 333
    g = np.random.default_rng(61)
    x = g.integers(-8, 9, size=(n, d_in)).astype(np.float32)
    y = (x[:, ::-1] * 2 + g.integers(-3, 4, size=(n, d_out))).astype(np.float32)
    xb, yb = workloads.f32_to_bf16_bits(x), workloads.f32_to_bf16_bits(y)
    dev = B.RidgeDeviceSums(d_in, d_out)
    dev.add(U.t16(xb).cuda(), U.t16(yb).cuda())
    merged = B.RidgeAccumulator(d_in, d_out)
    dev.merge(merged)
    host = B.RidgeAccumulator(d_in, d_out)
    host.add(x, y)
    for g_, h_ in zip(merged.sums(), host.sums()):
        assert np.array_equal(g_, h_)
    for lam in (0.03, 0.5):
        a_d, b_d = merged.solve(lam)
        a_h, b_h = host.solve(lam)
        assert np.array_equal(a_d, a_h) and np.array_equal(b_d, b_h)


def test_capture_at_27b_width():
    """d = 5120 (the 27B's split state and layer input), 4,096 rows in two calls,
    against the host accumulator on a slice of outputs."""
    d = 5120
    n = 4096
    _say("[capture 27b width] generating")
    s = workloads.spec("27b", n_late=1, prompt_lens=(n,), tail=16, seed=62)
    w = workloads.make(s)
    xb = w.x
    yb = workloads.make_layer_truth(s, n, outliers=w.outlier_channels)[0]
    dev = B.RidgeDeviceSums(d, d)
    xd, yd = U.t16(xb).cuda(), U.t16(yb).cuda()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    dev.add(xd[:1500], yd[:1500])
    dev.add(xd[1500:], yd[1500:])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    flop = 2.0 * n * d * (d / 2 + d)   # X^T X upper half + X^T Y
    _say(f"[capture 27b width] {ms:.2f} ms for {n} rows: {flop / ms / 1e9:.1f} TFLOP/s fp64 (algorithmic)")
    merged = B.RidgeAccumulator(d, d)
    dev.merge(merged)
    sxx, sxy, sx, sy, nn = merged.sums()
    ref = oracle.RidgeSums(d, d)
    ref.add(oracle.bf16_bits_to_f64(xb), oracle.bf16_bits_to_f64(yb))
    assert nn == n
    for got, want in ((sxx, ref.sxx), (sxy, ref.sxy), (sx, ref.sx), (sy, ref.sy)):
        scale = np.max(np.abs(want))
        assert np.max(np.abs(got - want)) <= 1e-12 * scale * np.sqrt(n), float(np.max(np.abs(got - want)) / scale)


# ---------------------------------------------------------------- the solve on the GPU

def _fill_sums(d_in, d_out, xb, yb, chunks=None):
    dev = B.RidgeDeviceSums(d_in, d_out)
    ref = oracle.RidgeSums(d_in, d_out)
    r0 = 0
    for c in (chunks or (xb.shape[0],)):
        dev.add(U.t16(xb[r0:r0 + c]).cuda(), U.t16(yb[r0:r0 + c]).cuda())
        ref.add(oracle.bf16_bits_to_f64(xb[r0:r0 + c]), oracle.bf16_bits_to_f64(yb[r0:r0 + c]))
        r0 += c
    return dev, ref


def _close(got, want, rel):
    scale = np.max(np.abs(want))
    err = np.max(np.abs(got - want)) / scale
    assert err <= rel, f"max error {err:.3e} relative to the largest entry"
    return err


@pytest.mark.parametrize("d_in,d_out", [(256, 384), (512, 256), (1024, 1024)])
def test_device_solve_matches_oracle(d_in, d_out):
    """rf_ridge_dev_solve against the fp64 oracle on the same bf16 values
    (outputs are fp32: 1e-6 of the largest entry), for two lambdas and the raw
    form; the sums survive the solve, and a repeated solve is bitwise equal."""
    _say(f"[gpu solve] d_in={d_in} d_out={d_out}")
    n = 3 * d_in + 17
    xb, yb = _data(70 + d_in + d_out, n, d_in, d_out)
    dev, ref = _fill_sums(d_in, d_out, xb, yb, chunks=(n // 3, n - n // 3))
    xf, yf = oracle.bf16_bits_to_f64(xb), oracle.bf16_bits_to_f64(yb)
    for lam in (0.03, 1.0):
        a, b = dev.solve(lam)
        a_r, b_r = ref.solve(lam)
        ea = _close(a.cpu().numpy(), a_r, 1e-6)
        eb = _close(b.cpu().numpy(), b_r, 1e-6)
        _say(f"[gpu solve] lambda={lam}: A {ea:.2e}, b {eb:.2e}")
    a_raw, b_raw = dev.solve(0.5, raw=True)
    a_rr, _ = oracle.ridge_fit_raw(xf, yf, 0.5)
    _close(a_raw.cpu().numpy(), a_rr, 1e-6)
    assert not torch.any(b_raw)
    a1, b1 = dev.solve(0.03)
    a2, b2 = dev.solve(0.03)
    assert torch.equal(a1, a2) and torch.equal(b1, b2)
    # the host solve of the merged sums agrees too
    merged = B.RidgeAccumulator(d_in, d_out)
    dev.merge(merged)
    a_h, b_h = merged.solve(0.03)
    _close(a1.cpu().numpy(), a_h, 2e-6)


def test_device_solve_reports_a_singular_system():
    """Constant rows: the centred X^T X is zero, so with any lambda the
    system is singular (alpha scales with its trace) and the call reports it."""
    d = 128
    xb = workloads.f32_to_bf16_bits(np.ones((50, d), dtype=np.float32))
    yb = workloads.f32_to_bf16_bits(np.random.default_rng(5).standard_normal((50, d)).astype(np.float32))
    dev, _ = _fill_sums(d, d, xb, yb)
    with pytest.raises(B.RfError) as e:
        dev.solve(0.1)
    assert e.value.status == -6
    assert "positive definite" in B.last_error()
    # raw with lambda > 0 is regular: X^T X + lambda I
    a, b = dev.solve(0.1, raw=True)
    assert torch.isfinite(a).all()


def test_device_solve_at_27b_width():
    """d = 5120 from 4,096 captured rows (fewer rows than width: only the
    penalty makes the system regular), against the fp64 oracle."""
    d, n = 5120, 4096
    _say("[gpu solve 27b width] generating")
    s = workloads.spec("27b", n_late=1, prompt_lens=(n,), tail=16, seed=63)
    w = workloads.make(s)
    xb = w.x
    yb = workloads.make_layer_truth(s, n, outliers=w.outlier_channels)[0]
    dev = B.RidgeDeviceSums(d, d)
    dev.add(U.t16(xb).cuda(), U.t16(yb).cuda())
    ws = torch.empty(dev.solve_workspace_bytes(), dtype=torch.uint8, device="cuda:0")
    dev.solve(0.03, workspace=ws)
    import time
    t0 = time.perf_counter()
    a, b = dev.solve(0.03, workspace=ws)
    ms = (time.perf_counter() - t0) * 1e3
    _say(f"[gpu solve 27b width] {ms:.1f} ms per solve (including its sync)")
    ref = oracle.RidgeSums(d, d)
    ref.add(oracle.bf16_bits_to_f64(xb), oracle.bf16_bits_to_f64(yb))
    a_r, b_r = ref.solve(0.03)
    ea = _close(a.cpu().numpy(), a_r, 1e-5)
    eb = _close(b.cpu().numpy(), b_r, 1e-5)
    _say(f"[gpu solve 27b width] A {ea:.2e}, b {eb:.2e}")
