"""Pins for the fp64 oracle: facts fixed by the pages or by mathematics.

Each pin takes a module ``o`` that exposes the oracle's functions, so the same
pins run on the real oracle (tests/test_oracle_pins.py) and on copies with a
planted mistake (tests/test_oracle_mutants.py).  Citations name sections of
"RidgeFill: Training-Free Late-Layer Cache Fill for Faster Prefill".
"""
import json
import math
import os

import numpy as np

import workloads
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _bits(a):
    return workloads.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


# ---------------------------------------------------------------- fill: rows

def pin_fill_rows_partition(o):
    """Section 2.1: each prefix row is exact or filled and the tail is exact,
    so filled and exact rows partition the prompt."""
    for name in ("tiny", "27b_120k", "8b_ragged_host"):
        s = workloads.spec(name)
        e = workloads.exact_row_list(s)
        f = o.fill_row_set(s.n_rows, e)
        assert np.all(np.diff(f) > 0), "fill rows must ascend"
        assert len(set(f.tolist()) & set(e.tolist())) == 0
        assert len(f) + len(set(e.tolist())) == s.n_rows
        start = 0
        for n in s.prompt_lens:
            tail = set(range(start + n - s.tail, start + n))
            assert not (tail & set(f.tolist())), "a tail row was filled"
            start += n
    # small case against Python sets, exact rows given unsorted and repeated
    e = [9, 3, 3, 17, 0]
    f = o.fill_row_set(20, np.array(e))
    assert f.tolist() == sorted(set(range(20)) - set(e))


# ---------------------------------------------------------------- fill: map

def pin_identity_map_is_exact_kv(o):
    """Sections 6-7: the identity fill (A = I, b = 0, POP's fill) makes each
    skipped layer project the unchanged state, so the fill equals the exact
    layer's cache write from the same input, bit for bit in fp64."""
    g = _rng(1)
    n, d, hd, nkv = 7, 64, 16, 2
    x = o.bf16_bits_to_f64(_bits(g.standard_normal((n, d))))
    gamma = 1 + 0.1 * g.standard_normal(d)
    wk = g.standard_normal((nkv * hd, d)) / 8
    wv = g.standard_normal((nkv * hd, d)) / 8
    pos = g.integers(0, 5000, n)
    y = o.predicted_input(x, np.eye(d), np.zeros(d))
    assert np.array_equal(y, x)
    k1, v1 = o.fill_layer(x, np.eye(d), np.zeros(d), gamma, wk, wv, pos, 1e4, hd, 1e-5)
    k2, v2 = o.layer_kv(x, gamma, wk, wv, pos, 1e4, hd, 1e-5)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def pin_map_orientation(o):
    """Section 2.2: A_l has d_out rows and d_in columns and x_hat = A_l x_S + b_l.
    A cyclic-shift matrix must move feature k to output (k+1) mod d, and a wide
    map [I | 0] (d_in > d_out, as on Flash-Next) must keep the leading d_out
    features; both are checked against numpy indexing."""
    g = _rng(2)
    d = 12
    x = g.standard_normal((5, d))
    perm = (np.arange(d) - 1) % d         # output n reads feature n-1
    a = np.zeros((d, d))
    a[np.arange(d), perm] = 1.0
    b = g.standard_normal(d)
    y = o.predicted_input(x, a, b)
    assert np.allclose(y, np.take(x, perm, axis=1) + b, rtol=0, atol=1e-15)
    d_in, d_out = 20, 8
    wide = np.zeros((d_out, d_in))
    wide[np.arange(d_out), np.arange(d_out)] = 1.0
    xw = g.standard_normal((3, d_in))
    yw = o.predicted_input(xw, wide, np.zeros(d_out))
    assert yw.shape == (3, d_out)
    assert np.array_equal(yw, xw[:, :d_out])


def pin_bias_only_map(o):
    """Section 2.2: with A = 0 every prediction is b; then every filled row's V is
    the same vector and each K is that one key rotated to the row's position
    (the rotation written as complex multiplication)."""
    g = _rng(3)
    d, hd, nkv, n = 32, 8, 2, 6
    bvec = g.standard_normal(d)
    gamma = 1 + 0.1 * g.standard_normal(d)
    wk = g.standard_normal((nkv * hd, d))
    wv = g.standard_normal((nkv * hd, d))
    pos = np.array([0, 1, 7, 100, 4095, 65535])
    x = g.standard_normal((n, d))
    k, v = o.fill_layer(x, np.zeros((d, d)), bvec, gamma, wk, wv, pos, 1e4, hd, 1e-5)
    assert np.allclose(v, v[0][None, :], rtol=0, atol=1e-13)
    k0 = k[0]  # position 0: unrotated
    half = hd // 2
    for r in range(n):
        for h in range(nkv):
            z0 = k0[h * hd:h * hd + half] + 1j * k0[h * hd + half:(h + 1) * hd]
            z = z0 * np.exp(1j * pos[r] * 1e4 ** (-2.0 * np.arange(half) / hd))
            got = k[r, h * hd:h * hd + half] + 1j * k[r, h * hd + half:(h + 1) * hd]
            assert np.allclose(got, z, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- fill: norm

def pin_rmsnorm_closed_forms(o):
    """The layer's RMSNorm (section 2.2 "At inference"): for a constant row c the
    output is gamma * c / sqrt(c^2 + eps); for any row, mean((h/gamma)^2) equals
    m / (m + eps) with m = mean(y^2); with eps = 0 it is scale free."""
    g = _rng(4)
    d = 40
    gamma = 1 + 0.1 * g.standard_normal(d)
    for c in (0.3, -2.0, 17.0):
        h = o.rms_norm(np.full((1, d), c), gamma, 1e-5)
        assert np.allclose(h[0], gamma * c / math.sqrt(c * c + 1e-5), rtol=1e-14, atol=0)
    y = g.standard_normal((9, d)) * g.uniform(0.1, 10, (9, 1))
    eps = 0.37
    h = o.rms_norm(y, gamma, eps)
    m = np.mean(y * y, axis=1)
    assert np.allclose(np.mean((h / gamma) ** 2, axis=1), m / (m + eps), rtol=1e-13)
    h1 = o.rms_norm(y, gamma, 0.0)
    h2 = o.rms_norm(5.5 * y, gamma, 0.0)
    assert np.allclose(h1, h2, rtol=1e-13, atol=1e-14)


def pin_one_hot_layer_kv(o):
    """Layer cache write for a scaled one-hot input c e_j (sections 2.1-2.2): the
    norm gives gamma_j c / sqrt(c^2/d + eps) on feature j only, so V is that
    number times column j of W_v, and at position 0 K is it times column j of
    W_k; V does not depend on the position."""
    g = _rng(5)
    d, hd, nkv = 24, 8, 3
    gamma = 1 + 0.1 * g.standard_normal(d)
    wk = g.standard_normal((nkv * hd, d))
    wv = g.standard_normal((nkv * hd, d))
    for j, c in ((0, 1.5), (5, -0.25), (23, 40.0)):
        hin = np.zeros((2, d))
        hin[:, j] = c
        k, v = o.layer_kv(hin, gamma, wk, wv, np.array([0, 12345]), 5e5, hd, 1e-5)
        s = gamma[j] * c / math.sqrt(c * c / d + 1e-5)
        assert np.allclose(v[0], s * wv[:, j], rtol=1e-13, atol=1e-13)
        assert np.allclose(v[1], v[0], rtol=0, atol=0)
        assert np.allclose(k[0], s * wk[:, j], rtol=1e-13, atol=1e-13)
        assert not np.allclose(k[1], k[0])


# ---------------------------------------------------------------- fill: rope

def pin_rope_is_complex_rotation(o):
    """Rotary embedding (section 2.2; section 6.6 "rotated at their own
    positions"): in each head, (k_j, k_{j+hd/2}) as the complex number
    k_j + i k_{j+hd/2} is multiplied by exp(i pos theta^(-2j/hd))."""
    g = _rng(6)
    for hd, theta in ((64, 1e4), (128, 5e5)):
        n, nkv = 5, 3
        k = g.standard_normal((n, nkv * hd))
        pos = np.array([0, 1, 511, 65535, 122879])
        out = o.rope(k, pos, theta, hd)
        half = hd // 2
        freq = theta ** (-2.0 * np.arange(half) / hd)
        for r in range(n):
            for h in range(nkv):
                z = (k[r, h * hd:h * hd + half] + 1j * k[r, h * hd + half:(h + 1) * hd]) \
                    * np.exp(1j * pos[r] * freq)
                assert np.allclose(out[r, h * hd:h * hd + half], z.real, rtol=1e-12, atol=1e-12)
                assert np.allclose(out[r, h * hd + half:(h + 1) * hd], z.imag, rtol=1e-12, atol=1e-12)


def pin_rope_invariants(o):
    """Rotations keep each pair's norm, position 0 is the identity, the dot
    product of two rotated keys depends only on the position difference, and
    pair 0 turns by exactly pos radians."""
    g = _rng(7)
    hd, theta = 128, 5e5
    half = hd // 2
    a = g.standard_normal((1, 2 * hd))
    c = g.standard_normal((1, 2 * hd))
    assert np.array_equal(o.rope(a, np.array([0]), theta, hd), a)
    ra = o.rope(a, np.array([9999]), theta, hd)
    for h in range(2):
        s = slice(h * hd, (h + 1) * hd)
        n0 = a[0, s][:half] ** 2 + a[0, s][half:] ** 2
        n1 = ra[0, s][:half] ** 2 + ra[0, s][half:] ** 2
        assert np.allclose(n0, n1, rtol=1e-12)
    for m, n, sh in ((3, 10, 1000), (0, 70000, 52879)):
        d1 = np.sum(o.rope(a, np.array([m]), theta, hd)[0, :hd] * o.rope(c, np.array([n]), theta, hd)[0, :hd])
        d2 = np.sum(o.rope(a, np.array([m + sh]), theta, hd)[0, :hd]
                    * o.rope(c, np.array([n + sh]), theta, hd)[0, :hd])
        assert abs(d1 - d2) < 1e-9 * (1 + abs(d1))
    e = np.zeros((1, hd))
    e[0, 0] = 1.0
    r = o.rope(e, np.array([2]), theta, hd)
    assert abs(r[0, 0] - math.cos(2.0)) < 1e-15 and abs(r[0, half] - math.sin(2.0)) < 1e-15


# ---------------------------------------------------------------- fill: whole

def pin_brute_force_tiny(o):
    """A separately written pure-Python loop version of the whole fill agrees
    with the vectorised oracle on a few rows of the tiny workload, every layer,
    including a large position."""
    w = workloads.make(workloads.spec("tiny"))
    s = w.spec
    rows = np.array([0, 1, 255, 447])
    ref = o.fill_workload(w, rows=rows)
    for l in range(s.n_late):
        for i, r in enumerate(rows):
            kb, vb = brute.filled_row(w.x[r].tolist(), w.map_a[l].tolist(), w.map_b[l].tolist(),
                                      w.gamma[l].tolist(), w.w_k[l].tolist(), w.w_v[l].tolist(),
                                      int(w.positions[r]), s.rope_theta, s.head_dim, s.rms_eps)
            kr, vr = ref[l][0][i], ref[l][1][i]
            assert np.max(np.abs(np.array(kb) - kr)) <= 1e-12 * np.max(np.abs(kr))
            assert np.max(np.abs(np.array(vb) - vr)) <= 1e-12 * np.max(np.abs(vr))


def _position_in_prompt(prompt_lens, r):
    """Row r's position inside its own prompt, by walking the prompt lengths."""
    start = 0
    for n in prompt_lens:
        if r < start + n:
            return r - start
        start += n
    raise IndexError(r)


def pin_ragged_positions_brute(o):
    """Sections 2.2 and 6.6: each key is rotated at its own row's position,
    and in a batch of requests that position restarts at 0 with every
    request.  A tiny batch of three prompts, rows taken from all three (the
    first row of a later prompt among them), against the plain-loop row of
    tests/brute.py for the four workload-level functions: filled K/V, exact
    K/V from given layer inputs, and the indexer keys of both.  Positions are
    counted here from the prompt lengths, not read from the workload."""
    s = workloads.spec("tiny", d_in=128, d_out=128, n_late=2, prompt_lens=(40, 24, 33), tail=8,
                       idx_heads=1, seed=11)
    w = workloads.make(s)
    rows = np.array([3, 41, 55, 64, 80])
    pos = [_position_in_prompt(s.prompt_lens, int(r)) for r in rows]
    assert pos == [3, 1, 15, 0, 16]
    truth = workloads.make_layer_truth(s, s.n_rows, outliers=w.outlier_channels)[0]
    eye = _bits(np.eye(s.d_out))
    zero = _bits(np.zeros(s.d_out))
    fill = o.fill_workload(w, rows=rows)
    exact = o.exact_kv_workload(w, truth, rows)
    fidx = o.fill_indexer_workload(w, rows=rows)
    eidx = o.exact_indexer_workload(w, truth, rows)

    def close(got, want):
        want = np.array(want)
        assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))

    for l in range(s.n_late):
        args = (w.gamma[l].tolist(), w.w_k[l].tolist(), w.w_v[l].tolist())
        for i, r in enumerate(rows):
            p = pos[i]
            kb, vb = brute.filled_row(w.x[r].tolist(), w.map_a[l].tolist(), w.map_b[l].tolist(), *args,
                                      p, s.rope_theta, s.head_dim, s.rms_eps)
            close(fill[l][0][i], kb)
            close(fill[l][1][i], vb)
            ke, ve = brute.filled_row(truth[r].tolist(), eye.tolist(), zero.tolist(), *args,
                                      p, s.rope_theta, s.head_dim, s.rms_eps)
            close(exact[l][0][i], ke)
            close(exact[l][1][i], ve)
            wi = w.w_idx[l].tolist()
            ki, _ = brute.filled_row(w.x[r].tolist(), w.map_a[l].tolist(), w.map_b[l].tolist(),
                                     w.gamma[l].tolist(), wi, wi, p, s.rope_theta, s.head_dim, s.rms_eps)
            close(fidx[l][i], ki)
            kie, _ = brute.filled_row(truth[r].tolist(), eye.tolist(), zero.tolist(), w.gamma[l].tolist(), wi, wi,
                                      p, s.rope_theta, s.head_dim, s.rms_eps)
            close(eidx[l][i], kie)


def pin_fill_row_independence(o):
    """Section 2.1: a filled row's input comes straight from its own split state,
    so its K/V do not depend on which other rows are filled with it."""
    w = workloads.make(workloads.spec("tiny", n_late=2))
    rows = np.array([3, 40, 41, 300])
    full = o.fill_workload(w, rows=rows)
    for i, r in enumerate(rows):
        one = o.fill_workload(w, rows=np.array([r]))
        for l in full:
            assert np.allclose(one[l][0][0], full[l][0][i], rtol=1e-13, atol=1e-13)
            assert np.allclose(one[l][1][0], full[l][1][i], rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- ridge

def _linear_data(seed, n, d_in, d_out, noise=0.0):
    g = _rng(seed)
    x = g.standard_normal((n, d_in)) * g.uniform(0.2, 3.0, d_in) + g.standard_normal(d_in)
    m = g.standard_normal((d_out, d_in))
    c = g.standard_normal(d_out)
    y = x @ m.T + c + noise * g.standard_normal((n, d_out))
    return x, y, m, c


def pin_ridge_recovers_linear_map(o):
    """Section 2.2: on noise-free data from a known affine map, the ridge map's
    error falls monotonically to zero as lambda goes to zero."""
    x, y, m, c = _linear_data(8, 200, 16, 12)
    errs = []
    for lam in (1e-1, 1e-3, 1e-6, 1e-12):
        a, b = o.ridge_fit(x, y, lam)
        errs.append(np.linalg.norm(a - m) / np.linalg.norm(m))
        if lam == 1e-12:
            assert np.allclose(b, c, rtol=0, atol=1e-8)
    assert all(e1 > e2 for e1, e2 in zip(errs, errs[1:]))
    assert errs[-1] < 1e-8


def pin_ridge_svd_form(o):
    """Section 2.2 at an intermediate lambda: with Xc = U S V^T and Y = X M^T + c
    the solution is A^T = V diag(s^2/(s^2+alpha)) V^T M^T, alpha = lambda sum(s^2)/d_in
    (the trace of the centred Gram matrix), and b = mu_Y - A mu_X."""
    x, y, m, c = _linear_data(9, 90, 10, 7)
    lam = 0.03
    xc = x - x.mean(axis=0)
    _, sv, vt = np.linalg.svd(xc, full_matrices=False)
    alpha = lam * np.sum(sv ** 2) / x.shape[1]
    at = vt.T @ np.diag(sv ** 2 / (sv ** 2 + alpha)) @ vt @ m.T
    a, b = o.ridge_fit(x, y, lam)
    assert np.allclose(a, at.T, rtol=1e-10, atol=1e-11)
    assert np.allclose(b, y.mean(axis=0) - at.T @ x.mean(axis=0), rtol=1e-10, atol=1e-10)


def pin_ridge_running_sums(o):
    """Section 2.2 "Fitting": sums accumulated document by document lead to the
    same map as one solve over all rows; a different lambda needs one more solve."""
    x, y, _, _ = _linear_data(10, 300, 14, 9, noise=0.5)
    acc = o.RidgeSums(14, 9)
    for a0, a1 in ((0, 17), (17, 150), (150, 151), (151, 300)):
        acc.add(x[a0:a1], y[a0:a1])
    for lam in (0.03, 0.001):
        a1, b1 = acc.solve(lam)
        a2, b2 = o.ridge_fit(x, y, lam)
        assert np.allclose(a1, a2, rtol=1e-9, atol=1e-11)
        assert np.allclose(b1, b2, rtol=1e-9, atol=1e-11)


def pin_ridge_penalty_scale(o):
    """Section 2.2 "The penalty": alpha = lambda tr(X^T X)/d_in scales with the
    inputs, so scaling X by c scales A by 1/c and leaves b and every prediction
    unchanged (a fixed alpha would not)."""
    x, y, _, _ = _linear_data(11, 120, 8, 5, noise=1.0)
    a1, b1 = o.ridge_fit(x, y, 0.2)
    a2, b2 = o.ridge_fit(7.0 * x, y, 0.2)
    assert np.allclose(a2, a1 / 7.0, rtol=1e-10, atol=1e-13)
    assert np.allclose(b1, b2, rtol=1e-10, atol=1e-12)
    assert np.allclose(x @ a1.T + b1, (7.0 * x) @ a2.T + b2, rtol=1e-10, atol=1e-10)


def pin_ridge_raw_form(o):
    """The uncentred form W = (X^T X + lambda I)^(-1) X^T Y tends to the least
    squares solution (numpy lstsq) as lambda -> 0 and has no offset."""
    g = _rng(12)
    x = g.standard_normal((80, 6))
    y = g.standard_normal((80, 4))
    a, b = o.ridge_fit_raw(x, y, 1e-13)
    w_ls = np.linalg.lstsq(x, y, rcond=None)[0]
    assert np.allclose(a, w_ls.T, rtol=1e-9, atol=1e-11)
    assert np.array_equal(b, np.zeros(4))
    a2, _ = o.ridge_fit_raw(x, y, 5.0)
    assert np.allclose(a2.T, np.linalg.solve(x.T @ x + 5.0 * np.eye(6), x.T @ y), rtol=1e-12)


# ---------------------------------------------------------------- int8 maps

def _q8_case(seed, d_out, d_in, max_code=True):
    """Random codes (each block's largest |code| = 127 when max_code) and
    random positive bf16 scales."""
    g = _rng(seed)
    q = g.integers(-60, 61, size=(d_out, d_in)).astype(np.int8)
    if max_code:
        for o in range(d_out):
            for b in range(d_in // 128):
                k = b * 128 + int(g.integers(0, 128))
                q[o, k] = 127 if g.integers(0, 2) else -127
    s = _bits(np.exp(g.uniform(-9.0, 1.0, size=(d_out, d_in // 128))))
    return q, s


def pin_q8_dequant_closed_form(o):
    """Section 2.2 ("Size and cost"): a weight is its int8 code times the bf16
    scale of its 128-weight block in the same row."""
    q = np.zeros((2, 256), dtype=np.int8)
    q[0, 0], q[0, 127], q[0, 128], q[0, 255] = 3, -5, 7, 127
    q[1, 64], q[1, 200] = -128, 1
    s = np.array([[0x3F00, 0x4000], [0x3E80, 0xC040]], dtype=np.uint16)  # 0.5, 2, 0.25, -3
    w = o.dequantize_q8(q, s)
    want = np.zeros((2, 256))
    want[0, 0], want[0, 127], want[0, 128], want[0, 255] = 1.5, -2.5, 14.0, 254.0
    want[1, 64], want[1, 200] = -32.0, -3.0
    assert w.dtype == np.float64 and np.array_equal(w, want), np.argwhere(w != want)


def pin_q8_dequant_brute(o):
    """The same definition written as plain loops (tests/brute.py)."""
    q, s = _q8_case(11, 3, 384)
    w = o.dequantize_q8(q, s)
    ref = np.array(brute.dequant_q8(q.tolist(), s.tolist()))
    assert np.array_equal(w, ref)


def pin_q8_grid_fixpoint(o):
    """A map already on the int8 grid, whose blocks each reach code +-127,
    quantizes back to the same codes and scales: 127*s/127 = s exactly and
    q*s/s = q exactly."""
    q, s = _q8_case(12, 8, 512)
    a = o.dequantize_q8(q, s).astype(np.float32)
    assert np.array_equal(a.astype(np.float64), o.dequantize_q8(q, s)), "grid values must be fp32-exact"
    q2, s2 = o.quantize_q8(a)
    assert q2.dtype == np.int8 and s2.dtype == np.uint16
    assert np.array_equal(s2, s) and np.array_equal(q2, q)
    q3, s3 = o.quantize_q8(-a)
    assert np.array_equal(s3, s) and np.array_equal(q3, -q), "the format is symmetric"


def pin_q8_quantize_bounds(o):
    """Absmax quantization: every weight is within half a step of its code
    times the scale, each block's largest weight gets code +-127 with its sign,
    and the scale is the block's largest |weight| / 127 to bf16 precision."""
    g = _rng(13)
    d = 256
    a = (np.eye(d) + 0.01 * g.standard_normal((d, d))).astype(np.float32)
    a[5, :128] *= 1e4                           # a block of large weights
    a[7, 128:] = g.standard_t(2, size=128)      # heavy tails
    a[9, :128] = 0.0                            # an all-zero block
    q, sb = o.quantize_q8(a)
    s = o.dequantize_q8(np.ones_like(q), sb)    # per-weight scale
    err = np.abs(a.astype(np.float64) - q * s)
    assert np.all(err <= 0.5 * s * (1 + 1e-12)), float(np.max(err / np.where(s > 0, s, 1)))
    blocks = np.abs(a.astype(np.float64)).reshape(d, 2, 128)
    m = blocks.max(axis=2)
    arg = blocks.argmax(axis=2)
    for r in range(d):
        for b in range(2):
            k = b * 128 + arg[r, b]
            if m[r, b] == 0:
                assert sb[r, b] == 0 and not q[r, b * 128:(b + 1) * 128].any()
                continue
            assert abs(int(q[r, k])) == 127 and np.sign(q[r, k]) == np.sign(a[r, k]), (r, b)
            sv = o.bf16_bits_to_f64(sb[r, b])
            assert abs(sv - m[r, b] / 127) <= 2.0 ** -8 * m[r, b] / 127, (r, b)


def pin_q8_quantize_ties(o):
    """Codes round to the nearest integer with halves to even: with scale 0.5
    (block max 63.5), 1.25 -> 2, 1.75 -> 4, -0.25 -> 0, -0.75 -> -2."""
    a = np.zeros((1, 128), dtype=np.float32)
    a[0, :5] = [63.5, 1.25, 1.75, -0.25, -0.75]
    q, s = o.quantize_q8(a)
    assert s[0, 0] == 0x3F00, hex(int(s[0, 0]))
    assert q[0, :5].tolist() == [127, 2, 4, 0, -2], q[0, :5]


def pin_q8_quantize_brute(o):
    """The quantizer against plain loops (tests/brute.py)."""
    g = _rng(14)
    a = (g.standard_normal((4, 256)) * np.exp(g.uniform(-6, 6, size=(4, 1)))).astype(np.float32)
    a[2, 128:] = 0.0
    q, s = o.quantize_q8(a)
    qb, sbr = brute.quantize_q8(a.tolist())
    assert np.array_equal(q, np.array(qb)) and np.array_equal(s, np.array(sbr))


def pin_bf16_rounding_library(o):
    """One rounding to bf16, nearest even, as torch's float32 -> bfloat16 cast
    does, on random values and on exact halfway points."""
    import torch
    g = _rng(15)
    v = np.concatenate([g.standard_normal(4000) * np.exp(g.uniform(-20, 20, 4000)),
                        [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3 * 2.0 ** -9, 0.0]])
    v = v.astype(np.float32).astype(np.float64)
    got = o.f64_to_bf16_bits(v)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    assert o.f64_to_bf16_bits(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8])).tolist() == [0x3F80, 0x3F82]
    q, s = _q8_case(16, 2, 256)
    r = o.dequantize_q8_bf16(q, s)
    assert np.array_equal(r, ref_q := torch.from_numpy(o.dequantize_q8(q, s).astype(np.float32))
                          .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)), ref_q


# ---------------------------------------------------------------- QK-norm

def pin_qk_norm_closed_form(o):
    """Sections 6.6-7: layers with QK-norm normalise each key head.  Worked by
    hand: heads of 2, gain (1, 2), eps 0; head (3, 4) has mean square 12.5,
    head (0, 2) has 2."""
    k = np.array([[3.0, 4.0, 0.0, 2.0]])
    got = o.qk_norm(k, np.array([1.0, 2.0]), 0.0, 2)
    r1, r2 = math.sqrt(12.5), math.sqrt(2.0)
    want = np.array([[3 / r1, 2 * 4 / r1, 0.0, 2 * 2 / r2]])
    assert np.allclose(got, want, rtol=1e-15, atol=0), got
    # eps sits inside the root
    got = o.qk_norm(np.array([[1.0, 1.0]]), np.array([1.0, 1.0]), 3.0, 2)
    assert np.allclose(got, [[0.5, 0.5]], rtol=1e-15)


def pin_qk_norm_invariants(o):
    """Unit gain and eps 0 give every head RMS 1; scaling a row changes
    nothing; heads are normalised independently."""
    g = _rng(33)
    k = g.standard_normal((5, 4 * 16)) * np.exp(g.uniform(-3, 3, (5, 1)))
    u = o.qk_norm(k, np.ones(16), 0.0, 16)
    rms = np.sqrt(np.mean(u.reshape(5, 4, 16) ** 2, axis=2))
    assert np.allclose(rms, 1.0, rtol=1e-13)
    assert np.allclose(o.qk_norm(7.5 * k, np.ones(16), 0.0, 16), u, rtol=1e-13)
    k2 = k.copy()
    k2[:, 16:32] *= 100.0
    k2[:, 48:] = g.standard_normal((5, 16))
    u2 = o.qk_norm(k2, np.ones(16), 0.0, 16)
    assert np.array_equal(u2[:, :16], u[:, :16]) and np.array_equal(u2[:, 32:48], u[:, 32:48])


def pin_qk_layer_brute(o):
    """A layer with QK-norm against plain loops (tests/brute.py): norm, key
    projection, per-head key norm with a non-uniform gain, then the rotation."""
    g = _rng(34)
    d, hd, nkv, n = 32, 8, 2, 3
    bits = lambda a: _bits(a)
    x = bits(g.standard_normal((n, d)))
    a = bits(np.eye(d) + 0.05 * g.standard_normal((d, d)))
    b = bits(0.1 * g.standard_normal(d))
    gam = bits(1 + 0.1 * g.standard_normal(d))
    wk = bits(g.standard_normal((nkv * hd, d)) / np.sqrt(d))
    wv = bits(g.standard_normal((nkv * hd, d)) / np.sqrt(d))
    kg = bits(1 + 0.3 * g.standard_normal(hd))
    pos = np.array([0, 5, 77])
    f = o.bf16_bits_to_f64
    k, v = o.fill_layer(f(x), f(a), f(b), f(gam), f(wk), f(wv), pos, 1e4, hd, 1e-5, f(kg))
    for i in range(n):
        kb, vb = brute.filled_row(x[i], a, b, gam, wk, wv, int(pos[i]), 1e4, hd, 1e-5, kg)
        assert np.allclose(k[i], kb, rtol=1e-11, atol=1e-12), i
        assert np.allclose(v[i], vb, rtol=1e-11, atol=1e-12), i
    # without a gain the layer is the plain one
    k0, _ = o.fill_layer(f(x), f(a), f(b), f(gam), f(wk), f(wv), pos, 1e4, hd, 1e-5)
    kb0, _ = brute.filled_row(x[1], a, b, gam, wk, wv, 5, 1e4, hd, 1e-5)
    assert np.allclose(k0[1], kb0, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- indexer keys

def pin_indexer_one_hot(o):
    """Section 2.1 / 5.1: filled rows also write the indexer's key head.  Worked
    by hand at position 0 (no rotation): a one-hot projection row c picks
    gamma_c * y_c / sqrt(mean(y^2) + eps) of the row's input; at position p
    the pair (j, j + hd/2) of a 2-wide head turns by p * theta^0 = p radians."""
    y = np.array([[3.0, -4.0, 0.0, 12.0]])          # mean square 169/4
    gam = np.array([1.0, 2.0, 0.5, 1.0])
    w = np.zeros((2, 4))
    w[0, 1] = 1.0                                    # dim 0 <- feature 1
    w[1, 3] = 1.0                                    # dim 1 <- feature 3
    r = math.sqrt(169 / 4)
    got = o.indexer_keys(y, gam, w, np.array([0]), 1e4, 2, 0.0)
    assert np.allclose(got, [[2 * -4 / r, 12 / r]], rtol=1e-15, atol=0), got
    got = o.indexer_keys(y, gam, w, np.array([1]), 1e4, 2, 0.0)
    a, b = -8 / r, 12 / r
    want = [[a * math.cos(1) - b * math.sin(1), b * math.cos(1) + a * math.sin(1)]]
    assert np.allclose(got, want, rtol=1e-14, atol=1e-15), got


def pin_indexer_brute(o):
    """Indexer keys of filled rows against plain loops: the map, the norm, the
    indexer projection and the per-head rotation (tests/brute.py, whose key
    path is independent of the oracle), for two heads of 8 at three positions."""
    g = _rng(41)
    d, hd, n = 32, 8, 3
    bits = _bits
    x = bits(g.standard_normal((n, d)))
    a = bits(np.eye(d) + 0.05 * g.standard_normal((d, d)))
    b = bits(0.1 * g.standard_normal(d))
    gam = bits(1 + 0.1 * g.standard_normal(d))
    wi = bits(g.standard_normal((2 * hd, d)) / np.sqrt(d))
    pos = np.array([0, 9, 301])
    f = o.bf16_bits_to_f64
    got = o.indexer_keys(o.predicted_input(f(x), f(a), f(b)), f(gam), f(wi), pos, 1e4, hd, 1e-5)
    for i in range(n):
        kb, _ = brute.filled_row(x[i], a, b, gam, wi, wi, int(pos[i]), 1e4, hd, 1e-5)
        assert np.allclose(got[i], kb, rtol=1e-11, atol=1e-12), i


def pin_indexer_is_a_plain_key_head(o):
    """With W_idx equal to the first key head's rows the indexer key equals
    that head of a layer without QK-norm, and a QK-normed layer's gain leaves
    the indexer key untouched (it has no norm of its own)."""
    g = _rng(42)
    d, hd, nkv, n = 48, 16, 3, 4
    h = g.standard_normal((n, d))
    gam = 1 + 0.1 * g.standard_normal(d)
    wk = g.standard_normal((nkv * hd, d)) / np.sqrt(d)
    wv = g.standard_normal((nkv * hd, d)) / np.sqrt(d)
    pos = np.array([0, 3, 1000, 65000])
    k, _ = o.layer_kv(h, gam, wk, wv, pos, 5e5, hd, 1e-5)
    ik = o.indexer_keys(h, gam, wk[:hd], pos, 5e5, hd, 1e-5)
    assert np.array_equal(ik, k[:, :hd])
    kq, _ = o.layer_kv(h, gam, wk, wv, pos, 5e5, hd, 1e-5, 1 + 0.3 * g.standard_normal(hd))
    assert not np.allclose(kq[:, :hd], ik)


# ---------------------------------------------------------------- value rescale

def pin_rescale_closed_form(o):
    """Section 2.3 ("Value rescale"), worked by hand.  W_v = I, gain 1, eps 0,
    two heads of 2: an input row (3, 0, 0, 4) normalises to (1.2, 0, 0, 1.6),
    one of all ones to itself, so the head norms are (1.2, 1.6) and
    (sqrt 2, sqrt 2).  Request 0 has two rows, request 1 one; scales are
    means of per-row ratios, not ratios of mean norms."""
    s2 = math.sqrt(2.0)
    v_ex = np.array([[1.2, 0.0, 0.0, 1.6], [1.0, 1.0, 1.0, 1.0], [0.0, 3.0, 4.0, 0.0]])
    v_pr = np.array([[1.0, 1.0, 1.0, 1.0], [2.0, 0.0, 0.0, 1.0], [0.6, 0.8, 0.0, 2.0]])
    got = o.scales_from_values(v_ex, v_pr, np.array([0, 0, 1]), 2, 2)
    want = np.array([[(1.2 / s2 + s2 / 2.0) / 2, (1.6 / s2 + s2 / 1.0) / 2],
                     [3.0 / 1.0, 4.0 / 2.0]])
    assert np.allclose(got, want, rtol=1e-14, atol=0), (got, want)
    # a request with no rows, and a zero predicted head, keep scale 1
    got = o.scales_from_values(v_ex[:1], np.array([[0.0, 0.0, 3.0, 4.0]]), np.array([1]), 3, 2)
    assert np.allclose(got, [[1, 1], [1, 1.6 / 5.0], [1, 1]], rtol=1e-14)
    # the normalisation on the way in
    h = o.rms_norm(np.array([[3.0, 0.0, 0.0, 4.0]]), np.ones(4), 0.0)
    assert np.allclose(h, [[1.2, 0.0, 0.0, 1.6]], rtol=1e-15)
    # the rescale multiplies each head of each row by its request's scale
    sc = np.array([[2.0, 3.0], [5.0, 7.0]])
    r = o.rescale_values(np.ones((2, 4)), sc, np.array([1, 0]), 2)
    assert np.array_equal(r, [[5, 5, 7, 7], [2, 2, 3, 3]])


def _rescale_case(o, seed=30):
    s = workloads.spec("tiny", prompt_lens=(200, 120, 80), tail=40, seed=seed)
    w = workloads.make(s)
    rows, grp = workloads.calibration_row_list(s, 16)
    truth = workloads.make_layer_truth(s, len(rows), outliers=w.outlier_channels)
    return s, w, rows, grp, truth


def pin_rescale_identity_and_invariances(o):
    """True input = predicted input gives scale 1 exactly and leaves values
    unchanged; the norm removes any positive scaling of the true inputs
    (eps = 0); row order inside a request and other requests' rows do not
    matter."""
    s, w, rows, grp, truth = _rescale_case(o)
    xs = o.bf16_bits_to_f64(w.x[rows])
    g = o.bf16_bits_to_f64(w.gamma[0])
    wv = o.bf16_bits_to_f64(w.w_v[0])
    y_pred = o.predicted_input(xs, o.map_matrix(w, 0), o.bf16_bits_to_f64(w.map_b[0]))
    v_pred = o.project(o.rms_norm(y_pred, g, 0.0), wv)
    one = o.scales_from_values(v_pred, v_pred, grp, 3, s.head_dim)
    assert np.array_equal(one, np.ones_like(one))
    v = np.arange(8.0).reshape(2, 4) + 1
    assert np.array_equal(o.rescale_values(v, np.ones((3, 2)), np.array([2, 0]), 2), v)
    yt = o.bf16_bits_to_f64(truth[0])
    ve = o.project(o.rms_norm(yt, g, 0.0), wv)
    ve3 = o.project(o.rms_norm(3.5 * yt, g, 0.0), wv)
    a = o.scales_from_values(ve, v_pred, grp, 3, s.head_dim)
    b = o.scales_from_values(ve3, v_pred, grp, 3, s.head_dim)
    assert np.allclose(a, b, rtol=1e-12) and not np.allclose(a, 1.0, rtol=1e-3)
    perm = np.random.default_rng(1).permutation(len(rows))
    c = o.scales_from_values(ve[perm], v_pred[perm], grp[perm], 3, s.head_dim)
    assert np.allclose(a, c, rtol=1e-12)
    ve2 = ve.copy()
    ve2[grp == 1] *= 4.0
    d = o.scales_from_values(ve2, v_pred, grp, 3, s.head_dim)
    assert np.array_equal(d[[0, 2]], a[[0, 2]]) and np.allclose(d[1], 4.0 * a[1], rtol=1e-12)


def pin_rescale_brute(o):
    """value_scales against plain loops over the same projections (tests/brute.py)."""
    s, w, rows, grp, truth = _rescale_case(o, seed=31)
    sc = o.value_scales(w, truth, rows, grp, 3, layers=[1])
    g = o.bf16_bits_to_f64(w.gamma[1])
    wv = o.bf16_bits_to_f64(w.w_v[1])
    xs = o.bf16_bits_to_f64(w.x[rows])
    a = o.bf16_bits_to_f64(w.map_a[1])
    b = o.bf16_bits_to_f64(w.map_b[1])
    vp = (rms_ref(xs @ a.T + b, g, s.rms_eps)) @ wv.T
    ve = rms_ref(o.bf16_bits_to_f64(truth[1]), g, s.rms_eps) @ wv.T
    ref = np.array(brute.value_scale(ve.tolist(), vp.tolist(), grp.tolist(), 3, s.head_dim))
    assert np.allclose(sc[1], ref, rtol=1e-12), (sc[1], ref)


def rms_ref(y, g, eps):
    return g * y / np.sqrt((y * y).sum(axis=1, keepdims=True) / y.shape[1] + eps)


def pin_calibration_rows(o):
    """The first c rows of every request's tail: 4 ragged prompts, c below,
    at and above the tail length; the workload generator's list agrees."""
    lens, tail = (30, 9, 20, 5), 8
    rows, grp = o.calibration_rows(lens, tail, 3)
    assert rows.tolist() == [22, 23, 24, 31, 32, 33, 51, 52, 53, 59, 60, 61]
    assert grp.tolist() == [0, 0, 0, 1, 1, 1, 2, 2, 2, 3, 3, 3]
    rows, grp = o.calibration_rows(lens, tail, 50)
    assert rows.tolist() == list(range(22, 30)) + list(range(31, 39)) + list(range(51, 59)) + list(range(59, 64))
    for name in ("27b_120k", "8b_ragged_host"):
        s = workloads.spec(name)
        r1, g1 = o.calibration_rows(s.prompt_lens, s.tail, 512)
        r2, g2 = workloads.calibration_row_list(s, 512)
        assert np.array_equal(r1, r2) and np.array_equal(g1, g2)
        assert set(r1.tolist()) <= set(workloads.exact_row_list(s).tolist()), "calibration rows are tail rows"


def pin_rescaled_fill(o):
    """The rescaled fill keeps the keys and multiplies each value head by the
    scale of its row's request."""
    s, w, rows, grp, truth = _rescale_case(o, seed=32)
    fill = o.fill_row_set(s.n_rows, w.exact_rows)[::7]
    g_of_row = workloads.prompt_of_row(s)
    sc = {l: np.array([[1.5, 0.5], [2.0, 1.0], [0.25, 4.0]]) for l in range(s.n_late)}
    base = o.fill_workload(w, rows=fill)
    res = o.fill_workload_rescaled(w, sc, g_of_row, fill)
    for l in range(s.n_late):
        assert np.array_equal(res[l][0], base[l][0])
        f = sc[l][g_of_row[fill]]
        want = base[l][1] * np.repeat(f, s.head_dim, axis=1)
        assert np.array_equal(res[l][1], want)


# ---------------------------------------------------------------- ceilings

def pin_printed_ceilings(o):
    """Values the pages print (tests/golden/ceilings.json)."""
    with open(os.path.join(GOLDEN, "ceilings.json")) as f:
        gold = json.load(f)
    for c in gold["layer_ceiling"]["cases"]:
        v = o.layer_ceiling(c["L"], c["S"], c["T"], c["N"])
        assert abs(v - c["printed"]) <= 0.005 + 1e-12, (c, v)
    for c in gold["mac_ceiling"]["cases"]:
        v = o.mac_ceiling(c["skipped"])
        assert abs(v - c["printed"]) <= 0.005 + 1e-12, (c, v)


def pin_printed_map_sizes(o):
    """The map sizes the pages print (tests/golden/map_sizes.json), at the
    precision printed.  The 0.60 GiB of Flash-Next's maps pins the int8
    format's scale overhead to between 1.55% and 3.3% of the codes: a
    two-byte scale per 128 weights (1.56%) fits, one scale per row or none
    does not, and neither does bf16 storage."""
    with open(os.path.join(GOLDEN, "map_sizes.json")) as f:
        gold = json.load(f)
    for c in gold["cases"]:
        total = c["layers"] * o.map_bytes(c["d_in"], c["d_out"], c["format"])
        v = round(total / c["unit_bytes"], c["digits"])
        assert abs(v - c["printed"]) < 1e-9, (c, total / c["unit_bytes"])


FILL_PINS = [pin_fill_rows_partition, pin_identity_map_is_exact_kv, pin_map_orientation,
             pin_bias_only_map, pin_rmsnorm_closed_forms, pin_one_hot_layer_kv,
             pin_rope_is_complex_rotation, pin_rope_invariants, pin_brute_force_tiny,
             pin_ragged_positions_brute, pin_fill_row_independence, pin_qk_norm_closed_form, pin_qk_norm_invariants,
             pin_qk_layer_brute, pin_indexer_one_hot, pin_indexer_brute, pin_indexer_is_a_plain_key_head]
RIDGE_PINS = [pin_ridge_recovers_linear_map, pin_ridge_svd_form, pin_ridge_running_sums,
              pin_ridge_penalty_scale, pin_ridge_raw_form]
CEILING_PINS = [pin_printed_ceilings]
QUANT_PINS = [pin_q8_dequant_closed_form, pin_q8_dequant_brute, pin_q8_grid_fixpoint,
              pin_q8_quantize_bounds, pin_q8_quantize_ties, pin_q8_quantize_brute,
              pin_bf16_rounding_library, pin_printed_map_sizes]
RESCALE_PINS = [pin_rescale_closed_form, pin_rescale_identity_and_invariances, pin_rescale_brute,
                pin_calibration_rows, pin_rescaled_fill]
ALL_PINS = FILL_PINS + RIDGE_PINS + CEILING_PINS + QUANT_PINS + RESCALE_PINS
