"""Planted mistakes in copies of the oracle must each fail some pin (CPU only).

Every mutant is the oracle's own source with one plausible mistake edited in
(a transposed operand, a dropped term, a wrong sign or index, a wrong axis),
executed as a fresh module.  The real oracle is never modified.
"""
import itertools
import os
import sys
import types

import pytest

from tests import pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
FILES = ("fill.py", "ridge.py", "ceiling.py", "quant.py", "rescale.py")

MUTANTS = {
    # the map
    "map_transposed": ("fill.py", [("return x_s @ a.T + b", "return x_s @ a + b")]),
    "map_bias_dropped": ("fill.py", [("return x_s @ a.T + b", "return x_s @ a.T")]),
    "map_bias_sign": ("fill.py", [("return x_s @ a.T + b", "return x_s @ a.T - b")]),
    # the norm
    "norm_eps_outside_root": ("fill.py", [(
        "gamma * y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)",
        "gamma * y / (np.sqrt(np.mean(y * y, axis=-1, keepdims=True)) + eps)")]),
    "norm_one_plus_gamma": ("fill.py", [("return gamma * y / np.sqrt", "return (1 + gamma) * y / np.sqrt")]),
    "norm_sum_not_mean": ("fill.py", [("np.mean(y * y, axis=-1", "np.sum(y * y, axis=-1")]),
    "norm_wrong_axis": ("fill.py", [("np.mean(y * y, axis=-1", "np.mean(y * y, axis=0")]),
    "norm_skipped": ("fill.py", [("h = rms_norm(h_in, gamma, eps)", "h = h_in")]),
    # the projections
    "proj_transposed": ("fill.py", [("return h @ w.T", "return h @ w")]),
    "proj_k_v_swapped": ("fill.py", [("k = project(h, w_k)", "k = project(h, w_v)"),
                                     ("v = project(h, w_v)", "v = project(h, w_k)")]),
    # the rotation
    "rope_freq_exponent": ("fill.py", [("-2.0 * j / head_dim", "-1.0 * j / head_dim")]),
    "rope_direction": ("fill.py", [("[lo * c - hi * s, hi * c + lo * s]", "[lo * c + hi * s, hi * c - lo * s]")]),
    "rope_interleaved_pairs": ("fill.py", [("lo = kh[..., :half]", "lo = kh[..., 0::2]"),
                                           ("hi = kh[..., half:]", "hi = kh[..., 1::2]")]),
    "rope_position_off_by_one": ("fill.py", [("np.asarray(positions, dtype=np.float64)[:, None]",
                                              "(np.asarray(positions, dtype=np.float64)[:, None] + 1)")]),
    "rope_on_values_too": ("fill.py", [("v = project(h, w_v)\n    return k, v", "v = rope(project(h, w_v), positions, theta, head_dim)\n    return k, v")]),
    # QK-norm
    "qk_eps_outside_root": ("fill.py", [("return (kh / np.sqrt(ms + eps) * k_gamma)", "return (kh / (np.sqrt(ms) + eps) * k_gamma)")]),
    "qk_mean_over_row": ("fill.py", [("ms = np.mean(kh * kh, axis=2, keepdims=True)", "ms = np.mean(kh * kh, axis=(1, 2), keepdims=True)")]),
    "qk_gain_before_norm": ("fill.py", [("return (kh / np.sqrt(ms + eps) * k_gamma)", "return (kh * k_gamma / np.sqrt(np.mean((kh * k_gamma) ** 2, axis=2, keepdims=True) + eps))")]),
    "qk_after_rope": ("fill.py", [("""    k = project(h, w_k)
    if k_gamma is not None:
        k = qk_norm(k, k_gamma, eps, head_dim)
    k = rope(k, positions, theta, head_dim)""", """    k = rope(project(h, w_k), positions, theta, head_dim)
    if k_gamma is not None:
        k = qk_norm(k, k_gamma, eps, head_dim)""")]),
    "qk_gain_reversed": ("fill.py", [("return (kh / np.sqrt(ms + eps) * k_gamma)", "return (kh / np.sqrt(ms + eps) * k_gamma[::-1])")]),
    # rows and decoding
    "rows_union_not_difference": ("fill.py", [("np.setdiff1d(", "np.union1d(")]),
    "rows_wrong_positions": ("fill.py", [("pos = w.positions[r]\n    out = {}\n    for l in (range(s.n_late) if layers is None else layers):\n        out[l] = fill_layer",
                                          "pos = w.positions[:len(r)]\n    out = {}\n    for l in (range(s.n_late) if layers is None else layers):\n        out[l] = fill_layer")]),
    # positions: the global row index instead of the row's position in its own prompt
    "pos_global_row_fill": ("fill.py", [("pos = w.positions[r]\n    out = {}\n    for l in (range(s.n_late) if layers is None else layers):\n        out[l] = fill_layer",
                                         "pos = r\n    out = {}\n    for l in (range(s.n_late) if layers is None else layers):\n        out[l] = fill_layer")]),
    "pos_global_row_exact_kv": ("fill.py", [("pos = w.positions[r]\n    out = {}\n    for l in (range(s.n_late) if layers is None else layers):\n        out[l] = layer_kv",
                                             "pos = r\n    out = {}\n    for l in (range(s.n_late) if layers is None else layers):\n        out[l] = layer_kv")]),
    "pos_global_row_fill_indexer": ("fill.py", [("pos = w.positions[r]\n    out = {}\n    for l in (range(s.n_late) if layers is None else layers):\n        y = predicted_input",
                                                 "pos = r\n    out = {}\n    for l in (range(s.n_late) if layers is None else layers):\n        y = predicted_input")]),
    "pos_global_row_exact_indexer": ("fill.py", [("pos = w.positions[r]\n    return {l: indexer_keys",
                                                  "pos = r\n    return {l: indexer_keys")]),
    "bf16_decode_shift": ("fill.py", [("astype(np.uint32) << 16", "astype(np.uint32) << 15")]),
    # the ridge fit
    "ridge_not_centred": ("ridge.py", [("xc = x - mu_s", "xc = x")]),
    # indexer keys
    "idx_no_rope": ("fill.py", [("return rope(project(rms_norm(h_in, gamma, eps), w_idx), positions, theta, head_dim)",
                                 "return project(rms_norm(h_in, gamma, eps), w_idx)")]),
    "idx_unnormed": ("fill.py", [("return rope(project(rms_norm(h_in, gamma, eps), w_idx), positions, theta, head_dim)",
                                  "return rope(project(h_in, w_idx), positions, theta, head_dim)")]),
    "idx_gain_dropped": ("fill.py", [("return rope(project(rms_norm(h_in, gamma, eps), w_idx), positions, theta, head_dim)",
                                      "return rope(project(rms_norm(h_in, 1.0, eps), w_idx), positions, theta, head_dim)")]),
    "idx_half_heads": ("fill.py", [("return rope(project(rms_norm(h_in, gamma, eps), w_idx), positions, theta, head_dim)",
                                    "return rope(project(rms_norm(h_in, gamma, eps), w_idx), positions, theta, head_dim // 2)")]),
    "idx_transposed": ("fill.py", [("return rope(project(rms_norm(h_in, gamma, eps), w_idx), positions, theta, head_dim)",
                                    "return rope(rms_norm(h_in, gamma, eps) @ w_idx, positions, theta, head_dim)")]),
    "ridge_alpha_not_trace_scaled": ("ridge.py", [("alpha = lam * np.trace(gram) / x.shape[1]", "alpha = lam")]),
    "ridge_offset_sign": ("ridge.py", [("b = mu_l - a @ mu_s\n    return a, b", "b = mu_l + a @ mu_s\n    return a, b")]),
    "ridge_sums_not_centred": ("ridge.py", [("cxx = self.sxx - self.n * np.outer(mu_s, mu_s)", "cxx = self.sxx")]),
    "ridge_raw_penalty": ("ridge.py", [("x.T @ x + lam * np.eye", "x.T @ x + lam * lam * np.eye")]),
    # the ceilings
    "ceiling_prefix_denominator": ("ceiling.py", [("* tail / n_rows", "* tail / (n_rows - tail)")]),
    "ceiling_mac_sign": ("ceiling.py", [("1.0 / (1.0 - skipped_share)", "1.0 / (1.0 + skipped_share)")]),
    # the int8 map format
    "q8_scale_tiled_not_repeated": ("quant.py", [("np.repeat(s, BLOCK, axis=1)", "np.tile(s, (1, BLOCK))")]),
    "q8_block_64": ("quant.py", [("BLOCK = 128", "BLOCK = 64")]),
    "q8_code_abs": ("quant.py", [("return q.astype(np.float64) * np.repeat", "return np.abs(q.astype(np.float64)) * np.repeat")]),
    "q8_absmax_over_128": ("quant.py", [("(m / 127.0)", "(m / 128.0)")]),
    "q8_round_floor": ("quant.py", [("q = np.rint(blocks / safe)", "q = np.floor(blocks / safe)")]),
    "q8_round_half_away": ("quant.py", [("q = np.rint(blocks / safe)", "q = np.trunc(blocks / safe + 0.5 * np.sign(blocks))")]),
    "q8_scale_truncated": ("quant.py", [("((u + 0x7FFF + ((u >> 16) & 1)) >> 16)", "(u >> 16)")]),
    "q8_max_over_rows": ("quant.py", [("m = np.abs(blocks).max(axis=2)", "m = np.abs(blocks).max(axis=2).max(axis=0, keepdims=True) + 0 * blocks[:, :, 0]")]),
    "bf16_round_truncates": ("quant.py", [("return ((u + 0x7FFF + lsb) >> 16)", "return ((u) >> 16)")]),
    "q8_size_one_scale_per_row": ("quant.py", [("return d_in * d_out + 2 * d_out * (d_in // BLOCK)",
                                                "return d_in * d_out + 2 * d_out")]),
    "q8_size_as_bf16": ("quant.py", [("return d_in * d_out + 2 * d_out * (d_in // BLOCK)",
                                      "return 2 * d_in * d_out + 2 * d_out * (d_in // BLOCK)")]),
    "bf16_round_ties_up": ("quant.py", [("return ((u + 0x7FFF + lsb) >> 16)", "return ((u + 0x8000) >> 16)")]),
    # the value rescale
    "rescale_ratio_of_means": ("rescale.py", [("np.mean(ne[ok, h] / npr[ok, h])", "np.mean(ne[ok, h]) / np.mean(npr[ok, h])")]),
    "rescale_inverted": ("rescale.py", [("np.mean(ne[ok, h] / npr[ok, h])", "np.mean(npr[ok, h] / ne[ok, h])")]),
    "rescale_squared_norms": ("rescale.py", [("return np.linalg.norm(v.reshape(n, width // head_dim, head_dim), axis=2)",
                                              "return np.sum(v.reshape(n, width // head_dim, head_dim) ** 2, axis=2)")]),
    "rescale_groups_ignored": ("rescale.py", [("sel = np.asarray(group) == g", "sel = np.ones(len(group), dtype=bool)")]),
    "rescale_last_c_rows": ("rescale.py", [("rows.extend(range(first, first + k))", "rows.extend(range(start + n - k, start + n))")]),
    "rescale_exact_not_normed": ("rescale.py", [("v_exact = project(rms_norm(bf16_bits_to_f64(layer_true[l]), g, s.rms_eps), wv)",
                                                 "v_exact = project(bf16_bits_to_f64(layer_true[l]), wv)")]),
    "rescale_keys_too": ("rescale.py", [("return {l: (k, rescale_values(v, scales[l], g, w.spec.head_dim))",
                                         "return {l: (rescale_values(k, scales[l], g, w.spec.head_dim), rescale_values(v, scales[l], g, w.spec.head_dim))")]),
    "rescale_heads_interleaved": ("rescale.py", [("np.repeat(scale[np.asarray(group_of_rows)], head_dim, axis=1)",
                                                  "np.tile(scale[np.asarray(group_of_rows)], (1, head_dim))")]),
    "rescale_zero_rows_counted": ("rescale.py", [("ok = sel & (npr[:, h] > 0)", "ok = sel")]),
    # more rotary, norm and ridge slips
    "rope_cos_sin_swapped": ("fill.py", [("c = np.cos(ang)[:, None, :]\n    s = np.sin(ang)[:, None, :]",
                                          "c = np.sin(ang)[:, None, :]\n    s = np.cos(ang)[:, None, :]")]),
    "rope_theta_exponent_positive": ("fill.py", [("np.power(np.float64(theta), -2.0 * j / head_dim)",
                                                  "np.power(np.float64(theta), 2.0 * j / head_dim)")]),
    "rope_theta_fixed_1e4": ("fill.py", [("np.power(np.float64(theta), -2.0 * j / head_dim)",
                                          "np.power(np.float64(10000.0), -2.0 * j / head_dim)")]),
    "norm_eps_dropped": ("fill.py", [("np.mean(y * y, axis=-1, keepdims=True) + eps)",
                                      "np.mean(y * y, axis=-1, keepdims=True))")]),
    "qk_eps_dropped": ("fill.py", [("np.sqrt(ms + eps)", "np.sqrt(ms)")]),
    "ridge_alpha_over_d_out": ("ridge.py", [("alpha = lam * np.trace(gram) / x.shape[1]",
                                             "alpha = lam * np.trace(gram) / y.shape[1]")]),
    "ridge_alpha_not_scaled": ("ridge.py", [("alpha = lam * np.trace(gram) / x.shape[1]", "alpha = lam")]),
    "ridge_sums_alpha_over_d_out": ("ridge.py", [("alpha = lam * np.trace(cxx) / cxx.shape[0]",
                                                  "alpha = lam * np.trace(cxx) / cxy.shape[1]")]),
    "ridge_sums_cross_not_centred": ("ridge.py", [("cxy = self.sxy - self.n * np.outer(mu_s, mu_l)", "cxy = self.sxy")]),
    "ridge_offset_mean_only": ("ridge.py", [("b = mu_l - a @ mu_s\n    return a, b", "b = mu_l\n    return a, b")]),
    # Not planted: leaving Y uncentred in ridge_fit while X is centred.  The
    # columns of Xc sum to zero, so Xc^T Y = Xc^T Yc and that copy computes the
    # same map (an equivalent mutant, not a mistake).
}

PINS_FOR = {"fill.py": pins.FILL_PINS, "ridge.py": pins.RIDGE_PINS, "ceiling.py": pins.CEILING_PINS,
            "quant.py": pins.QUANT_PINS, "rescale.py": pins.RESCALE_PINS}


_loads = itertools.count()


def _load(target, edits):
    """The oracle's files executed as a fresh package, with one file mutated.

    Each copy is registered under a package name of its own, so the relative
    imports between the oracle's files (rescale.py takes fill_workload from
    fill.py; fill.py takes the int8 expansion from quant.py when called)
    resolve to the copies, mutated one included, never to the real oracle."""
    pkg_name = f"_oracle_mutant_{next(_loads)}"
    pkg = types.ModuleType(pkg_name)
    pkg.__path__ = []
    sys.modules[pkg_name] = pkg
    ns = types.SimpleNamespace()
    for fn in FILES:
        with open(os.path.join(ORACLE_DIR, fn)) as f:
            src = f.read()
        if fn == target:
            for old, new in edits:
                assert src.count(old) >= 1, f"mutation anchor not found in {fn}: {old!r}"
                src = src.replace(old, new, 1)
        mod = types.ModuleType(f"{pkg_name}.{fn[:-3]}")
        mod.__package__ = pkg_name
        sys.modules[mod.__name__] = mod
        setattr(pkg, fn[:-3], mod)
        exec(compile(src, os.path.join(ORACLE_DIR, fn), "exec"), mod.__dict__)
        for k, v in vars(mod).items():
            if not k.startswith("_") and not hasattr(ns, k):
                setattr(ns, k, v)
    return ns


def test_mutant_imports_resolve_to_the_copy():
    """A mutation in fill.py reaches rescale.py's use of fill_workload."""
    o = _load("fill.py", [("return x_s @ a.T + b", "return x_s @ a.T + 2 * b")])
    assert o.fill_workload_rescaled.__globals__["fill_workload"] is o.fill_workload
    assert o.fill_workload.__module__ != "oracle.fill"


def test_unmutated_copy_passes():
    o = _load(None, [])
    for p in pins.ALL_PINS:
        p(o)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    target, edits = MUTANTS[name]
    o = _load(target, edits)
    caught = []
    for p in PINS_FOR[target]:
        try:
            p(o)
        except Exception as e:  # an assertion or a shape error both count
            caught.append((p.__name__, type(e).__name__))
            break
    assert caught, f"no pin fails for the planted mistake {name}"
