"""Pure-Python loop version of one filled row, used only to pin the oracle.

Written from the method's description (RidgeFill, sections 2.1-2.2), not from
``oracle/fill.py``: explicit loops over features, ``math.cos``/``math.sin`` for
the rotation, no numpy arithmetic.  Small inputs only.
"""
import math


def _f(bits):
    import struct
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def filled_row(x_bits, a_bits, b_bits, g_bits, wk_bits, wv_bits, pos, theta, hd, eps, kg_bits=None):
    """K and V (lists of floats) that one late layer stores for one filled row.
    With kg_bits (a key-norm gain of hd values) each key head is RMS-normalised
    and scaled by the gain before its rotation."""
    d_out = len(a_bits)
    d_in = len(a_bits[0])
    x = [_f(v) for v in x_bits]
    y = []
    for n in range(d_out):
        acc = _f(b_bits[n])
        row = a_bits[n]
        for k in range(d_in):
            acc += _f(row[k]) * x[k]
        y.append(acc)
    ms = 0.0
    for v in y:
        ms += v * v
    ms /= d_out
    scale = 1.0 / math.sqrt(ms + eps)
    h = [_f(g_bits[n]) * y[n] * scale for n in range(d_out)]
    width = len(wk_bits)
    kk, vv = [], []
    for c in range(width):
        sk = 0.0
        sv = 0.0
        for n in range(d_out):
            sk += _f(wk_bits[c][n]) * h[n]
            sv += _f(wv_bits[c][n]) * h[n]
        kk.append(sk)
        vv.append(sv)
    if kg_bits is not None:
        for head in range(width // hd):
            base = head * hd
            ms = 0.0
            for j in range(hd):
                ms += kk[base + j] ** 2
            ms /= hd
            f = 1.0 / math.sqrt(ms + eps)
            for j in range(hd):
                kk[base + j] = kk[base + j] * f * _f(kg_bits[j])
    out = list(kk)
    half = hd // 2
    for head in range(width // hd):
        base = head * hd
        for j in range(half):
            phi = pos * theta ** (-(2.0 * j) / hd)
            c, s = math.cos(phi), math.sin(phi)
            p, q = kk[base + j], kk[base + j + half]
            out[base + j] = p * c - q * s
            out[base + j + half] = q * c + p * s
    return out, vv


# ---------------------------------------------------------------- int8 maps
# Written from the format's description (RidgeFill, section 2.2 "Size and
# cost": int8 codes, one bf16 scale for each 128-weight block of a row), with
# Python floats and struct only.

def _f32(v):
    """Nearest fp32 value of a Python float (struct rounds to nearest even)."""
    import struct
    return struct.unpack("<f", struct.pack("<f", v))[0]


def _bf16_nearest(v):
    """bf16 bit pattern nearest a finite fp32-representable value, ties to the
    even pattern, found by comparing the two bracketing bf16 values."""
    import struct
    u = struct.unpack("<I", struct.pack("<f", v))[0]
    lo = u >> 16
    cands = [lo, lo + 1]
    vals = [_f(c) for c in cands]
    d0, d1 = abs(vals[0] - v), abs(vals[1] - v)
    if d0 < d1:
        return cands[0]
    if d1 < d0:
        return cands[1]
    return cands[0] if cands[0] % 2 == 0 else cands[1]


def dequant_q8(q_rows, scale_bits_rows):
    """w[o][k] = q[o][k] * scale[o][k // 128], as nested lists of floats."""
    out = []
    for o, row in enumerate(q_rows):
        out.append([int(row[k]) * _f(scale_bits_rows[o][k // 128]) for k in range(len(row))])
    return out


def quantize_q8(a_rows):
    """Absmax int8 codes and bf16 scale bits per 128-weight block of each row."""
    q_rows, s_rows = [], []
    for row in a_rows:
        qr, sr = [], []
        for b0 in range(0, len(row), 128):
            blk = [float(v) for v in row[b0:b0 + 128]]
            m = 0.0
            for v in blk:
                m = max(m, abs(v))
            sb = _bf16_nearest(_f32(m / 127.0))
            s = _f(sb)
            sr.append(sb)
            for v in blk:
                if s == 0.0:
                    qr.append(0)
                    continue
                t = v / s
                n = round(t)  # Python rounds halves to even
                qr.append(max(-127, min(127, n)))
        q_rows.append(qr)
        s_rows.append(sr)
    return q_rows, s_rows


# ---------------------------------------------------------------- value rescale
# Written from the description of the value rescale (RidgeFill, section 2.3):
# per head, the mean over one request's calibration rows of each row's exact
# value norm divided by its predicted value norm.

def value_scale(v_exact_rows, v_pred_rows, groups, n_groups, head_dim):
    """Nested lists: scale[g][h] = mean over rows of group g of |ve_h| / |vp_h|."""
    width = len(v_exact_rows[0])
    n_heads = width // head_dim
    out = []
    for g in range(n_groups):
        row = []
        for h in range(n_heads):
            tot, cnt = 0.0, 0
            for ve, vp, gr in zip(v_exact_rows, v_pred_rows, groups):
                if gr != g:
                    continue
                se = sum(ve[h * head_dim + j] ** 2 for j in range(head_dim)) ** 0.5
                sp = sum(vp[h * head_dim + j] ** 2 for j in range(head_dim)) ** 0.5
                if sp == 0.0:
                    continue
                tot += se / sp
                cnt += 1
            row.append(tot / cnt if cnt else 1.0)
        out.append(row)
    return out
