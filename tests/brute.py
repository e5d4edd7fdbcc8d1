"""Pure-Python loop version of one filled row, used only to pin the oracle.

Written from the method's description (RidgeFill, sections 2.1-2.2), not from
``oracle/fill.py``: explicit loops over features, ``math.cos``/``math.sin`` for
the rotation, no numpy arithmetic.  Small inputs only.
"""
import math


def _f(bits):
    import struct
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def filled_row(x_bits, a_bits, b_bits, g_bits, wk_bits, wv_bits, pos, theta, hd, eps):
    """K and V (lists of floats) that one late layer stores for one filled row."""
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
