"""fp64 oracle of the int8 map format: dequantization and quantization.

Test infrastructure only (see ``oracle/__init__.py``).

"RidgeFill: Training-Free Late-Layer Cache Fill for Faster Prefill", section
2.2 ("Size and cost") and section 4.2 (the 27B configuration): a map keeps its
d_out x d_in shape, each weight is an int8 code, and each row carries one bf16
scale per 128 consecutive weights.  Readings the pages leave open, taken here:

* a weight is its code times its block's scale, w[o][k] = q[o][k] * s[o][k // 128]
  (a symmetric format: no zero point);
* the quantizer is absmax per block: s = the bf16 value (round to nearest even)
  of the fp32 value nearest max|a| / 127, and q = a / s rounded to the nearest
  integer (ties to even) and clipped to [-127, 127]; an all-zero block gets
  s = 0 and q = 0;
* scales are stored [d_out][d_in / 128] row-major, codes [d_out][d_in].
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


BLOCK = 128


def map_bytes(d_in: int, d_out: int, fmt: str) -> int:
    """Stored bytes of one map (section 2.2, "Size and cost": d_out rows of
    d_in weights): two per weight in bf16; for int8, one code per weight plus
    one two-byte bf16 scale for each block of BLOCK weights of a row."""
    if fmt == "bf16":
        return 2 * d_in * d_out
    if fmt == "q8":
        return d_in * d_out + 2 * d_out * (d_in // BLOCK)
    raise ValueError(f"unknown map format {fmt!r}")


def _decode_bf16(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _check(q: np.ndarray, scale_bits: np.ndarray) -> Tuple[int, int]:
    d_out, d_in = q.shape
    if d_in % BLOCK:
        raise ValueError(f"d_in={d_in} is not a multiple of {BLOCK}")
    if scale_bits.shape != (d_out, d_in // BLOCK):
        raise ValueError(f"scales have shape {scale_bits.shape}, expected {(d_out, d_in // BLOCK)}")
    return d_out, d_in


def dequantize_q8(q: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Exact fp64 weights of an int8 map: code times its block's bf16 scale."""
    d_out, d_in = _check(q, scale_bits)
    s = _decode_bf16(scale_bits)
    return q.astype(np.float64) * np.repeat(s, BLOCK, axis=1)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of float64 values that fp32 holds exactly, nearest even.

    Used for values such as q * s (an 8-bit code times an 8-bit significand,
    at most 16 significant bits), where going through fp32 adds no rounding.
    """
    f = np.asarray(v, dtype=np.float64)
    f32 = f.astype(np.float32)
    if not np.array_equal(f32.astype(np.float64), f, equal_nan=True):
        raise ValueError("values are not exactly representable in fp32")
    u = f32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def dequantize_q8_bf16(q: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """The int8 map rounded once to bf16 (bit patterns): RNE(q * s) per weight.

    The exact product q * s has at most 16 significant bits, so this is one
    rounding of the exact weight, the form a bf16 matrix unit consumes.
    """
    return f64_to_bf16_bits(dequantize_q8(q, scale_bits))


def _f32_to_bf16_bits(f32: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def quantize_q8(a: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Absmax int8 codes and bf16 block scales of an fp32 map [d_out][d_in].

    Returns (q int8 [d_out][d_in], scale bits uint16 [d_out][d_in/128]).
    """
    a = np.asarray(a, dtype=np.float32)
    d_out, d_in = a.shape
    if d_in % BLOCK:
        raise ValueError(f"d_in={d_in} is not a multiple of {BLOCK}")
    blocks = a.astype(np.float64).reshape(d_out, d_in // BLOCK, BLOCK)
    m = np.abs(blocks).max(axis=2)
    s_bits = _f32_to_bf16_bits((m / 127.0).astype(np.float32))
    s = _decode_bf16(s_bits)
    safe = np.where(s > 0, s, 1.0)[:, :, None]
    q = np.rint(blocks / safe)
    q = np.where(s[:, :, None] > 0, q, 0.0)
    q = np.clip(q, -127, 127).astype(np.int8).reshape(d_out, d_in)
    return q, s_bits
