"""Speedup ceilings of section 2.5 and section 4.4 (reporting helpers).

Test infrastructure only (see ``oracle/__init__.py``).
"""
from __future__ import annotations


def layer_ceiling(n_layers: int, split: int, tail: int, n_rows: int) -> float:
    """Section 2.5, the compute-share equation: with every layer costing the same
    per row and free maps, r = S/L + (1 - S/L) T/N of exact prefill remains and
    the speedup is at most 1/r."""
    r = split / n_layers + (1.0 - split / n_layers) * tail / n_rows
    return 1.0 / r


def mac_ceiling(skipped_share: float) -> float:
    """Section 4.4 / Figure 10b: when run time scales with the multiply-accumulates
    done, skipping a share s of them speeds the work up by at most 1/(1 - s)."""
    return 1.0 / (1.0 - skipped_share)
