"""fp64 oracle of the closed-form ridge map (validation of the maps only).

Test infrastructure only (see ``oracle/__init__.py``).

Section 2.2 of "RidgeFill: Training-Free Late-Layer Cache Fill for Faster
Prefill": with X and Y_l centred by their means mu_S and mu_l,

    A_l = Y_l^T X (X^T X + alpha I)^(-1),   b_l = mu_l - A_l mu_S,

only A is penalised, and ("The penalty") alpha = lambda tr(X^T X) / d_in,
the trace taken over the centred X.  "Fitting": X^T X, X^T Y and both means,
accumulated document by document, lead to the same maps as one solve over all
rows, and changing lambda needs only a new solve.

A is returned [d_out][d_in], the orientation the paper sizes it in.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def ridge_fit(x: np.ndarray, y: np.ndarray, lam: float) -> Tuple[np.ndarray, np.ndarray]:
    """Section 2.2: centred ridge with the trace-scaled penalty."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    mu_s = x.mean(axis=0)
    mu_l = y.mean(axis=0)
    xc = x - mu_s
    yc = y - mu_l
    gram = xc.T @ xc
    alpha = lam * np.trace(gram) / x.shape[1]
    # (X^T X + alpha I)^(-1) X^T Y is A^T because the Gram matrix is symmetric
    a = np.linalg.solve(gram + alpha * np.eye(x.shape[1]), xc.T @ yc).T
    b = mu_l - a @ mu_s
    return a, b


def ridge_fit_raw(x: np.ndarray, y: np.ndarray, lam: float) -> Tuple[np.ndarray, np.ndarray]:
    """The uncentred form W = (X^T X + lam I)^(-1) X^T Y with no offset: A = W^T, b = 0."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    w = np.linalg.solve(x.T @ x + lam * np.eye(x.shape[1]), x.T @ y)
    return w.T, np.zeros(y.shape[1])


class RidgeSums:
    """Section 2.2 "Fitting": running sums over documents, then one solve."""

    def __init__(self, d_in: int, d_out: int):
        self.n = 0
        self.sx = np.zeros(d_in)
        self.sy = np.zeros(d_out)
        self.sxx = np.zeros((d_in, d_in))
        self.sxy = np.zeros((d_in, d_out))

    def add(self, x: np.ndarray, y: np.ndarray) -> None:
        x = np.asarray(x, dtype=np.float64)
        y = np.asarray(y, dtype=np.float64)
        self.n += x.shape[0]
        self.sx += x.sum(axis=0)
        self.sy += y.sum(axis=0)
        self.sxx += x.T @ x
        self.sxy += x.T @ y

    def solve(self, lam: float) -> Tuple[np.ndarray, np.ndarray]:
        mu_s = self.sx / self.n
        mu_l = self.sy / self.n
        cxx = self.sxx - self.n * np.outer(mu_s, mu_s)
        cxy = self.sxy - self.n * np.outer(mu_s, mu_l)
        alpha = lam * np.trace(cxx) / cxx.shape[0]
        a = np.linalg.solve(cxx + alpha * np.eye(cxx.shape[0]), cxy).T
        b = mu_l - a @ mu_s
        return a, b
