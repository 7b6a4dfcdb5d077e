"""CPU oracle for the steered combine (test infrastructure only).

A steering direction is one unit vector v per steered layer; after the layer
the residual stream loses its component along v, h <- h - (h . v) v (kwkr.cn
Coder write-up, "实验加速投影": a per-layer unit direction projected out of the
stream after each steered layer).  Here it follows the combine: h is the
weighted sum of the token's K expert rows plus the residual, in fp64, and the
projection is taken before the one rounding to the output type.  Plain numpy;
shares nothing with the HIP library.
"""
from __future__ import annotations

import numpy as np


def project_out(h: np.ndarray, v: np.ndarray) -> np.ndarray:
    """h [T][H] (or [H]) minus its component along the unit vector v, in fp64."""
    h = np.asarray(h, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    return h - np.multiply.outer(h @ v, v)


def combine_rows(y_perm: np.ndarray, inv: np.ndarray, w: np.ndarray, residual=None) -> np.ndarray:
    """fp64 h[t] = sum_k w[t][k] y_perm[inv[t*K+k]] (+ residual[t]); y_perm and
    residual given as their values (floats)."""
    y = np.asarray(y_perm, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, K = w.shape
    inv = np.asarray(inv).reshape(T, K)
    h = np.zeros((T, y.shape[1]), dtype=np.float64)
    for k in range(K):
        h += w[:, k:k + 1] * y[inv[:, k]]
    if residual is not None:
        h += np.asarray(residual, dtype=np.float64)
    return h


def combine_steer(y_perm, inv, w, v, residual=None) -> np.ndarray:
    """The steered combine before rounding: project_out(combine_rows(...), v)."""
    return project_out(combine_rows(y_perm, inv, w, residual), v)
