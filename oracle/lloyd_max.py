"""Lloyd-Max codebook for f_d by plain Lloyd iteration (oracle; test
infrastructure only).

OrbitQuant summary (picx.dev), "Theoretical Basis", item 2: an MSE-optimal
scalar quantizer precomputed offline from f_d with 2^b centroids.  TurboQuant
slides (docswell), "Page. 13" and "Page. 16": the codebook solves a continuous
one-dimensional k-means problem over the known density.

Lloyd's iteration alternates the two optimality conditions of a 1-D k-means:
  boundaries are midpoints of neighbouring centroids;
  each centroid is the conditional mean of f_d over its cell.
Start: Gaussian quantiles scaled by 1/sqrt(d) (the N(0, 1/d) limit).
f_d is even, so each step is projected onto exactly antisymmetric codebooks.
Stop when max |change| * sqrt(d) < tol.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.stats import norm

from .density import cell_mass, cell_moment


def lloyd_max(d: int, bits: int, tol: float = 1e-15, max_iter: int = 2_000_000,
              return_iters: bool = False):
    """2^bits float64 centroids, ascending and exactly antisymmetric."""
    n_lv = 1 << bits
    c = norm.ppf((np.arange(n_lv) + 0.5) / n_lv) / math.sqrt(d)
    c = 0.5 * (c - c[::-1])
    it = 0
    for it in range(1, max_iter + 1):
        b = 0.5 * (c[:-1] + c[1:])
        b[n_lv // 2 - 1] = 0.0
        lo = np.concatenate(([-1.0], b))
        hi = np.concatenate((b, [1.0]))
        new = cell_moment(lo, hi, d) / cell_mass(lo, hi, d)
        new = 0.5 * (new - new[::-1])
        delta = np.max(np.abs(new - c)) * math.sqrt(d)
        c = new
        if delta < tol:
            break
    else:
        raise RuntimeError(f"Lloyd iteration did not converge for d={d}, bits={bits}")
    return (c, it) if return_iters else c


def thresholds_midpoint(centroids) -> np.ndarray:
    """Exact midpoints (float64) between neighbouring centroids."""
    c = np.asarray(centroids, dtype=np.float64)
    return 0.5 * (c[:-1] + c[1:])
