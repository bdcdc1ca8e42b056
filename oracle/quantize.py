"""Rotate, normalise and quantize rows (oracle; test infrastructure only).

OrbitQuant summary (picx.dev):
  "Online Activation Quantization": x' = Pi x; s = ||x'||_2; x~' = x'/(s + eps);
      x^' = s * Q(x~') with Q the nearest-centroid quantizer.
  "Offline Weight Quantization": W' = W Pi^T; r'_i = ||w'_i||_2; w~'_i = w'_i / r'_i;
      W^' = diag(r') Q(W~'); r' is stored in BF16.
  "Theoretical Basis", item 2: q(t) = argmin over the codebook of |t - c|.

Readings where the pages are silent:
  * eps = 1e-8 unless given; weight rows use the same s + eps form.
  * argmin ties go to the lower centroid index (numpy argmin returns the first).
  * r' is rounded to bf16 with round-to-nearest-even from the exact norm; the
    direction is normalised with the unrounded norm.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .rpbh import rotate


def bf16_rne(x) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even) of float64 x, as float64."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                  # x = m * 2^e, 0.5 <= |m| < 1
    q = np.rint(m * 256.0)              # 8 significant bits, round half to even
    return np.ldexp(q, e - 8)


def argmin_codes(T, centroids, chunk: int = 1 << 18) -> np.ndarray:
    """Brute-force nearest centroid index of every entry of T (int64, same shape).

    Distances |t - c| are taken in float64 over all centroids.  Where the two
    smallest float64 distances are within rounding of each other, the choice is
    settled with exact rational arithmetic (fractions.Fraction of the float64 t
    and of the centroid), and an exact tie goes to the lower index.
    """
    c = np.asarray(centroids, dtype=np.float64)
    T = np.asarray(T, dtype=np.float64)
    flat = T.reshape(-1)
    out = np.empty(flat.shape, dtype=np.int64)
    cq = [Fraction(float(v)) for v in c]
    for i in range(0, flat.size, chunk):
        tt = flat[i:i + chunk]
        dist = np.abs(tt[:, None] - c[None, :])
        k = np.argmin(dist, axis=1)
        dmin = dist[np.arange(len(tt)), k]
        near = np.abs(dist - dmin[:, None]) <= 4 * np.spacing(np.maximum(dmin, np.abs(tt)))[:, None]
        ambiguous = np.nonzero(near.sum(axis=1) > 1)[0]
        for a in ambiguous:
            tq = Fraction(float(tt[a]))
            cand = np.nonzero(near[a])[0]
            k[a] = min(cand, key=lambda j: (abs(tq - cq[j]), j))
        out[i:i + chunk] = k
    return out.reshape(T.shape)


def rotate_normalize(X, Pi, eps: float = 1e-8):
    """(x', s, t) for every row: x' = Pi x, s = ||x'||, t = x'/(s + eps)."""
    Xp = rotate(X, Pi)
    s = np.sqrt(np.sum(Xp * Xp, axis=1))
    T = Xp / (s + eps)[:, None]
    return Xp, s, T


def quantize_activations(X, Pi, centroids, eps: float = 1e-8):
    """Online activation quantization: (codes int64 [n, d], s float64 [n], t [n, d])."""
    _, s, T = rotate_normalize(X, Pi, eps)
    return argmin_codes(T, centroids), s, T


def fold_weights(W, Pi, centroids, eps: float = 1e-8):
    """Offline weight fold + quantize.

    Returns (codes int64 [m, d], r' as bf16 values in float64 [m],
    unrounded norms [m], t [m, d]).  Rows of W Pi^T are Pi w_i, so the fold is
    the same row operation as the activation path with the weight codebook.
    """
    codes, s, T = quantize_activations(W, Pi, centroids, eps)
    return codes, bf16_rne(s), s, T
