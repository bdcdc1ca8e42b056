"""RPBH rotation as an explicit dense matrix (oracle; test infrastructure only).

OrbitQuant summary (picx.dev), "Randomized Permuted Block-Hadamard (RPBH)
Rotation": Pi_d = blkdiag(H_h D_1, ..., H_h D_{d/h}) P_pi, with H_h an h x h
Walsh-Hadamard matrix, D_i Rademacher sign diagonals and P_pi a uniform random
permutation matrix.

Readings where the page is silent:
  * H_h is the Sylvester (natural-order) Hadamard matrix, scaled by 1/sqrt(h)
    so that Pi_d is orthogonal, as "Offline Weight Quantization" requires.
  * (P_pi x)_j = x_{perm[j]}; D_i multiplies position j after the
    permutation by signs[j]; the factors act right to left.
The fast transform is NOT used here: x' = Pi x is a plain dense product.
"""
from __future__ import annotations

import numpy as np


def hadamard(h: int) -> np.ndarray:
    """Sylvester Hadamard matrix H[i, j] = (-1)^popcount(i & j), int64 [h, h]."""
    if h < 1 or h & (h - 1):
        raise ValueError("h must be a power of two")
    i = np.arange(h, dtype=np.int64)
    parity = np.bitwise_count(i[:, None] & i[None, :]) & 1
    return np.where(parity == 0, 1, -1).astype(np.int64)


def rpbh_matrix(d: int, h: int, perm: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """Dense Pi_d (float64 [d, d]) = blkdiag(H_h D_i / sqrt(h)) P_pi.

    Row r of block b = r // h has entries H[r mod h, j mod h] * signs[j] / sqrt(h)
    at column perm[j] for every j in block b; all other entries are 0.
    """
    perm = np.asarray(perm, dtype=np.int64)
    signs = np.asarray(signs, dtype=np.float64)
    if d % h or perm.shape != (d,) or signs.shape != (d,):
        raise ValueError("bad rotation shape")
    if not np.array_equal(np.sort(perm), np.arange(d)):
        raise ValueError("perm is not a permutation")
    H = hadamard(h).astype(np.float64) / np.sqrt(h)
    Pi = np.zeros((d, d), dtype=np.float64)
    for b in range(d // h):
        rows = slice(b * h, (b + 1) * h)
        cols = np.arange(b * h, (b + 1) * h)
        # (blkdiag(H D) P)[r, perm[j]] = H[r, j] * signs[j]
        Pi[rows, perm[cols]] = H * signs[cols][None, :]
    return Pi


def rotate(X: np.ndarray, Pi: np.ndarray) -> np.ndarray:
    """x' = Pi x for every row x of X, i.e. X Pi^T ("Online Activation
    Quantization", step 1: applied as x Pi^T for token batches)."""
    return np.asarray(X, dtype=np.float64) @ Pi.T
