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


def rpbh_composed(d: int, h: int, perm, signs: np.ndarray, passes: int) -> np.ndarray:
    """Pi = Pi_{passes-1} ... Pi_1 Pi_0 (float64 [d, d]): `passes` RPBH rotations applied one
    after the other, pass p with permutation perm[p d:(p+1) d] (None: the identity) and signs
    signs[p d:(p+1) d].

    "Quantizing With Randomized Hadamard Transforms" (gist.science), "Method": the composition
    R_k of k randomized Hadamard transforms, each a Hadamard matrix times its own Rademacher
    diagonal; here each factor is a whole RPBH pass, whose permutation mixes across blocks.
    """
    signs = np.asarray(signs)
    Pi = np.eye(d)
    for p in range(passes):
        pp = np.arange(d) if perm is None else np.asarray(perm)[p * d:(p + 1) * d]
        Pi = rpbh_matrix(d, h, pp, signs[p * d:(p + 1) * d]) @ Pi
    return Pi


def flatness(X: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-row (rho3, rhoinf) = (sqrt(d) ||x||_3^3 / ||x||_2^3, sqrt(d) ||x||_inf / ||x||_2),
    both 0 for a zero row.

    "Quantizing With Randomized Hadamard Transforms", "Method" (adaptive check): an O(d) look
    at the input's l3 norm (scalar quantization) or l_inf norm (vector quantization) tells
    whether it is already flat enough for fewer randomized Hadamard transforms.  Scaled so
    that a constant vector gives 1 and a one-hot vector sqrt(d).
    """
    X = np.asarray(X, dtype=np.float64)
    d = X.shape[1]
    l2 = np.sqrt(np.sum(X * X, axis=1))
    l3c = np.sum(np.abs(X) ** 3, axis=1)
    linf = np.max(np.abs(X), axis=1)
    safe = np.where(l2 > 0, l2, 1.0)
    rho3 = np.where(l2 > 0, np.sqrt(d) * l3c / safe ** 3, 0.0)
    rhoinf = np.where(l2 > 0, np.sqrt(d) * linf / safe, 0.0)
    return rho3, rhoinf
