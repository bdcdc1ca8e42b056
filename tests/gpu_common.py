"""Shared helpers for the GPU parity tests (test infrastructure)."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import workloads

_PI_CACHE: dict = {}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def dev_bf16(bits: np.ndarray):
    """bf16 bit patterns (uint16 numpy) -> torch bf16 tensor on the GPU."""
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t) -> np.ndarray:
    """torch bf16 tensor -> uint16 bit patterns on the host."""
    torch = torch_mod()
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dense_pi(d: int, h: int):
    key = (d, h)
    if key not in _PI_CACHE:
        perm, signs = workloads.rotation(d)
        _PI_CACHE.clear()
        _PI_CACHE[key] = oracle.rpbh_matrix(d, h, perm, signs)
    return _PI_CACHE[key]


def boundary_distance(T: np.ndarray, centroids: np.ndarray) -> np.ndarray:
    """Distance (t units) of every t to the nearest decision boundary (midpoint)."""
    m = oracle.thresholds_midpoint(centroids)
    idx = np.clip(np.searchsorted(m, T), 1, len(m) - 1)
    return np.minimum(np.abs(T - m[idx - 1]), np.abs(T - m[idx]))


def check_codes(k_gpu: np.ndarray, k_ref: np.ndarray, T_ref: np.ndarray, centroids, what: str,
                tol_t: float = 1e-5, max_frac: float = 1e-5) -> int:
    """Codes must be bit-exact except coordinates within tol_t of a decision boundary;
    those are counted and may be at most max_frac of all coordinates."""
    mism = k_gpu != k_ref
    n_m = int(mism.sum())
    if n_m:
        dist = boundary_distance(T_ref[mism], centroids)
        assert np.all(dist < tol_t), f"{what}: code mismatch {dist.max():.3g} from a boundary"
        assert np.all(np.abs(k_gpu[mism] - k_ref[mism]) == 1), f"{what}: non-adjacent code mismatch"
    assert n_m <= max_frac * k_ref.size, f"{what}: {n_m} mismatches of {k_ref.size}"
    log(f"  {what}: {n_m} boundary mismatches / {k_ref.size}")
    return n_m


def gemm_error(Y_gpu: np.ndarray, A: np.ndarray, B: np.ndarray, s: np.ndarray, r: np.ndarray) -> float:
    """max |Y_gpu - Y| / (s_i r_j sum_k |A_ik B_jk|) with A, B the decoded (bf16) operands."""
    Y = (A @ B.T) * s[:, None] * r[None, :]
    den = (np.abs(A) @ np.abs(B).T) * s[:, None] * r[None, :]
    return float(np.max(np.abs(Y_gpu - Y) / np.maximum(den, 1e-300)))


def check_rprime(got: np.ndarray, s_ref: np.ndarray, what: str) -> int:
    """Stored weight-row norms r' (bf16, as float64) against the oracle's exact norms s_ref: equal
    to the oracle's round-to-nearest-even bf16, or one bf16 ulp away only where the exact norm
    lies within 1e-6 (relative) of the bf16 rounding midpoint between the two (the fp32 norm the
    kernel rounds carries ~1e-7 relative error).  Returns the count of such midpoint cases."""
    r_ref = oracle.bf16_rne(s_ref)
    diff = got != r_ref
    n = int(diff.sum())
    if n:
        ulp = 2.0 ** (np.floor(np.log2(r_ref[diff])) - 7)
        assert np.all(np.abs(got[diff] - r_ref[diff]) <= ulp), f"{what}: r' more than one bf16 ulp off"
        mid = r_ref[diff] + np.sign(got[diff] - r_ref[diff]) * ulp / 2
        far = np.abs(s_ref[diff] - mid) > 1e-6 * s_ref[diff]
        assert not far.any(), (f"{what}: r' one ulp off away from a rounding midpoint "
                               f"(norm {s_ref[diff][far][:3]}, got {got[diff][far][:3]})")
    log(f"  {what}: r' differs from the oracle's bf16 at {n} midpoint rows of {got.size}")
    return n
