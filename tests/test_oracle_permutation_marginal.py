"""The permutation's effect on the marginal of the rotated, normalised coordinates (informational;
parity unpinned: the pages state the effect qualitatively and print no figure for it).

OrbitQuant summary (picx.dev), "Randomized Permuted Block-Hadamard (RPBH) Rotation",
Proposition 1: the block-Hadamard rotation keeps each coordinate's marginal close to f_d, and
the fixed permutation drawn once per dimension spreads potential outliers across blocks.  The
distance from f_d is measured here with the oracle's dense rotation (oracle.rpbh_matrix) and
the closed-form CDF of f_d (oracle.density): the Kolmogorov-Smirnov distance of the pooled
coordinates t = x'/||x'||, and E[t^4] against its f_d value 3 / (d (d + 2)).

Measured on the inputs below (d = 1024, h = 64, 256 tokens): eight adjacent outlier channels
(x30, all inside one block without the permutation): KS 0.092 with pi against 0.195 without,
E[t^4] ratio 1.7 against 9.6; the heavy-tailed workload generator (outlier channels at random
positions): KS 0.034 against 0.029, ratio 1.45 against 1.37 (scattered outliers gain nothing
from the permutation).
"""
import numpy as np

import oracle
import workloads
from oracle import density

D, H, N = 1024, 64, 256


def _fd_cdf(x, d):
    x = np.asarray(x, dtype=np.float64)
    up = density._upper_tail(np.abs(x), d)  # mass of f_d above |x|
    return np.where(x >= 0, 1.0 - up, up)


def _distance(X, Pi):
    _, _, T = oracle.rotate_normalize(X, Pi)
    t = np.sort(T.ravel())
    emp = (np.arange(t.size) + 0.5) / t.size
    ks = float(np.max(np.abs(_fd_cdf(t, D) - emp)))
    m4 = float(np.mean(T ** 4) * D * (D + 2) / 3.0)
    return ks, m4


def _rotations():
    perm, signs = workloads.rotation(D, seed=11)
    return oracle.rpbh_matrix(D, H, perm, signs), oracle.rpbh_matrix(D, H, np.arange(D), signs)


def test_isotropic_inputs_have_the_fd_marginal():
    """Gaussian rows are rotation invariant, so t is uniform on the sphere and each coordinate
    has exactly the marginal f_d, with or without the permutation: a closed-form pin of the
    rotate-normalise step and of the f_d CDF used below."""
    X = np.random.default_rng(3).standard_normal((N, D))
    for Pi in _rotations():
        ks, m4 = _distance(X, Pi)
        assert ks < 0.01, ks
        assert abs(m4 - 1.0) < 0.03, m4


def test_permutation_spreads_clustered_outliers():
    X = np.random.default_rng(5).standard_normal((N, D))
    X[:, 0:8] *= 30.0  # adjacent outlier channels: one Hadamard block without the permutation
    P_perm, P_id = _rotations()
    ks_p, m4_p = _distance(X, P_perm)
    ks_i, m4_i = _distance(X, P_id)
    assert ks_p < 0.6 * ks_i, (ks_p, ks_i)
    assert m4_p < 0.5 * m4_i, (m4_p, m4_i)
