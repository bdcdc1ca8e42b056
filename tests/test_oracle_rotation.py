"""Pins for oracle/rpbh.py (RPBH rotation as a dense matrix).

RPBH definition: OrbitQuant summary (picx.dev), "Randomized Permuted
Block-Hadamard (RPBH) Rotation"; orthogonality: "Offline Weight Quantization";
cancellation: "Online Activation Quantization".
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
import workloads


@pytest.mark.parametrize("h", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_is_sylvester_and_orthogonal(h):
    H = oracle.hadamard(h)
    # scipy builds the Sylvester matrix by recursive doubling, a different construction
    assert np.array_equal(H, scipy.linalg.hadamard(h))
    assert np.array_equal(H @ H.T, h * np.eye(h, dtype=np.int64))


@pytest.mark.parametrize("d,h", [(256, 64), (384, 128), (512, 128), (192, 64)])
def test_rpbh_orthogonal_and_norm_preserving(d, h):
    perm, signs = workloads.rotation(d, seed=7 + d)
    Pi = oracle.rpbh_matrix(d, h, perm, signs)
    assert np.max(np.abs(Pi @ Pi.T - np.eye(d))) < 1e-12
    x = np.random.default_rng(1).standard_normal((5, d))
    xr = oracle.rotate(x, Pi)
    assert np.allclose(np.linalg.norm(xr, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_rpbh_identity_permutation_is_block_hadamard():
    d, h = 256, 64
    Pi = oracle.rpbh_matrix(d, h, np.arange(d), np.ones(d, np.int8))
    ref = scipy.linalg.block_diag(*([scipy.linalg.hadamard(h) / np.sqrt(h)] * (d // h)))
    assert np.array_equal(Pi, ref)


@pytest.mark.parametrize("d,h", [(256, 64), (384, 128)])
def test_rpbh_factor_order_and_conventions(d, h):
    """x' = blkdiag(H_h D_i) P_pi x with (P x)_j = x[perm[j]] and D applied after P,
    built here from scipy's Hadamard block by block instead of one dense matrix."""
    perm, signs = workloads.rotation(d, seed=3 * d)
    x = np.random.default_rng(2).standard_normal(d)
    y = x[perm] * signs                      # D P x
    Hs = scipy.linalg.hadamard(h) / np.sqrt(h)
    ref = np.concatenate([Hs @ y[b * h:(b + 1) * h] for b in range(d // h)])
    got = oracle.rotate(x[None, :], oracle.rpbh_matrix(d, h, perm, signs))[0]
    assert np.allclose(got, ref, rtol=0, atol=1e-13)
    # the reversed order (sign by original index) must give a different result
    wrong = np.concatenate([Hs @ (x * signs)[perm][b * h:(b + 1) * h] for b in range(d // h)])
    assert not np.allclose(got, wrong)


def test_rotation_cancels_in_unquantized_product():
    """(X Pi^T)(W Pi^T)^T = X W^T: the rotation cancels (bound 1e-5 relative; float64 gives ~1e-15)."""
    d, h = 384, 128
    perm, signs = workloads.rotation(d)
    Pi = oracle.rpbh_matrix(d, h, perm, signs)
    rng = np.random.default_rng(5)
    X = rng.standard_t(3, (40, d)) * np.exp(rng.standard_normal(d))
    W = rng.standard_normal((30, d)) * 0.02
    Y = oracle.unquantized_fold(X, W, Pi)
    ref = X @ W.T
    assert np.linalg.norm(Y - ref) / np.linalg.norm(ref) < 1e-12


def test_rpbh_rejects_non_permutation():
    with pytest.raises(ValueError):
        oracle.rpbh_matrix(128, 64, np.zeros(128, np.int64), np.ones(128))


# ---------------------------------------------------------------- composed passes, flatness
def test_composed_single_pass_is_rpbh():
    perm, signs = workloads.rotation(256)
    assert np.array_equal(oracle.rpbh_composed(256, 64, perm, signs, 1), oracle.rpbh_matrix(256, 64, perm, signs))


def test_composed_order_by_hadamard_involution():
    """(H/sqrt h)^2 = I: a second pass with the identity permutation and all signs +1 undoes the
    first pass's block transform, leaving the signed permutation D_0 P_0 (Pi[j, perm[j]] =
    signs[j]).  Composing in the other order would leave dense blocks."""
    d, h = 512, 128
    perm, signs = workloads.rotation(d)
    P2 = np.concatenate([perm, np.arange(d, dtype=np.int32)])
    S2 = np.concatenate([signs, np.ones(d, np.int8)])
    Pi = oracle.rpbh_composed(d, h, P2, S2, 2)
    want = np.zeros((d, d))
    want[np.arange(d), perm] = signs
    assert np.max(np.abs(Pi - want)) < 1e-12


def test_composed_is_orthogonal_and_mixes_a_spike():
    d, h = 1024, 64
    p0, s0 = workloads.rotation(d)
    p1, s1 = workloads.rotation(d, seed=d + 7)
    Pi2 = oracle.rpbh_composed(d, h, np.concatenate([p0, p1]), np.concatenate([s0, s1]), 2)
    assert np.max(np.abs(Pi2 @ Pi2.T - np.eye(d))) < 1e-12
    # a one-hot input: one pass spreads it over exactly one block (h entries of 1/sqrt(h), so
    # rho3 = sqrt(d / h) exactly); the second pass spreads it over many blocks
    e = np.zeros((1, d)); e[0, 5] = 1.0
    one = oracle.rotate(e, oracle.rpbh_matrix(d, h, p0, s0))
    r1, _ = oracle.flatness(one)
    assert abs(r1[0] - np.sqrt(d / h)) < 1e-12 and np.count_nonzero(np.abs(one) > 1e-12) == h
    r2, _ = oracle.flatness(oracle.rotate(e, Pi2))
    assert r2[0] < 0.5 * r1[0]


def test_flatness_closed_forms():
    d = 4096
    X = np.zeros((4, d))
    X[0] = 3.0                       # constant: rho3 = rhoinf = 1
    X[1, 17] = -2.5                  # one-hot: sqrt(d) for both
    X[3] = np.random.default_rng(0).standard_normal(d)  # Gaussian: rho3 -> E|g|^3 = 2 sqrt(2/pi)
    r3, ri = oracle.flatness(X)
    assert abs(r3[0] - 1) < 1e-12 and abs(ri[0] - 1) < 1e-12
    assert abs(r3[1] - 64) < 1e-12 and abs(ri[1] - 64) < 1e-12
    assert r3[2] == 0 and ri[2] == 0  # zero row
    assert abs(r3[3] - 2 * np.sqrt(2 / np.pi)) < 0.05
    assert 2.5 < ri[3] < 5.5          # max of d Gaussians ~ sqrt(2 ln d) = 4.08


def test_two_passes_recover_gaussian_distortion_on_spikes():
    """The composed-transform claim ("Quantizing With Randomized Hadamard Transforms": two
    transforms give Gaussian scalar marginals for any input) in the layer's own terms: one-hot
    tokens quantized after one RPBH pass (h nonzero coordinates, the rest exactly 0) lose ~20x
    more than Gaussian tokens; after two passes they lose what Gaussian tokens lose."""
    from tests.conftest import oracle_codebook
    d, h = 3072, 128
    c = oracle_codebook(d, 4)
    P, S = workloads.rotation_passes(d, 2)
    rng = np.random.default_rng(0)
    spikes = np.zeros((12, d)); spikes[np.arange(12), rng.integers(0, d, 12)] = 1.0
    gauss = rng.standard_normal((12, d))

    def nmse(X, k):
        Pi = oracle.rpbh_composed(d, h, P, S, k)
        codes, s, _ = oracle.quantize_activations(X, Pi, c)
        err = c[codes] * s[:, None] - oracle.rotate(X, Pi)
        return float(np.mean(np.sum(err ** 2, axis=1) / np.sum(X ** 2, axis=1)))

    g1, s1, s2 = nmse(gauss, 1), nmse(spikes, 1), nmse(spikes, 2)
    assert s1 > 10 * g1
    assert abs(s2 - g1) < 0.25 * g1
