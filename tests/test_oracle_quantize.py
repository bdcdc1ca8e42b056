"""Pins for oracle/quantize.py and oracle/linear.py.

Quantizer q(t) = argmin |t - c| over the codebook: OrbitQuant summary
(picx.dev) "Theoretical Basis" item 2.  Activation path: "Online Activation
Quantization"; weight fold: "Offline Weight Quantization"; product and
cancellation: "Online Activation Quantization" (last paragraph).
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import workloads


def test_argmin_against_threshold_count(cb):
    """Nearest-centroid index == number of midpoints strictly below t (ascending
    codebook, ties to the lower index), checked on every midpoint and its fp32
    neighbours plus a dense grid."""
    for d, bits in ((256, 4), (3072, 2), (1536, 6)):
        c = cb(d, bits)
        m = oracle.thresholds_midpoint(c)
        probes = [np.linspace(-1.2 * c[-1], 1.2 * c[-1], 20001)]
        for mid in m:
            f = np.float32(mid)
            probes.append(np.array([mid, np.nextafter(f, np.float32(-1)), f,
                                    np.nextafter(f, np.float32(1))], dtype=np.float64))
        t = np.concatenate(probes)
        k = oracle.argmin_codes(t, c)
        assert np.array_equal(k, np.searchsorted(m, t, side="left"))
        # every centroid maps to itself; exact midpoints go to the lower index
        assert np.array_equal(oracle.argmin_codes(c.astype(np.float64), c), np.arange(len(c)))
        assert np.array_equal(oracle.argmin_codes(m, c), np.arange(len(m)))


def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-6, 6, 100000),
                        [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -(1.0 + 2 ** -8)]])
    x32 = x.astype(np.float32)        # values exactly representable in fp32
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_rne(x32.astype(np.float64)), ref)


def test_quantize_brute_force_tiny(cb):
    """Tiny case against explicit Python loops over the definition."""
    d, h = 128, 64
    c = cb(128, 4)
    perm, signs = workloads.rotation(d, seed=11)
    Pi = oracle.rpbh_matrix(d, h, perm, signs)
    X = workloads.f64_from_bf16_bits(workloads.activations(3, d, seed=12, kind="heavy"))
    codes, s, T = oracle.quantize_activations(X, Pi, c, eps=1e-8)
    H = oracle.hadamard(h)
    for r in range(3):
        xr = [0.0] * d
        for i in range(d):                    # x'_i = sum_j Pi_ij x_j, written as the RPBH factors
            b, ii = divmod(i, h)
            xr[i] = sum(H[ii, jj] * signs[b * h + jj] * X[r, perm[b * h + jj]]
                        for jj in range(h)) / math.sqrt(h)
        sr = math.sqrt(sum(v * v for v in xr))
        assert abs(sr - s[r]) <= 1e-12 * sr
        for i in range(d):
            t = xr[i] / (sr + 1e-8)
            best = min(range(len(c)), key=lambda k: (abs(t - float(c[k])), k))
            assert codes[r, i] == best


def test_fold_norm_is_bf16_of_row_norm(cb):
    d, h = 256, 64
    perm, signs = workloads.rotation(d)
    Pi = oracle.rpbh_matrix(d, h, perm, signs)
    W = workloads.weights(50, d, seed=3, as_float=True)
    codes, r, s, _ = oracle.fold_weights(W, Pi, cb(d, 4))
    assert np.allclose(s, np.linalg.norm(W, axis=1), rtol=1e-13)      # rotation keeps the norm
    ref = torch.from_numpy(np.linalg.norm(W, axis=1).astype(np.float32)).to(torch.bfloat16)
    # one bf16 ulp at most, from double rounding through fp32 in the reference cast
    assert np.all(np.abs(r - ref.double().numpy()) <= 2.0 ** (np.floor(np.log2(r)) - 7))


def test_lut_gemm_triple_loop_tiny(cb):
    rng = np.random.default_rng(4)
    ca, cw = cb(64, 4), cb(64, 2)
    n, m, d = 3, 4, 16
    kx = rng.integers(0, 16, (n, d))
    kw = rng.integers(0, 4, (m, d))
    s = rng.uniform(0.5, 2.0, n)
    r = oracle.bf16_rne(rng.uniform(0.5, 2.0, m))
    Y = oracle.lut_gemm(kx, s, ca, kw, r, cw)
    la, lw = oracle.decode_lut_bf16(ca), oracle.decode_lut_bf16(cw)
    for i, j in itertools.product(range(n), range(m)):
        acc = 0.0
        for k in range(d):
            acc += la[kx[i, k]] * lw[kw[i * 0 + j, k]]
        assert abs(Y[i, j] - s[i] * r[j] * acc) <= 1e-14 * abs(s[i] * r[j]) * d


def test_lut_gemm_constant_codes(cb):
    ca, cw = cb(256, 4), cb(256, 4)
    n, m, d = 5, 7, 256
    s = np.linspace(1, 2, n)
    r = oracle.bf16_rne(np.linspace(0.1, 0.3, m))
    for k0 in (0, 7, 8, 15):
        Y = oracle.lut_gemm(np.full((n, d), k0), s, ca, np.full((m, d), k0), r, cw)
        ref = s[:, None] * r[None, :] * d * oracle.decode_lut_bf16(ca)[k0] * oracle.decode_lut_bf16(cw)[k0]
        assert np.allclose(Y, ref, rtol=1e-14)


@pytest.mark.parametrize("bits", [2, 4, 6])
def test_end_to_end_error_tracks_codebook_distortion(bits, cb):
    """The quantized product approaches X W^T with relative error ~ sqrt(D_a + D_w),
    D_b = d E(t - q(t))^2 (the per-vector MSE).  A dropped norm, an uncancelled
    rotation or a transposed operand gives O(1) error instead."""
    d, h, n, m = 256, 64, 64, 96
    perm, signs = workloads.rotation(d)
    Pi = oracle.rpbh_matrix(d, h, perm, signs)
    X = workloads.activations(n, d, seed=21, kind="heavy", outlier_frac=2 / 256, outlier_gain=50,
                              as_float=True)
    W = workloads.weights(m, d, seed=22, as_float=True)
    c = cb(d, bits)
    kw, r, _, _ = oracle.fold_weights(W, Pi, c)
    Y, _, _ = oracle.orbq_linear(X, Pi, c, kw, r, c)
    ref = X @ W.T
    err = np.linalg.norm(Y - ref) / np.linalg.norm(ref)
    # distortion of this codebook by Monte Carlo over f_d (independent draws of unit vectors)
    u = np.random.default_rng(9).standard_normal((2000, d))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    q = c.astype(np.float64)[oracle.argmin_codes(u, c)]
    D = np.mean(np.sum((u - q) ** 2, axis=1))
    assert 0.5 * math.sqrt(2 * D) < err < 2.0 * math.sqrt(2 * D), (err, math.sqrt(2 * D))


@pytest.mark.parametrize("bits", [2, 3, 4, 6])
def test_pack_unpack_roundtrip_and_layout(bits):
    rng = np.random.default_rng(bits)
    k = rng.integers(0, 1 << bits, (3, 64))
    p = oracle.pack_codes(k, bits)
    assert p.shape == (3, 64 * bits // 8) and p.dtype == np.uint8
    assert np.array_equal(oracle.unpack_codes(p, bits, 64), k)


def test_packed_layout_hand_example():
    """Hand-written bytes for the documented layout (sign-magnitude, LSB first).
    4-bit, ascending indices [0, 7, 8, 15]: sign-magnitude [15, 8, 0, 7]
    -> bytes 0x8F, 0x70.  2-bit [0, 1, 2, 3] -> [3, 2, 0, 1] -> 0b01_00_10_11 = 0x4B.
    6-bit [0, 31, 32, 63] -> [63, 32, 0, 31] -> 24-bit group
    63 | 32<<6 | 0<<12 | 31<<18 = 0x7C083F -> bytes 0x3F, 0x08, 0x7C."""
    assert list(oracle.pack_codes(np.array([[0, 7, 8, 15]]), 4)[0]) == [0x8F, 0x70]
    assert list(oracle.pack_codes(np.array([[0, 1, 2, 3]]), 2)[0]) == [0x4B]
    assert list(oracle.pack_codes(np.array([[0, 31, 32, 63]]), 6)[0]) == [0x3F, 0x08, 0x7C]
    # 3-bit [0, 3, 4, 7, 1, 2, 5, 6] -> sign-magnitude [7, 4, 0, 3, 6, 5, 1, 2] -> 24-bit group
    # 0b010_001_101_110_011_000_100_111 = 0x46E627 -> bytes 0x27, 0xE6, 0x46
    assert list(oracle.pack_codes(np.array([[0, 3, 4, 7, 1, 2, 5, 6]]), 3)[0]) == [0x27, 0xE6, 0x46]


def test_linear_a16_rotation_cancels(cb):
    """Weights built so that their folded rows are exactly r_j C^[codes_j] (W = W' Pi): the
    weight-only product must reproduce X W^T up to the one bf16 rounding of the rotated
    activations (2^-9 relative per term).  Forgetting the rotation, or rotating by Pi^T, is off
    by O(1)."""
    d, h, bits = 256, 64, 4
    c = cb(d, bits)
    perm, signs = workloads.rotation(d)
    Pi = oracle.rpbh_matrix(d, h, perm, signs)
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16, (9, d))
    r = rng.uniform(0.5, 2.0, 9)
    Wp = oracle.decode_lut_bf16(c)[codes] * r[:, None]
    W = Wp @ Pi
    X = rng.standard_normal((5, d)) * np.exp(rng.standard_normal(d))
    Y = oracle.linear_a16(X, Pi, codes, r, c)
    scale = np.abs(oracle.rotate(X, Pi)) @ np.abs(Wp).T
    err = np.abs(Y - X @ W.T) / scale
    assert err.max() <= 2.0 ** -9 * 1.01
    assert err.max() > 0  # the bf16 rounding is there
    wrong = (oracle.bf16_rne(X) @ Wp.T)  # no rotation
    assert np.max(np.abs(wrong - X @ W.T) / scale) > 0.05
