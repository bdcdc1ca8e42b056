"""Pins for oracle/lloyd_max.py.

Codebook definition: OrbitQuant summary (picx.dev) "Theoretical Basis" item 2;
TurboQuant slides (docswell) "Page. 13", "Page. 16" (printed 1- and 2-bit
values), "Page. 11" / "Page. 17" (distortion between the Shannon lower bound
and sqrt(3)*pi/2 * 4^-b).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import integrate
from scipy.stats import norm

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "turboquant_slides_codebook.json")


def _quad(f, lo, hi, d):
    w = 14.0 / math.sqrt(d)
    lo, hi = max(lo, -w), min(hi, w)
    if hi <= lo:
        return 0.0
    return integrate.quad(f, lo, hi, limit=400, epsabs=0, epsrel=1e-13)[0]


@pytest.mark.parametrize("d", [64, 256, 3072, 12288])
def test_one_bit_is_plus_minus_mean_abs(d, cb):
    c = oracle.lloyd_max(d, 1)
    assert abs(c[1] / oracle.mean_abs_t(d) - 1) < 1e-10 and c[0] == -c[1]


def test_printed_slide_values():
    """sqrt(d) * centroids at large d against the values the slides print.

    1 bit: sqrt(2/pi) (printed as a closed form); 2 bits: 0.453 and 1.51 (three
    significant digits, so half a unit in the last printed place is allowed)."""
    g = json.load(open(GOLDEN))
    d = 12288
    c1 = oracle.lloyd_max(d, 1)[1] * math.sqrt(d)
    assert abs(c1 - g["sqrt_d_times_centroids"]["1"][0]) < 1e-4
    c2 = oracle.lloyd_max(d, 2)[2:] * math.sqrt(d)
    for got, want, half_ulp in zip(c2, g["sqrt_d_times_centroids"]["2"], (5e-4, 5e-3)):
        assert abs(got - want) <= half_ulp, (got, want)


@pytest.mark.parametrize("d,bits", [(256, 4), (3072, 2), (3072, 4), (1536, 6), (12288, 4)])
def test_lloyd_conditions(d, bits, cb):
    c = cb(d, bits).astype(np.float64)
    c64 = oracle.lloyd_max(d, bits)
    assert np.array_equal(c64, -c64[::-1])                 # exact antisymmetry
    assert np.all(np.diff(c64) > 0)
    b = 0.5 * (c64[:-1] + c64[1:])
    edges = np.concatenate(([-1.0], b, [1.0]))
    f = lambda t: oracle.fd(np.array([t]), d)[0]
    tf = lambda t: t * oracle.fd(np.array([t]), d)[0]
    # centroid condition, checked by numerical quadrature of f_d itself
    for k in range(len(c64)):
        lo, hi = edges[k], edges[k + 1]
        cond = _quad(tf, lo, hi, d) / _quad(f, lo, hi, d)
        assert abs(cond - c64[k]) * math.sqrt(d) < 1e-9, (k, cond, c64[k])
    # the fp32 codebook is the float64 one rounded
    assert np.array_equal(c, c64.astype(np.float32))


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 6])
def test_distortion_between_shannon_and_turboquant_bounds(bits):
    d = 3072
    c = oracle.lloyd_max(d, bits)
    b = 0.5 * (c[:-1] + c[1:])
    edges = np.concatenate(([-1.0], b, [1.0]))
    D = 0.0
    for k in range(len(c)):
        D += _quad(lambda t, ck=c[k]: (t - ck) ** 2 * oracle.fd(np.array([t]), d)[0],
                   edges[k], edges[k + 1], d)
    D *= d     # distortion of a whole unit vector: d coordinates
    assert 4.0 ** -bits <= D <= math.sqrt(3) * math.pi / 2 * 4.0 ** -bits, D


def _gaussian_lloyd(bits):
    """Lloyd-Max for N(0,1) from the Gaussian closed forms (independent of f_d)."""
    n = 1 << bits
    c = norm.ppf((np.arange(n) + 0.5) / n)
    for _ in range(200000):
        e = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
        new = (norm.pdf(e[:-1]) - norm.pdf(e[1:])) / (norm.cdf(e[1:]) - norm.cdf(e[:-1]))
        new = 0.5 * (new - new[::-1])
        if np.max(np.abs(new - c)) < 1e-14:
            return new
        c = new
    return c


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_approaches_gaussian_lloyd_max(bits):
    g = _gaussian_lloyd(bits)
    gaps = []
    dims = [64, 256, 1536, 3072, 12288]
    for d in dims:
        gaps.append(np.max(np.abs(oracle.lloyd_max(d, bits) * math.sqrt(d) - g)))
    gaps = np.array(gaps)
    assert np.all(np.diff(gaps) < 0)
    scaled = gaps * np.array(dims)
    assert scaled.max() / scaled.min() < 1.6, scaled
