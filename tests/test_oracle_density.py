"""Pins for oracle/density.py (the sphere-coordinate marginal f_d).

f_d: OrbitQuant summary (picx.dev), "Theoretical Basis" item 1; TurboQuant
slides (docswell) "Page. 14" (same formula), "Page. 15" (N(0, 1/d) limit).
"""
import math

import numpy as np
import pytest
from scipy import integrate

import oracle
import oracle.density

DIMS = [64, 256, 1536, 3072, 8960, 12288]


def _quad(f, d, lo=-1.0, hi=1.0):
    # integrate over +-12 sigma where the density lives (it underflows beyond)
    w = 12.0 / math.sqrt(d)
    lo, hi = max(lo, -w), min(hi, w)
    pts = [p for p in (0.0,) if lo < p < hi]
    val, err = integrate.quad(f, lo, hi, points=pts or None, limit=400, epsabs=0, epsrel=1e-13)
    return val


@pytest.mark.parametrize("d", DIMS)
def test_fd_is_a_density_with_variance_one_over_d(d):
    assert abs(_quad(lambda t: oracle.fd(np.array([t]), d)[0], d) - 1.0) < 1e-10
    # sum_i t_i^2 = 1 for a unit vector and the coordinates are exchangeable: E t^2 = 1/d
    assert abs(_quad(lambda t: t * t * oracle.fd(np.array([t]), d)[0], d) * d - 1.0) < 1e-10


@pytest.mark.parametrize("d", DIMS)
def test_mean_abs_closed_form(d):
    by_quad = 2 * _quad(lambda t: t * oracle.fd(np.array([t]), d)[0], d, 0.0, 1.0)
    assert abs(by_quad / oracle.mean_abs_t(d) - 1) < 1e-10
    assert abs(2 * oracle.cell_moment(0.0, 1.0, d) / oracle.mean_abs_t(d) - 1) < 1e-10


def test_small_d_special_cases():
    t = np.linspace(-0.99, 0.99, 41)
    assert np.allclose(oracle.fd(t, 3), 0.5, rtol=1e-14)                    # uniform on [-1, 1]
    assert np.allclose(oracle.fd(t, 4), 2 / math.pi * np.sqrt(1 - t * t), rtol=1e-14)  # semicircle


@pytest.mark.parametrize("d", [256, 3072, 12288])
def test_cell_integrals_match_quadrature(d):
    s = 1 / math.sqrt(d)
    rng = np.random.default_rng(d)
    for _ in range(6):
        lo, hi = np.sort(rng.uniform(0, 5 * s, 2))
        for a, b in ((lo, hi), (-hi, -lo)):
            m = _quad(lambda t: oracle.fd(np.array([t]), d)[0], d, a, b)
            mo = _quad(lambda t: t * oracle.fd(np.array([t]), d)[0], d, a, b)
            assert abs(oracle.cell_mass(a, b, d) / m - 1) < 1e-10
            assert abs(oracle.cell_moment(a, b, d) / mo - 1) < 1e-10


def test_gaussian_limit_approach():
    """sup |f_d - N(0,1/d)| relative to the peak shrinks roughly like 1/d."""
    errs = []
    for d in DIMS:
        t = np.linspace(-6, 6, 4001) / math.sqrt(d)
        g = oracle.gaussian_limit_pdf(t, d)
        errs.append(np.max(np.abs(oracle.fd(t, d) - g)) / g.max())
    errs = np.array(errs)
    assert np.all(np.diff(errs) < 0)
    scaled = errs * np.array(DIMS)
    assert scaled.max() / scaled.min() < 1.5
    assert errs[0] < 0.02            # "approximated by N(0, 1/d)" already at d = 64


@pytest.mark.parametrize("d", [4, 64, 256, 1536, 3072, 8960, 12288])
def test_gamma_ratio_against_exact_rationals(d):
    """log Gamma(d/2) - log Gamma((d-1)/2) for even d = 2m: Gamma(m) / Gamma(m - 1/2)
    = ((m-1)!)^2 4^(m-1) / ((2m-2)! sqrt(pi)), evaluated as an exact rational."""
    from fractions import Fraction
    m = d // 2
    r = Fraction(math.factorial(m - 1) ** 2 * 4 ** (m - 1), math.factorial(2 * m - 2))
    exact = math.log(float(r)) - 0.5 * math.log(math.pi)
    assert abs(oracle.density.log_gamma_ratio_half((d - 1) / 2.0) - exact) < 2e-15
