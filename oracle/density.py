"""The marginal f_d of one coordinate of a uniformly random unit vector
(oracle; test infrastructure only).

OrbitQuant summary (picx.dev), "Theoretical Basis", item 1, and the TurboQuant
slides (docswell), "Page. 14":
    f_d(t) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) * (1 - t^2)^((d-3)/2),  t in [-1, 1],
approximately N(0, 1/d) for d >= 64 (summary item 1; slides "Page. 15").

Cell integrals use closed forms (outside the pages, textbook calculus):
  * substituting u = t^2 turns the mass of [0, x] into half the regularised
    incomplete beta function I_{x^2}(1/2, (d-1)/2);
  * the first moment integrates exactly:
        int t (1-t^2)^a dt = -(1-t^2)^(a+1) / (2(a+1)),   a = (d-3)/2.
Everything is evaluated in log space: at d = 12288 the constant and the power
over- and underflow in plain float64.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import betaincc


def _a(d: int) -> float:
    return (d - 3) / 2.0


def log_gamma_ratio_half(x: float) -> float:
    """log(Gamma(x + 1/2) / Gamma(x)) for x > 0.

    For x >= 10 the asymptotic series (outside the pages, textbook)
        1/2 log x - 1/(8x) + 1/(192x^3) - 1/(640x^5) + 17/(14336x^7) - 31/(18432x^9)
    is used; its truncation error is below 1e-14 there, while subtracting two large
    lgamma values would lose ~1e-16 * lgamma(x) (2e-12 at x ~ 4500), an error the Lloyd
    fixed point amplifies by the inverse of its slowest contraction rate.
    """
    if x < 10.0:
        return math.lgamma(x + 0.5) - math.lgamma(x)
    return (0.5 * math.log(x) - 1.0 / (8 * x) + 1.0 / (192 * x ** 3) - 1.0 / (640 * x ** 5)
            + 17.0 / (14336 * x ** 7) - 31.0 / (18432 * x ** 9))


def log_norm_const(d: int) -> float:
    """log(Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)))."""
    return log_gamma_ratio_half((d - 1) / 2.0) - 0.5 * math.log(math.pi)


def log_fd(t, d: int):
    """log f_d(t) for |t| < 1."""
    t = np.asarray(t, dtype=np.float64)
    return log_norm_const(d) + _a(d) * np.log1p(-t * t)


def fd(t, d: int):
    """f_d(t) on [-1, 1] (0 outside)."""
    t = np.asarray(t, dtype=np.float64)
    out = np.zeros_like(t)
    inside = np.abs(t) < 1.0
    out[inside] = np.exp(log_fd(t[inside], d))
    return out


def gaussian_limit_pdf(t, d: int):
    """The N(0, 1/d) density that f_d approaches for large d."""
    t = np.asarray(t, dtype=np.float64)
    return math.sqrt(d / (2 * math.pi)) * np.exp(-0.5 * d * t * t)


def _upper_tail(x, d: int):
    """int_x^1 f_d for 0 <= x <= 1 (= 0.5 * I^c_{x^2}(1/2, a+1))."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * betaincc(0.5, _a(d) + 1.0, np.minimum(x * x, 1.0))


def cell_mass(lo, hi, d: int):
    """int_lo^hi f_d(t) dt for cells that do not straddle 0 (lo < hi)."""
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    pos = lo >= 0.0
    # f_d is even: a cell [lo, hi] with hi <= 0 has the mass of [-hi, -lo].
    a = np.where(pos, lo, -hi)
    b = np.where(pos, hi, -lo)
    if np.any(a < 0.0):
        raise ValueError("cell straddles 0")
    return _upper_tail(a, d) - _upper_tail(b, d)


def cell_moment(lo, hi, d: int):
    """int_lo^hi t f_d(t) dt for cells that do not straddle 0 (lo < hi)."""
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    pos = lo >= 0.0
    a = np.where(pos, lo, -hi)
    b = np.where(pos, hi, -lo)
    if np.any(a < 0.0):
        raise ValueError("cell straddles 0")
    ap1 = _a(d) + 1.0
    la = ap1 * np.log1p(-np.minimum(a * a, 1.0))      # log (1-a^2)^(a+1)
    with np.errstate(divide="ignore"):
        lb = np.where(b >= 1.0, -np.inf, ap1 * np.log1p(-np.minimum(b * b, 1.0)))
    # (1-a^2)^(a+1) - (1-b^2)^(a+1) = e^la * (1 - e^(lb - la)), accurate via expm1
    diff = -np.exp(la) * np.expm1(lb - la)
    m = math.exp(log_norm_const(d)) / (2.0 * ap1) * diff
    return np.where(pos, m, -m)


def mean_abs_t(d: int) -> float:
    """E|t| under f_d in closed form: Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))."""
    return math.exp(-log_gamma_ratio_half(d / 2.0)) / math.sqrt(math.pi)
