"""Pins of the oracle's GELU forms (oracle/activation.py) against facts that do not come from
its own formulas: printed standard-normal table values, an independent quadrature of the
normal density, symmetry identities, Taylor coefficients derived by hand, and the tails."""
import math

import numpy as np

import oracle

# Standard normal CDF values as printed in normal tables (e.g. Abramowitz & Stegun, Table 26.1)
PHI_TABLE = {0.5: 0.6914624612740131, 1.0: 0.8413447460685429, 1.959963984540054: 0.975,
             2.0: 0.9772498680518208, 3.0: 0.9986501019683699}


def test_gelu_erf_table_values():
    for x, phi in PHI_TABLE.items():
        assert abs(oracle.gelu_erf(x) - x * phi) <= 1e-15 * max(1.0, x)
        assert abs(oracle.gelu_erf(-x) - (-x) * (1.0 - phi)) <= 1e-15 * max(1.0, x)


def test_gelu_erf_against_density_quadrature():
    """Phi(x) = 1/2 + integral_0^x of the normal density, by composite Simpson (no erf)."""
    for x in (-3.7, -1.3, -0.2, 0.4, 1.1, 2.9):
        t = np.linspace(0.0, x, 20001)
        f = np.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)
        h = x / 20000
        simpson = h / 3.0 * (f[0] + f[-1] + 4.0 * f[1:-1:2].sum() + 2.0 * f[2:-1:2].sum())
        assert abs(oracle.gelu_erf(x) - x * (0.5 + simpson)) < 1e-13


def test_gelu_symmetry_identity():
    """GELU(x) - GELU(-x) = x for both forms (Phi(x) + Phi(-x) = 1; tanh is odd)."""
    x = np.random.default_rng(0).standard_normal(10001) * 4
    for g in (oracle.gelu_erf, oracle.gelu_tanh):
        assert np.max(np.abs(g(x) - g(-x) - x)) < 1e-13
        assert g(0.0) == 0.0


def test_gelu_taylor_coefficients():
    """Near 0: GELU(x) = x/2 + x^2/sqrt(2 pi) + c4 x^4 + O(x^6), with
    c4 = -1/(6 sqrt(2 pi)) for the erf form (Phi's series) and
    c4 = sqrt(2/pi)/2 (0.044715 - 2/(3 pi)) for the tanh form (tanh y = y - y^3/3 + ...)."""
    c = math.sqrt(2.0 / math.pi)
    want = {oracle.gelu_erf: -1.0 / (6.0 * math.sqrt(2.0 * math.pi)),
            oracle.gelu_tanh: 0.5 * c * (0.044715 - 2.0 / (3.0 * math.pi))}
    for g, c4 in want.items():
        for x in (1e-2, -1e-2, 2e-2):
            got = (g(x) - x / 2 - x * x / math.sqrt(2.0 * math.pi)) / x ** 4
            assert abs(got - c4) < 2e-3 * abs(c4) + 1e-6, (g.__name__, x, got, c4)


def test_gelu_tails_and_forms_agree():
    assert abs(oracle.gelu_erf(10.0) - 10.0) < 1e-20
    assert 0.0 > oracle.gelu_erf(-10.0) > -1e-21
    assert abs(oracle.gelu_tanh(10.0) - 10.0) < 1e-20
    assert 0.0 >= oracle.gelu_tanh(-10.0) > -1e-20
    # the tanh form tracks the erf form within 5e-4 everywhere (and is a different function)
    x = np.linspace(-8, 8, 400001)
    d = np.abs(oracle.gelu_tanh(x) - oracle.gelu_erf(x))
    assert 1e-4 < d.max() < 5e-4


def test_lut_gemm_act_is_activation_of_product():
    rng = np.random.default_rng(1)
    c = np.sort(rng.standard_normal(16)) / 40
    xa, xw = rng.integers(0, 16, (5, 64)), rng.integers(0, 16, (7, 64))
    s, r = rng.uniform(10, 40, 5), rng.uniform(0.5, 2, 7)
    Y = oracle.lut_gemm(xa, s, c, xw, r, c)
    assert np.array_equal(oracle.lut_gemm_act(xa, s, c, xw, r, c, "none"), Y)
    # elementwise: a row of outputs equals GELU of that row's products, computed one by one
    G = oracle.lut_gemm_act(xa, s, c, xw, r, c, "gelu_erf")
    for j in range(7):
        y = Y[2, j]
        assert abs(G[2, j] - y * 0.5 * math.erfc(-y / math.sqrt(2.0))) <= 1e-15 * abs(y)
