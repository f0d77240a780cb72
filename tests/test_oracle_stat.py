"""Pins for the oracle's statistical threshold (Spark Transformer article,
section 2.2: Gaussian fit, t = mu + sigma * Phi^-1(1 - s), keep x > t).

Checks: Phi^-1 against mpmath at 40 digits and textbook values; the exact
moments of arithmetic progressions (closed form); special cases (s = 0.5,
sigma = 0, strictness); numpy's own mean/var as a different algorithm; and the
realised keep fraction on Gaussian scores.
"""
import math
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import oracle

mpmath.mp.dps = 40


def _ulps(a, b):
    if a == b:
        return 0
    return abs(a - b) / math.ulp(max(abs(a), abs(b)))


@pytest.mark.parametrize("p", [1e-300, 1e-30, 1e-12, 1e-4, 0.01, 0.02425, 0.075, 0.1, 0.2, 0.3,
                               0.45, 0.5, 0.55, 0.7, 0.8, 0.9, 0.925, 0.97575, 0.99, 0.9999,
                               1 - 1e-12])
def test_normal_quantile_vs_mpmath(p):
    z = oracle.normal_quantile(p)
    # solve ncdf(t) = p at 40 digits (accurate in both tails, unlike 2p - 1)
    exact = float(mpmath.findroot(lambda t: mpmath.ncdf(t) - mpmath.mpf(p), mpmath.mpf(z)))
    assert _ulps(z, exact) <= 4


def test_normal_quantile_textbook_and_symmetry():
    assert oracle.normal_quantile(0.5) == 0.0
    assert abs(oracle.normal_quantile(0.975) - 1.959963984540054) < 4e-16 * 2
    assert abs(oracle.normal_quantile(0.9) - 1.2815515655446004) < 3e-16 * 2
    assert oracle.normal_quantile(0.1) == -oracle.normal_quantile(0.9)


@pytest.mark.parametrize("n", [1, 2, 3, 7, 64, 1001])
def test_moments_arithmetic_progression_closed_form(n):
    # a, a+d, ..., a+(n-1)d: mean a + (n-1)d/2, population variance d^2 (n^2-1)/12
    g = np.random.default_rng(n)
    for _ in range(5):
        a = np.float32(g.integers(0, 2 ** 12)) * np.float32(2.0 ** -7)
        d = np.float32(g.integers(1, 2 ** 8)) * np.float32(2.0 ** -9)
        s = (a + d * np.arange(n, dtype=np.float32)).astype(np.float32)
        assert np.all(s.astype(np.float64) == float(a) + float(d) * np.arange(n))  # exact
        mu, var = oracle.stat_moments(s)
        A, D = Fraction(float(a)), Fraction(float(d))
        assert mu == float(A + D * (n - 1) / 2)
        assert var == float(D * D * (n * n - 1) / 12)


def test_moments_vs_numpy():
    g = np.random.default_rng(7)
    s = np.abs(g.laplace(0, 1, 5000)).astype(np.float32) * np.float32(0.3)
    mu, var = oracle.stat_moments(s)
    s64 = s.astype(np.float64)
    assert _ulps(mu, float(np.mean(s64))) <= 2
    assert _ulps(var, float(np.var(s64))) <= 8


def test_threshold_half_is_mean_and_strict():
    s = np.array([1.0, 2.0, 3.0], np.float32)  # mu = 2; z(0.5) = 0 -> t = 2
    mask, t = oracle.stat_gate(s, 0.5)
    assert t == 2.0 and mask.tolist() == [False, False, True]


def test_threshold_worked_example():
    # scores 1..4: mu = 2.5, sigma^2 = 1.25; s = 0.1 -> z = Phi^-1(0.9)
    s = np.array([1.0, 2.0, 3.0, 4.0], np.float32)
    mu, var = oracle.stat_moments(s)
    assert (mu, var) == (2.5, 1.25)
    t = oracle.stat_threshold(s, 0.1)
    z = float(mpmath.sqrt(2) * mpmath.erfinv(mpmath.mpf(0.8)))
    assert abs(t - (2.5 + math.sqrt(1.25) * z)) < 1e-14
    mask, _ = oracle.stat_gate(s, 0.1)  # t ~ 3.93 -> only 4 kept
    assert mask.tolist() == [False, False, False, True]


def test_threshold_degenerate_constant():
    s = np.full(100, 0.75, np.float32)
    mask, t = oracle.stat_gate(s, 0.1)
    assert t == 0.75 and not mask.any()


@pytest.mark.parametrize("s_keep", [0.1, 0.3, 0.5])
def test_realised_fraction_on_gaussian_scores(s_keep):
    # with c = 1 and x ~ N(10, 1) the scores are Gaussian, so the fitted
    # threshold keeps about a fraction s_keep
    g = np.random.default_rng(11)
    n = 20000
    x = (10.0 + g.standard_normal(n)).astype(np.float32)
    sc = oracle.scores(x, np.ones(n, np.float32))
    mask, _ = oracle.stat_gate(sc, s_keep)
    frac = mask.mean()
    assert abs(frac - s_keep) <= 4 * math.sqrt(s_keep * (1 - s_keep) / n)
