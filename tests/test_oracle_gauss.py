"""Pins of the oracle's Gaussian-aware selector (EntmaxKV summary sec. 2.B):
expectations against numerical quadrature, the normalisation equation
reducing to the exact entmax threshold when every page has zero variance,
monotonicity, hand-derived values, and the keep rule with its floor."""
import json
import math
import os

import numpy as np
import pytest
from scipy import integrate

from oracle import entmax, select

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_derived.json")))


@pytest.mark.parametrize("case", GOLD["gauss"], ids=lambda c: f"a{c['alpha']}-sd{c['sd']}")
def test_golden(case):
    E = select.gauss_expected_mass(np.array([case["mu"]]), np.array([case["sd"]]), case["t"], case["alpha"])
    assert E[0] == pytest.approx(case["E"], abs=1e-15)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_expectation_vs_quadrature(alpha):
    rng = np.random.default_rng(20)
    beta = 1.0 / (alpha - 1.0)
    for _ in range(40):
        mu, sd, t = rng.normal(0, 2), rng.uniform(0.05, 2.0), rng.normal(0, 2)

        def integrand(y):
            return (y - t) ** beta * math.exp(-0.5 * ((y - mu) / sd) ** 2) / (sd * math.sqrt(2 * math.pi))

        ref, _ = integrate.quad(integrand, t, mu + 40 * sd + abs(t), epsabs=1e-14, epsrel=1e-13, limit=200)
        got = select.gauss_expected_mass(np.array([mu]), np.array([sd]), t, alpha)[0]
        assert got == pytest.approx(ref, abs=1e-10, rel=1e-9)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_zero_variance_reduces_to_exact_tau(alpha):
    """All keys of a page identical -> sd = 0 -> F(t) = sum_p n_p (mu_p - t)_+^e,
    which is the exact entmax equation of the token multiset."""
    rng = np.random.default_rng(21)
    for _ in range(40):
        npg = int(rng.integers(1, 30))
        mu = rng.standard_normal(npg) * 2
        cnt = rng.integers(1, 17, npg)
        th = select.gauss_tau_hat(mu, np.zeros(npg), cnt, alpha)
        tokens = np.repeat(mu, cnt)
        assert th == pytest.approx(entmax.threshold_sort(tokens, alpha), abs=1e-10)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_tau_hat_solves_normalisation(alpha):
    rng = np.random.default_rng(22)
    for _ in range(20):
        npg = int(rng.integers(1, 200))
        mu = rng.standard_normal(npg)
        sd = rng.uniform(0.0, 1.0, npg)
        cnt = rng.integers(1, 65, npg)
        th = select.gauss_tau_hat(mu, sd, cnt, alpha)
        F = lambda t: float(np.sum(cnt * select.gauss_expected_mass(mu, sd, t, alpha)))
        assert F(th) == pytest.approx(1.0, abs=1e-9)
        assert F(th - 1e-3) > 1.0 > F(th + 1e-3)
        # larger sd pushes more mass above any threshold -> larger tau_hat
        assert select.gauss_tau_hat(mu, sd * 1.5, cnt, alpha) >= th - 1e-12


def test_keep_rule_and_floor():
    e = np.array([[1.0, 2.0, 0.5, 3.0], [0.0, 0.0, 2.75, 0.0]])
    tau = np.array([2.5, 3.0])
    # margins: max(e0 - 2.5, e1 - 3.0) = [-1.5, -0.5, -0.25, 0.5] (exact in binary)
    np.testing.assert_array_equal(select.gauss_keep_pages(e, tau, 0.75), [1, 2, 3])
    np.testing.assert_array_equal(select.gauss_keep_pages(e, tau, 0.5), [2, 3])  # strict >
    np.testing.assert_array_equal(select.gauss_keep_pages(e, tau, 0.25), [3])
    # nothing kept -> argmax, lowest id on ties
    e2 = np.array([[0.0, 1.0, 1.0]])
    np.testing.assert_array_equal(select.gauss_keep_pages(e2, np.array([10.0]), 0.5), [1])
