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


# ---- general alpha: the truncated normal moment M_beta(u) = E[Z_+^beta], Z ~ N(u, 1) ----

def _phi(u):
    return math.exp(-0.5 * u * u) / math.sqrt(2 * math.pi)


def _Phi(u):
    return 0.5 * math.erfc(-u / math.sqrt(2))


def test_moment_integer_orders_closed_forms():
    """beta = 1 and 2 have the elementary forms u Phi + phi and
    (u^2 + 1) Phi + u phi; both branches (u <= 25 and above) must give them."""
    for u in [-7.0, -3.2, -0.4, 0.0, 0.9, 4.0, 12.5, 24.9, 25.1, 31.0, 60.0]:
        m1 = select.truncated_normal_moment(np.array([u]), 1.0)[0]
        m2 = select.truncated_normal_moment(np.array([u]), 2.0)[0]
        assert m1 == pytest.approx(u * _Phi(u) + _phi(u), rel=1e-12, abs=1e-300)
        assert m2 == pytest.approx((u * u + 1) * _Phi(u) + u * _phi(u), rel=1e-12, abs=1e-300)


@pytest.mark.parametrize("beta", [1.0 / 0.1, 1.0 / 0.25, 1.0 / 0.3, 1.25, 1.0 / 0.9])
def test_moment_vs_quadrature(beta):
    for u in [-6.5, -2.0, -0.3, 0.0, 1.7, 6.0, 18.0, 24.99, 25.01, 33.0]:
        ref, _ = integrate.quad(lambda z: z ** beta * _phi(z - u), 0.0, max(u, 0.0) + 40.0,
                                points=[max(u, 0.0)], epsabs=0.0, epsrel=1e-13, limit=400)
        got = select.truncated_normal_moment(np.array([u]), beta)[0]
        assert got == pytest.approx(ref, rel=1e-9)


@pytest.mark.parametrize("beta", [1.3, 2.7, 4.25])
def test_moment_recurrence_and_derivative(beta):
    """Integration by parts gives M_{b+1}(u) = u M_b(u) + b M_{b-1}(u), and
    differentiating under the integral d/du M_b = b M_{b-1}: relations
    between three fractional orders that no single closed form checks."""
    M = select.truncated_normal_moment
    for u in [-5.0, -1.5, 0.0, 0.8, 3.0, 10.0, 24.0, 26.0, 40.0]:
        uu = np.array([u])
        lhs = M(uu, beta + 1.0)[0]
        rhs = u * M(uu, beta)[0] + beta * M(uu, beta - 1.0)[0]
        assert lhs == pytest.approx(rhs, rel=1e-10)
        h = 1e-5 * max(1.0, abs(u))
        d = (M(np.array([u + h]), beta)[0] - M(np.array([u - h]), beta)[0]) / (2 * h)
        assert d == pytest.approx(beta * M(uu, beta - 1.0)[0], rel=1e-6)


@pytest.mark.parametrize("alpha", [1.1, 1.25, 1.3, 1.8])
def test_general_alpha_expectation_and_tau_hat(alpha):
    """Per-page expectation against quadrature in the y domain, the zero
    variance limit against the exact entmax threshold, and tau_hat solving
    the normalisation equation."""
    rng = np.random.default_rng(23)
    beta = 1.0 / (alpha - 1.0)
    for _ in range(15):
        mu, sd, t = rng.normal(0, 1), rng.uniform(0.05, 1.5), rng.normal(0, 1)

        def integrand(y):
            return (y - t) ** beta * math.exp(-0.5 * ((y - mu) / sd) ** 2) / (sd * math.sqrt(2 * math.pi))

        ref, _ = integrate.quad(integrand, t, max(mu, t) + 40 * sd, epsabs=0.0, epsrel=1e-12, limit=400)
        got = select.gauss_expected_mass(np.array([mu]), np.array([sd]), t, alpha)[0]
        assert got == pytest.approx(ref, rel=1e-8, abs=1e-300)
    for _ in range(10):
        npg = int(rng.integers(1, 20))
        mu = rng.standard_normal(npg)
        cnt = rng.integers(1, 17, npg)
        th = select.gauss_tau_hat(mu, np.zeros(npg), cnt, alpha)
        assert th == pytest.approx(entmax.threshold_sort(np.repeat(mu, cnt), alpha), abs=1e-9)
        sd = rng.uniform(0.0, 0.8, npg)
        th = select.gauss_tau_hat(mu, sd, cnt, alpha)
        F = lambda t: float(np.sum(cnt * select.gauss_expected_mass(mu, sd, t, alpha)))
        assert F(th) == pytest.approx(1.0, abs=1e-9)
        assert F(th - 1e-3) > 1.0 > F(th + 1e-3)


def test_alpha_limits_of_the_general_branch():
    """The general branch near alpha = 1.5 and 2 approaches the closed forms."""
    mu, sd = np.array([0.4, -0.2, 1.1]), np.array([0.3, 0.7, 0.0])
    for a0 in (1.5, 2.0):
        ref = select.gauss_expected_mass(mu, sd, 0.1, a0)
        near = select.gauss_expected_mass(mu, sd, 0.1, a0 * (1 + 1e-9))
        np.testing.assert_allclose(near, ref, rtol=1e-7)
    with pytest.raises(ValueError):
        select.gauss_tau_hat(mu, sd, np.array([1, 1, 1]), 2.5)


def test_keep_floor_of_several_pages_brute_force():
    """With a floor of m pages: the kept set when it holds at least
    min(m, n) pages, else the min(m, n)-subset of largest margin sum, the
    lexicographically first on ties (brute force over all subsets)."""
    import itertools
    rng = np.random.default_rng(23)
    for _ in range(200):
        n, G = int(rng.integers(1, 9)), int(rng.integers(1, 4))
        e = rng.integers(-4, 3, (G, n)).astype(float) * 0.5  # coarse values force ties
        tau = rng.integers(-2, 3, G).astype(float) * 0.5
        delta, m = 0.5, int(rng.integers(1, n + 3))
        got = select.gauss_keep_pages(e, tau, delta, m)
        margin = np.max(e - tau[:, None], axis=0)
        kept = [p for p in range(n) if margin[p] > -delta]
        mm = min(m, n)
        if len(kept) >= mm:
            assert list(got) == kept
            continue
        best = None
        for sub in itertools.combinations(range(n), mm):
            sc = margin[list(sub)].sum()
            if best is None or sc > best[0]:
                best = (sc, sub)
        assert list(got) == list(best[1])
        assert set(kept) <= set(got.tolist())


def test_keep_floor_hand_case():
    # margins (one head, tau 0): [-1, -3, -0.5, -2]; delta 0.25 keeps nothing
    e = np.array([[-1.0, -3.0, -0.5, -2.0]])
    np.testing.assert_array_equal(select.gauss_keep_pages(e, np.array([0.0]), 0.25, 1), [2])
    np.testing.assert_array_equal(select.gauss_keep_pages(e, np.array([0.0]), 0.25, 2), [0, 2])
    np.testing.assert_array_equal(select.gauss_keep_pages(e, np.array([0.0]), 0.25, 3), [0, 2, 3])
    np.testing.assert_array_equal(select.gauss_keep_pages(e, np.array([0.0]), 0.25, 9), [0, 1, 2, 3])
    # delta 1.5 keeps pages 0 and 2: a floor of 2 changes nothing, 3 adds page 3
    np.testing.assert_array_equal(select.gauss_keep_pages(e, np.array([0.0]), 1.5, 2), [0, 2])
    np.testing.assert_array_equal(select.gauss_keep_pages(e, np.array([0.0]), 1.5, 3), [0, 2, 3])
