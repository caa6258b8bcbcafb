"""Pins of the oracle's exact alpha-entmax against mathematics the pages fix:
the simplex and exact zeros (EntmaxKV summary sec. 2), hand-derived closed
forms (tests/golden/hand_derived.json), two-element closed forms, brute force
over every candidate support, and shift/permutation invariance."""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import entmax

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_derived.json")))


@pytest.mark.parametrize("case", GOLD["entmax"], ids=lambda c: f"a{c['alpha']}-{len(c['x'])}")
def test_golden_hand_derived(case):
    x = np.array(case["x"])
    tau = entmax.threshold_sort(x, case["alpha"])
    assert tau == pytest.approx(case["tau"], abs=1e-14)
    p = entmax.probs(x, case["alpha"], tau)
    np.testing.assert_allclose(p, case["p"], atol=1e-14)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_simplex_and_exact_zeros(alpha):
    rng = np.random.default_rng(1)
    for _ in range(300):
        n = int(rng.integers(1, 200))
        x = rng.standard_normal(n) * rng.uniform(0.1, 5.0)
        tau = entmax.threshold_sort(x, alpha)
        p = entmax.probs(x, alpha, tau)
        assert abs(p.sum() - 1.0) <= 1e-12
        assert np.all(p >= 0.0)
        # KKT: zero exactly where x <= tau, positive where x > tau
        assert np.all((p == 0.0) == (x <= tau))
        # tau lies in [max-1, max - n^(1-alpha)]
        assert x.max() - 1.0 - 1e-12 <= tau <= x.max() - n ** (1.0 - alpha) + 1e-12


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_sort_matches_bisection(alpha):
    rng = np.random.default_rng(2)
    for _ in range(200):
        x = rng.standard_normal(int(rng.integers(1, 300))) * 3
        assert entmax.threshold_sort(x, alpha) == pytest.approx(entmax.threshold_bisect(x, alpha), abs=1e-12)


def test_two_element_closed_forms():
    rng = np.random.default_rng(3)
    for _ in range(500):
        x1, x2 = rng.uniform(-3, 3, 2)
        # alpha=2 (sparsemax): p1 = clip((x1 - x2 + 1)/2, 0, 1)
        p = entmax.probs(np.array([x1, x2]), 2.0)
        assert p[0] == pytest.approx(min(max((x1 - x2 + 1) / 2, 0.0), 1.0), abs=1e-13)
        # alpha=1.5: with D = |x1-x2| < 1, sqrt(p_hi) - sqrt(p_lo) = D, p_hi + p_lo = 1
        p = entmax.probs(np.array([x1, x2]), 1.5)
        D = abs(x1 - x2)
        hi = (1 + D * math.sqrt(2 - D * D)) / 2 if D < 1 else 1.0
        assert max(p) == pytest.approx(hi, abs=1e-12)


def _closed_form_tau(xs, alpha):
    k = len(xs)
    s = float(np.sum(xs))
    if alpha == 2.0:
        return (s - 1.0) / k
    mu = s / k
    disc = mu * mu - (float(np.sum(np.square(xs))) - 1.0) / k
    if disc < 0:
        return None
    return mu - math.sqrt(disc)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_brute_force_over_supports(alpha):
    """Exactly one subset S gives a closed-form tau with x_S > tau >= x_rest,
    and it is the oracle's support."""
    rng = np.random.default_rng(4)
    for _ in range(60):
        n = int(rng.integers(1, 9))
        x = rng.standard_normal(n) * 1.5
        found = []
        for r in range(1, n + 1):
            for S in itertools.combinations(range(n), r):
                t = _closed_form_tau(x[list(S)], alpha)
                if t is None:
                    continue
                rest = [j for j in range(n) if j not in S]
                if np.all(x[list(S)] > t) and np.all(x[rest] <= t):
                    found.append((set(S), t))
        assert len(found) == 1
        p = entmax.probs(x, alpha)
        assert set(np.nonzero(p)[0]) == found[0][0]
        assert entmax.threshold_sort(x, alpha) == pytest.approx(found[0][1], abs=1e-12)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 3.0])
def test_shift_and_permutation(alpha):
    rng = np.random.default_rng(5)
    for _ in range(50):
        x = rng.standard_normal(int(rng.integers(2, 60)))
        p = entmax.probs(x, alpha)
        np.testing.assert_allclose(entmax.probs(x + 7.25, alpha), p, atol=1e-9)
        perm = rng.permutation(x.size)
        np.testing.assert_allclose(entmax.probs(x[perm], alpha), p[perm], atol=1e-9)


@pytest.mark.parametrize("alpha", [1.25, 3.0])
def test_general_alpha_kkt(alpha):
    rng = np.random.default_rng(6)
    for _ in range(50):
        x = rng.standard_normal(int(rng.integers(1, 100)))
        tau = entmax.threshold_sort(x, alpha)
        p = entmax.probs(x, alpha, tau)
        assert abs(p.sum() - 1.0) < 1e-10
        assert np.all((p == 0) == (x <= tau))


def test_bf16_upcast_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F], dtype=np.uint16)
    v = entmax.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -1.0 and v[3] == 0.0
    assert v[2] == 3.140625  # 0x4049 = 1.5703125 * 2
    assert v[5] == pytest.approx(3.3895313892515355e38)


@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.3])
def test_count_bound_on_threshold(alpha):
    """If n scores lie at or above a level l, tau >= l - n^-(alpha-1): those
    scores alone (a subset) already have a threshold at least that high.  The
    decode path filters candidates with this bound."""
    rng = np.random.default_rng(11)
    for trial in range(300):
        n_tok = int(rng.integers(1, 400))
        spread = [0.05, 0.5, 3.0][trial % 3]
        x = rng.standard_normal(n_tok) * spread
        tau = entmax.threshold_sort(x, alpha) if alpha in (1.5, 2.0) else entmax.threshold_bisect(x, alpha)
        m = x.max()
        for c in (0.0, 0.125, 0.25, 0.5, 1.0):
            lvl = m - c
            n = int((x >= lvl).sum())
            assert tau >= lvl - n ** (-(alpha - 1.0)) - 1e-12
