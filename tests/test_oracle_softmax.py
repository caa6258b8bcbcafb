"""Pins of the softmax comparison oracle: a library implementation, the
two-token closed form, the alpha -> 1 limit of the entmax oracle, and the
truncation facts the EntmaxKV summary states in sec. 3 (renormalised
attention over a kept set errs by at most 2 B delta; softmax drops positive
mass whenever any token is dropped, entmax none once the support is kept)."""
import numpy as np
import pytest
from scipy.special import logsumexp, softmax as sp_softmax

from oracle import decode, entmax, softmax


def test_matches_library_softmax():
    rng = np.random.default_rng(40)
    for _ in range(50):
        z = rng.standard_normal(int(rng.integers(1, 300))) * rng.uniform(0.1, 20)
        v = rng.standard_normal((z.size, 5))
        r = softmax.attend(z, v)
        np.testing.assert_allclose(r["p"], sp_softmax(z), rtol=1e-12, atol=1e-300)
        assert r["lse"] == pytest.approx(logsumexp(z), abs=1e-12 * max(1.0, abs(logsumexp(z))))
        assert r["psum"] == pytest.approx(1.0, abs=1e-12)
        np.testing.assert_allclose(r["out"], sp_softmax(z) @ v, atol=1e-12)


def test_two_tokens_closed_form_and_shift():
    for a, b in [(0.0, 0.0), (1.0, -2.0), (30.0, 29.5), (-5.0, 7.0)]:
        r = softmax.attend(np.array([a, b]), np.eye(2))
        assert r["p"][0] == pytest.approx(1.0 / (1.0 + np.exp(b - a)), rel=1e-12)
        r2 = softmax.attend(np.array([a + 100.0, b + 100.0]), np.eye(2))
        np.testing.assert_allclose(r["p"], r2["p"], rtol=1e-12)


def test_entmax_tends_to_softmax_as_alpha_to_one():
    """alpha-entmax of z approaches softmax(z) as alpha -> 1 (its scaled
    domain is x = (alpha-1) z, with exponent 1/(alpha-1))."""
    rng = np.random.default_rng(41)
    z = rng.standard_normal(40)
    ps = sp_softmax(z)
    errs = []
    for alpha in (1.01, 1.001):
        x = (alpha - 1.0) * z
        p = entmax.probs(x, alpha, entmax.threshold_bisect(x, alpha))
        errs.append(np.abs(p - ps).max())
    assert errs[1] < errs[0] and errs[1] < 5e-3


def test_truncation_bound_and_dropped_mass():
    rng = np.random.default_rng(42)
    for _ in range(200):
        n, d = int(rng.integers(2, 100)), 6
        q = rng.standard_normal(d) * 2
        k = rng.standard_normal((n, d))
        v = rng.standard_normal((n, d))
        allt = np.arange(n)
        full = softmax.decode_head(q, k, v, allt, 0.5)
        kept = np.sort(rng.choice(n, int(rng.integers(1, n)), replace=False))
        sub = softmax.decode_head(q, k, v, kept, 0.5)
        delta = softmax.dropped_mass(full, kept)
        assert delta > 0.0  # every dropped token had positive weight
        assert delta == pytest.approx(1.0 - np.exp(sub["lse"] - full["lse"]), abs=1e-12)
        B = decode.value_norm_bound(v)
        assert np.linalg.norm(sub["out"] - full["out"]) <= 2 * B * delta + 1e-10
        # entmax on the same kept set drops nothing once it holds the support
        fe = decode.decode_head(q, k, v, allt, 1.5, 0.5)
        kept_e = np.union1d(fe["support"], kept)
        assert decode.dropped_mass(fe, kept_e) == 0.0
        assert decode.support_retention(fe, kept_e) == 1.0
