"""Pins of the truncation analysis the EntmaxKV summary states in sec. 3:
support recovery (kept set contains the support -> exact output) and the
output error bound ||o - o_kept|| <= 2 B delta; plus the reading that the
threshold over a kept subset never exceeds the full one."""
import numpy as np
import pytest

from oracle import decode, entmax


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_support_recovery_and_error_bound(alpha):
    rng = np.random.default_rng(30)
    for _ in range(200):
        n, d = int(rng.integers(2, 120)), 8
        q = rng.standard_normal(d) * 2
        k = rng.standard_normal((n, d))
        v = rng.standard_normal((n, d)) * rng.uniform(0.1, 3)
        allt = np.arange(n)
        full = decode.decode_head(q, k, v, allt, alpha, 0.5)
        B = decode.value_norm_bound(v)
        # random kept subsets
        kept = np.sort(rng.choice(n, int(rng.integers(1, n + 1)), replace=False))
        sub = decode.decode_head(q, k, v, kept, alpha, 0.5)
        delta = decode.dropped_mass(full, kept)
        assert sub["tau"] <= full["tau"] + 1e-12
        assert np.linalg.norm(sub["out"] - full["out"]) <= 2 * B * delta + 1e-10
        # kept superset of the support -> identical result
        sup = np.union1d(full["support"], rng.choice(n, int(rng.integers(0, n)), replace=False))
        sub2 = decode.decode_head(q, k, v, sup, alpha, 0.5)
        assert decode.dropped_mass(full, sup) == 0.0
        assert sub2["tau"] == pytest.approx(full["tau"], abs=1e-12)
        np.testing.assert_allclose(sub2["out"], full["out"], atol=1e-12)


def test_scores_scaling():
    q = np.array([1.0, 2.0])
    k = np.array([[3.0, -1.0]])
    assert decode.scaled_scores(q, k, 1.5, 0.25)[0] == pytest.approx(0.5 * 0.25 * 1.0)


def test_pages_to_tokens_partial_last_page():
    np.testing.assert_array_equal(decode.pages_to_tokens(np.array([0, 2]), 10, 4), [0, 1, 2, 3, 8, 9])
