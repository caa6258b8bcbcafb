"""Pins of the oracle's page metadata, bounding-box bound and top-k against
what the EntmaxKV summary (sec. 2.A/2.B) fixes: the box bound is an upper
bound on every token score of the page (and the tightest one the box allows,
checked against all box vertices), and top-k keeps the k best pages (brute
force over all k-subsets)."""
import itertools
import math
import json
import os

import numpy as np
import pytest

from oracle import metadata, scoring, select

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_derived.json")))


def test_golden_bbox():
    c = GOLD["bbox"][0]
    k = np.array(c["keys"])
    md = metadata.page_metadata(k, len(k), len(k))
    np.testing.assert_array_equal(md["kmin"][0], c["kmin"])
    np.testing.assert_array_equal(md["kmax"][0], c["kmax"])
    U = scoring.bbox_bound(np.array(c["q"]), md["kmin"], md["kmax"], c["scale"])
    assert U[0] == c["bound"]
    np.testing.assert_allclose(k @ np.array(c["q"]), c["token_scores"])


def test_metadata_invariants():
    rng = np.random.default_rng(10)
    for L, P in [(1, 4), (4, 4), (17, 4), (100, 16), (65, 64)]:
        k = rng.standard_normal((L + 3, 5))
        md = metadata.page_metadata(k, L, P)
        n = metadata.page_count(L, P)
        assert md["kmin"].shape == (n, 5) and md["count"].sum() == L
        for p in range(n):
            blk = k[p * P : p * P + md["count"][p]]
            # per-token loop, independent of the vectorised code
            for i in range(5):
                col = [float(blk[t, i]) for t in range(len(blk))]
                assert md["kmin"][p, i] == min(col) and md["kmax"][p, i] == max(col)
                m = sum(col) / len(col)
                assert md["mean"][p, i] == pytest.approx(m, abs=1e-13)
                # E[k^2] - E[k]^2 (a different formula from the two-pass one)
                assert md["var"][p, i] == pytest.approx(sum(c * c for c in col) / len(col) - m * m, abs=1e-12)
        # tokens beyond L must not leak into the last page
        k2 = k.copy()
        k2[L:] = 1e9
        np.testing.assert_array_equal(metadata.page_metadata(k2, L, P)["kmax"], md["kmax"])


def test_bbox_is_upper_bound_and_tight():
    rng = np.random.default_rng(11)
    for _ in range(40):
        d = 4
        P = int(rng.integers(1, 9))
        L = int(rng.integers(1, 40))
        k = rng.standard_normal((L, d)) * rng.uniform(0.2, 3)
        q = rng.standard_normal(d) * 2
        md = metadata.page_metadata(k, L, P)
        U = scoring.bbox_bound(q, md["kmin"], md["kmax"], 0.5)
        for p in range(metadata.page_count(L, P)):
            blk = k[p * P : p * P + md["count"][p]]
            assert np.all(U[p] >= 0.5 * (blk @ q) - 1e-12)
            # tightest: equals the max of q.k over the 2^d vertices of the box
            verts = [np.where(np.array(bits) == 1, md["kmax"][p], md["kmin"][p])
                     for bits in itertools.product([0, 1], repeat=d)]
            assert U[p] == pytest.approx(0.5 * max(float(v @ q) for v in verts), abs=1e-12)
            if md["count"][p] == 1:
                assert U[p] == pytest.approx(0.5 * float(blk[0] @ q), abs=1e-12)


def test_bbox_monotone_under_append():
    rng = np.random.default_rng(12)
    k = rng.standard_normal((16, 6))
    q = rng.standard_normal(6)
    prev = -np.inf
    for L in range(1, 17):
        md = metadata.page_metadata(k, L, 16)
        U = scoring.bbox_bound(q, md["kmin"], md["kmax"], 1.0)[0]
        assert U >= prev
        prev = U


def test_group_score_bounds_every_head():
    rng = np.random.default_rng(13)
    k = rng.standard_normal((64, 8))
    md = metadata.page_metadata(k, 64, 8)
    qg = rng.standard_normal((4, 8))
    S = scoring.bbox_page_scores(qg, md["kmin"], md["kmax"], 0.3)
    Us = [scoring.bbox_bound(qg[h], md["kmin"], md["kmax"], 0.3) for h in range(4)]
    for U in Us:
        assert np.all(S >= U)
    # every page's score is attained by some head of the group
    assert all(any(S[p] == U[p] for U in Us) for p in range(S.size))


def test_topk_brute_force():
    rng = np.random.default_rng(14)
    for _ in range(60):
        n = int(rng.integers(1, 11))
        k = int(rng.integers(1, n + 3))
        S = rng.integers(0, 4, n).astype(float)  # small integers force ties
        got = select.topk_pages(S, k)
        m = min(k, n)
        best = None
        for sub in itertools.combinations(range(n), m):  # lexicographic order
            s = S[list(sub)].sum()
            if best is None or s > best[0]:
                best = (s, sub)
        assert list(got) == list(best[1])
        assert list(got) == sorted(got)


# ------------------------------------------------- Gaussian page model ---
# The summary (sec. 2.A) models a page's token scores as a Gaussian built
# from the page's first and second key moments.  With the diagonal reading,
# the model's mean and variance are exactly the mean and population variance
# of the page's true scaled token scores whenever the keys' covariance is
# diagonal; the pins below build such pages and compare against the token
# scores themselves (computed one product at a time, not through the model).

def _token_scores(q, blk, alpha, scale):
    return [(alpha - 1.0) * scale * sum(float(q[i]) * float(t[i]) for i in range(len(q))) for t in blk]


def test_golden_gauss_page():
    c = GOLD["gauss_page"][0]
    k = np.array(c["keys"])
    md = metadata.page_metadata(k, len(k), len(k))
    mu, sd, eh = scoring.gauss_page_stats(np.array(c["q"]), md["mean"], md["var"], md["count"], c["alpha"],
                                          c["scale"])
    assert mu[0] == pytest.approx(c["mean_y"], abs=1e-15)
    assert sd[0] == pytest.approx(c["sd_y"], abs=1e-15)
    assert eh[0] == pytest.approx(c["e_hat"], abs=1e-15)
    np.testing.assert_allclose(_token_scores(c["q"], k, c["alpha"], c["scale"]), c["token_scores"], atol=1e-15)


@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.3])
def test_gauss_stats_one_token_pages(alpha):
    """A page of one token: the model's mean is that token's scaled score,
    its spread is zero, and the estimated maximum is the score itself."""
    rng = np.random.default_rng(15)
    d, L = 7, 13
    k = rng.standard_normal((L, d)) * 2
    q = rng.standard_normal(d) * 2
    md = metadata.page_metadata(k, L, 1)
    mu, sd, eh = scoring.gauss_page_stats(q, md["mean"], md["var"], md["count"], alpha, 0.3)
    x = _token_scores(q, k, alpha, 0.3)
    np.testing.assert_allclose(mu, x, rtol=0, atol=1e-13)
    assert np.all(sd == 0.0)
    np.testing.assert_allclose(eh, x, rtol=0, atol=1e-13)


@pytest.mark.parametrize("alpha,scale", [(1.5, 0.125), (1.3, 0.37), (2.0, 0.7)])
def test_gauss_stats_match_token_scores_with_diagonal_covariance(alpha, scale):
    """Pages whose keys are a centre plus sign-balanced offsets along the
    coordinate axes (c + a_i e_i and c - a_i e_i), and pages whose keys
    differ in one coordinate only: the key covariance is diagonal, so the
    model's mean_Y and sd_Y^2 equal the mean and population variance of the
    page's exact scores (alpha-1) scale q.k_t.  A dropped (alpha-1), a
    missing square on the scale or on q_i, or a sample variance fails."""
    rng = np.random.default_rng(16)
    d = 6
    for _ in range(25):
        q = rng.standard_normal(d) * 2
        c = rng.standard_normal(d)
        axes = rng.choice(d, size=int(rng.integers(1, d + 1)), replace=False)
        offs = rng.uniform(0.2, 2.0, axes.size)
        balanced = [c + a * np.eye(d)[i] for i, a in zip(axes, offs)] + [c - a * np.eye(d)[i]
                                                                         for i, a in zip(axes, offs)]
        j = int(rng.integers(d))
        one_coord = [c + s * np.eye(d)[j] for s in rng.standard_normal(int(rng.integers(2, 9))) * 1.5]
        for blk in (np.array(balanced), np.array(one_coord)):
            n = len(blk)
            md = metadata.page_metadata(blk, n, n)
            mu, sd, eh = scoring.gauss_page_stats(q, md["mean"], md["var"], md["count"], alpha, scale)
            x = _token_scores(q, blk, alpha, scale)
            m = sum(x) / n
            var = sum((v - m) ** 2 for v in x) / n
            assert mu[0] == pytest.approx(m, abs=1e-12)
            assert sd[0] ** 2 == pytest.approx(var, abs=1e-12, rel=1e-12)
            assert eh[0] == pytest.approx(m + math.sqrt(var) * math.sqrt(2 * math.log(n)), abs=1e-12)
