"""The lower bounds on the threshold that the decode uses to skip work.

n scores at or above a level l give tau >= l - n^-(alpha-1) (their weights
alone would otherwise sum past 1; EntmaxKV summary sec. 2.C, sparse entmax
over the kept tokens). The threshold kernel assembles n per level from
per-item records: an item of 64 scores with maximum M contributes its count
of scores at or above M - 1/32, M - 1/16 or M - 1/8 (the largest of these
levels still at or above l), else 1 when M >= l. These tests rebuild that
rule in plain numpy, in float32 as the kernels do, on clustered, isotropic and
lone-top score sets. They check it against the exact threshold of the float64 oracle
(sort-based), and against a rule that counts a wrong level, which must fail."""
import numpy as np
import pytest

from oracle import entmax

ITEM = 64
ITEM_DELTAS = (np.float32(0.03125), np.float32(0.0625), np.float32(0.125))


def count_pow(n, alpha):
    return float(n) ** (-(alpha - 1.0))


def item_records(x32):
    """Per item: maximum M (float32) and the counts of scores >= M - delta."""
    n_items = -(-len(x32) // ITEM)
    recs = []
    for j in range(n_items):
        it = x32[j * ITEM:(j + 1) * ITEM]
        M = np.float32(it.max())
        cnt = [int(np.count_nonzero(it >= np.float32(M - d))) for d in ITEM_DELTAS]
        recs.append((M, cnt))
    return recs


def level_bound(recs, alpha, levels_from_max, wrong=False):
    """max over levels l = m - f of l - n(l)^-(alpha-1), n(l) from the item
    records by the kernel's rule (wrong=True: an item claims its widest count
    even where that level lies below l)."""
    m = max(M for M, _ in recs)
    best = -np.inf
    for f in levels_from_max:
        lvl = np.float32(m - np.float32(f))
        n = 0
        for M, cnt in recs:
            ls = [np.float32(M - d) for d in ITEM_DELTAS]
            if wrong:
                n += cnt[2] if M >= lvl else 0
            elif ls[2] >= lvl:
                n += cnt[2]
            elif ls[1] >= lvl:
                n += cnt[1]
            elif ls[0] >= lvl:
                n += cnt[0]
            elif M >= lvl:
                n += 1
        if n > 0:
            best = max(best, float(lvl) - count_pow(n, alpha))
    return best


LEVELS8 = (1 / 32, 1 / 16, 1 / 8, 2 / 8, 3 / 8, 4 / 8, 5 / 8, 6 / 8)


def scores(rng, kind, n):
    if kind == "clustered":  # runs of near-equal scores, as clustered keys give
        centres = rng.standard_normal(16)
        runs = rng.integers(0, 16, n // 256 + 1).repeat(256)[:n]
        return centres[runs] * 1.5 + 0.08 * rng.standard_normal(n)
    if kind == "lone_top":  # one score above a dense band lower than m - 1/4 (the case the deep levels serve)
        x = rng.uniform(-0.95, -0.3, n)
        x[rng.integers(n)] = 0.0
        return x
    return rng.standard_normal(n)


@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.3])
@pytest.mark.parametrize("kind", ["clustered", "lone_top", "isotropic"])
def test_item_level_count_bound_below_exact_threshold(alpha, kind):
    rng = np.random.default_rng(7)
    for _ in range(12):
        n = int(rng.integers(64 * 20, 64 * 200))
        x = scores(rng, kind, n)
        x32 = x.astype(np.float32)
        tau = entmax.threshold_sort(x32.astype(np.float64), alpha)
        recs = item_records(x32)
        b8 = level_bound(recs, alpha, LEVELS8)
        assert b8 <= tau + 1e-12, (kind, alpha, b8, tau)
        # the item-maximum bound the few-item path uses is valid too
        m = float(x32.max())
        for f in (1 / 32, 1 / 16, 1 / 8, 1 / 4):
            lvl = np.float32(m - f)
            nm = sum(1 for M, _ in recs if M >= lvl)
            if nm:
                assert float(lvl) - count_pow(nm, alpha) <= tau + 1e-12


def test_deep_levels_tighten_the_bound_on_a_lone_top_score():
    """A lone top score with a dense band below it: the item-maximum bound
    stays at m - 1 or lower, the item-count bound rises well above it."""
    rng = np.random.default_rng(3)
    x32 = scores(rng, "lone_top", 64 * 400).astype(np.float32)
    alpha = 1.5
    tau = entmax.threshold_sort(x32.astype(np.float64), alpha)
    recs = item_records(x32)
    m = float(x32.max())
    b_items = max(float(np.float32(m - f)) - count_pow(sum(1 for M, _ in recs if M >= np.float32(m - f)), alpha)
                  for f in (1 / 32, 1 / 16, 1 / 8, 1 / 4))
    b8 = level_bound(recs, alpha, LEVELS8)
    assert b_items <= m - 1.0 + 1e-9
    assert b8 > m - 0.8
    assert b8 <= tau + 1e-12


def test_wrong_level_rule_is_caught():
    """Crediting an item's widest count at a level it does not reach
    overstates n and can push the bound above the exact threshold."""
    rng = np.random.default_rng(11)
    hit = False
    for _ in range(40):
        x32 = scores(rng, "clustered", 64 * 60).astype(np.float32)
        tau = entmax.threshold_sort(x32.astype(np.float64), 1.5)
        if level_bound(item_records(x32), 1.5, LEVELS8, wrong=True) > tau + 1e-9:
            hit = True
            break
    assert hit
