"""Exact entmax attention over a token set, and the truncation analysis
(test infrastructure).

EntmaxKV summary section 2.C: once candidate pages are chosen, only their
keys and values are loaded and the alpha-entmax weights are computed over
that reduced set (reading: the threshold is recomputed over the set, not
the full-cache weights truncated).  Section 3: with delta the full-cache
probability mass on dropped tokens and B a bound on the value norms, the
output error is at most 2 B delta, and it is zero when the kept set contains
the support.

Scores: z = scale q.k with scale = 1/sqrt(d); the scaled score is
x = (alpha-1) z.
"""
from __future__ import annotations

import numpy as np

from . import entmax
from .metadata import page_token_counts


def scaled_scores(q: np.ndarray, k: np.ndarray, alpha: float, scale: float) -> np.ndarray:
    """x_j = (alpha-1) * scale * q.k_j, float64."""
    return (alpha - 1.0) * scale * (np.asarray(k, dtype=np.float64) @ np.asarray(q, dtype=np.float64))


def pages_to_tokens(pages: np.ndarray, L: int, P: int) -> np.ndarray:
    """Ascending valid token ids of the given logical pages."""
    cnt = page_token_counts(L, P)
    parts = [np.arange(p * P, p * P + cnt[p]) for p in np.asarray(pages, dtype=np.int64)]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def attend(x: np.ndarray, v: np.ndarray, alpha: float) -> dict:
    """Exact entmax attention: tau, p, output sum_j p_j v_j, support, psum."""
    tau = entmax.threshold_sort(x, alpha)
    p = entmax.probs(x, alpha, tau)
    out = p @ np.asarray(v, dtype=np.float64)
    supp = np.nonzero(p > 0.0)[0]
    return {"tau": tau, "p": p, "out": out, "support": supp, "psum": float(p.sum())}


def decode_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, tokens: np.ndarray,
                alpha: float, scale: float) -> dict:
    """Entmax decode of one query head over the token ids `tokens` (ascending).
    Returned "support" holds token ids, "x" the scaled scores of `tokens`."""
    tokens = np.asarray(tokens, dtype=np.int64)
    x = scaled_scores(q, k[tokens], alpha, scale)
    r = attend(x, v[tokens], alpha)
    r["support"] = tokens[r["support"]]
    r["x"] = x
    r["tokens"] = tokens
    return r


def dropped_mass(full: dict, kept_tokens: np.ndarray) -> float:
    """delta = full-cache entmax mass on tokens outside the kept set."""
    p = full["p"]
    tok = full["tokens"]
    keep = np.isin(tok, np.asarray(kept_tokens, dtype=np.int64))
    return float(p[~keep].sum())


def value_norm_bound(v: np.ndarray) -> float:
    """B = max_j ||v_j||_2."""
    return float(np.sqrt((np.asarray(v, dtype=np.float64) ** 2).sum(axis=1)).max())


def support_retention(full: dict, kept_tokens: np.ndarray) -> float:
    """Fraction of the full-cache support that lies in the kept set."""
    sup = full["support"]
    if sup.size == 0:
        return 1.0
    return float(np.isin(sup, np.asarray(kept_tokens, dtype=np.int64)).mean())
