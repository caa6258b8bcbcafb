"""Brute-force per-page key metadata (test infrastructure: see oracle/__init__).

The EntmaxKV summary (section 2.A) keeps two kinds of lightweight metadata
per KV page: the coordinate-wise minimum and maximum key vectors (k_min,
k_max) and the first and second moments (mean and variance) of the page's
keys.  Readings taken here:
  * the moments are per coordinate (a diagonal model); the variance is the
    population variance of the page's valid tokens;
  * a partial last page holds only its valid tokens (count n_p < P).
Computed directly from the keys, two-pass, in float64; never from any
incrementally maintained state.
"""
from __future__ import annotations

import numpy as np


def page_count(L: int, P: int) -> int:
    return -(-int(L) // int(P))


def page_token_counts(L: int, P: int) -> np.ndarray:
    n = page_count(L, P)
    c = np.full(n, P, dtype=np.int64)
    if n and L % P:
        c[-1] = L % P
    return c


def page_metadata(k: np.ndarray, L: int, P: int) -> dict:
    """k: float64 [>= L][d] keys of one (sequence, KV head).  Returns
    kmin, kmax, mean, var: float64 [n_pages][d]; count: int [n_pages]."""
    k = np.asarray(k, dtype=np.float64)[:L]
    d = k.shape[1]
    n = page_count(L, P)
    kmin = np.empty((n, d))
    kmax = np.empty((n, d))
    mean = np.empty((n, d))
    var = np.empty((n, d))
    count = page_token_counts(L, P)
    for p in range(n):
        blk = k[p * P : p * P + count[p]]
        kmin[p] = blk.min(axis=0)
        kmax[p] = blk.max(axis=0)
        mu = blk.sum(axis=0) / count[p]
        mean[p] = mu
        var[p] = ((blk - mu) ** 2).sum(axis=0) / count[p]
    return {"kmin": kmin, "kmax": kmax, "mean": mean, "var": var, "count": count}
