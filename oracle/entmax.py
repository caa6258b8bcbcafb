"""Exact alpha-entmax in float64 (test infrastructure: see oracle/__init__).

alpha-entmax maps scores to a probability vector with exact zeros for
alpha > 1 (EntmaxKV summary, section 2 "Methodik"; authors' abstract).  The
pages name the mapping but print no formula; the standard definition is used:

    p_j = [ (alpha-1) z_j - tau ]_+ ^ (1/(alpha-1)),   sum_j p_j = 1,

with tau the unique threshold making p sum to one.  Everything here works in
the scaled domain x = (alpha-1) z, where tau lives.

alpha = 2 is sparsemax (Martins & Astudillo 2016), alpha = 1.5 has the exact
sort-based solution of Peters, Niculae & Martins 2019; both follow from the
KKT conditions of the regularised argmax on a candidate support
S = top-k(x): for alpha=2, sum_{S}(x_j - tau) = 1; for alpha=1.5,
sum_{S}(x_j - tau)^2 = 1.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: bf16 is the top half of fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def stored_to_f64(arr: np.ndarray, kv_dtype: str) -> np.ndarray:
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(arr)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def threshold_sort(x: np.ndarray, alpha: float) -> float:
    """Exact tau by sorting (alpha in {1.5, 2}); bisection for other alpha.

    Sort descending: s_1 >= s_2 >= ..., c_k = s_1 + ... + s_k.
      alpha=2:   k* = max{k : s_k > (c_k - 1)/k},          tau = (c_k* - 1)/k*
      alpha=1.5: mu_k = c_k/k, m2_k = (s_1^2+..+s_k^2)/k,
                 D_k = (1 - k (m2_k - mu_k^2))/k, tau_k = mu_k - sqrt(D_k),
                 k* = max{k : D_k >= 0 and tau_k <= s_k},   tau = tau_k*
    """
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        raise ValueError("entmax over an empty set is undefined")
    if alpha == 2.0:
        s = np.sort(x)[::-1]
        c = np.cumsum(s)
        k = np.arange(1, s.size + 1, dtype=np.float64)
        ok = s > (c - 1.0) / k
        kstar = int(np.nonzero(ok)[0][-1]) + 1
        return float((c[kstar - 1] - 1.0) / kstar)
    if alpha == 1.5:
        s = np.sort(x)[::-1]
        # shift by the max for conditioning (entmax is shift-equivariant in tau)
        m = s[0]
        y = s - m
        k = np.arange(1, y.size + 1, dtype=np.float64)
        mu = np.cumsum(y) / k
        m2 = np.cumsum(y * y) / k
        D = (1.0 - k * (m2 - mu * mu)) / k
        tau = mu - np.sqrt(np.maximum(D, 0.0))
        ok = (D >= 0.0) & (tau <= y)
        kstar = int(np.nonzero(ok)[0][-1]) + 1
        return float(tau[kstar - 1] + m)
    return threshold_bisect(x, alpha)


def threshold_bisect(x: np.ndarray, alpha: float, iters: int = 200) -> float:
    """tau by bisection of f(t) = sum_j (x_j - t)_+^(1/(alpha-1)) - 1 on
    [max x - 1, max x - n^(1-alpha)] (f is >= 0 at the left end because the
    top score alone contributes 1, and <= 0 at the right end because every
    one of the n terms is at most 1/n there)."""
    x = np.asarray(x, dtype=np.float64)
    beta = 1.0 / (alpha - 1.0)
    m = float(x.max())
    lo, hi = m - 1.0, m - float(x.size) ** (1.0 - alpha)

    def f(t):
        return float(np.sum(np.maximum(x - t, 0.0) ** beta)) - 1.0

    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        if f(mid) >= 0.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def probs(x: np.ndarray, alpha: float, tau: float | None = None) -> np.ndarray:
    """p_j = [x_j - tau]_+^(1/(alpha-1)); zero exactly where x_j <= tau."""
    x = np.asarray(x, dtype=np.float64)
    if tau is None:
        tau = threshold_sort(x, alpha)
    beta = 1.0 / (alpha - 1.0)
    d = x - tau
    p = np.zeros_like(x)
    pos = d > 0.0
    p[pos] = d[pos] ** beta
    return p
