"""Candidate page selection (test infrastructure).

EntmaxKV summary section 2.B names two policies:

1. Fixed-budget top-k: keep the k pages with the highest bounding-box upper
   bounds.  Readings: ties go to the lower logical page id; k >= n keeps
   every page; the result is returned in ascending page order.

2. Gaussian-aware entmax selection: estimate the global alpha-entmax
   threshold from the page-level Gaussian statistics by solving an
   approximate normalisation equation for tau_hat, then keep the pages whose
   estimated maximum score exceeds tau_hat minus a safety margin Delta.
   Readings (the pages give no formula):
     * the normalisation equation is the expected total entmax mass under the
       per-page Gaussian score model,
           F(t) = sum_p n_p E[(Y_p - t)_+^(1/(alpha-1))] = 1,
         Y_p ~ N(mean_Y,p, sd_Y,p^2),
       solved per query head;
     * for alpha other than 1.5 and 2 the expectation is the truncated
       normal moment sd^e M_e(u) (a parabolic cylinder function), and the
       estimate is defined for 1 < alpha <= 2, where the left end of the
       bisection bracket follows from Jensen's inequality;
     * Delta is measured in the scaled domain where tau lives;
     * a page is kept for a KV head when any query head of its group keeps
       it: max_h (e_hat[h,p] - tau_hat[h]) > -Delta (strict);
     * if that keeps nothing, the single page maximising that quantity is
       kept (lowest page id on ties), since entmax over an empty set is
       undefined.  More generally, with a floor of m pages, a unit that
       keeps fewer than min(m, n) pages keeps the min(m, n) pages of largest
       margin instead (lowest page id on ties); m = 1 is the rule above.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erfc, gamma, pbdv

_INV_SQRT2 = 1.0 / math.sqrt(2.0)
_INV_SQRT2PI = 1.0 / math.sqrt(2.0 * math.pi)


def topk_pages(S: np.ndarray, k: int) -> np.ndarray:
    """Ascending ids of the min(k, n) highest scores, lower id wins ties."""
    S = np.asarray(S, dtype=np.float64)
    n = S.size
    order = np.lexsort((np.arange(n), -S))  # primary key -S, then id
    return np.sort(order[: min(k, n)])


def truncated_normal_moment(u: np.ndarray, beta: float) -> np.ndarray:
    """M_beta(u) = E[Z_+^beta] for Z ~ N(u, 1), beta > -1.

    The integral representation of the parabolic cylinder function (DLMF
    12.5.1 with D_nu = U(-nu - 1/2, .)) gives
        int_0^inf z^beta exp(-z^2/2 + u z) dz = Gamma(beta+1) exp(u^2/4) D_{-beta-1}(-u),
    so M_beta(u) = Gamma(beta+1) exp(-u^2/4) D_{-beta-1}(-u) / sqrt(2 pi).
    For u > 25 that product under/overflows; there P(Z < 0) < 1e-137, so
    M_beta(u) = u^beta E[(1 + W/u)^beta], W ~ N(0, 1), which is smooth in W
    over |W| < u and is taken by 80-point Gauss-Hermite quadrature."""
    u = np.atleast_1d(np.asarray(u, dtype=np.float64))
    out = np.empty_like(u)
    small = u <= 25.0
    if np.any(small):
        d, _ = pbdv(-beta - 1.0, -u[small])
        out[small] = gamma(beta + 1.0) * np.exp(-0.25 * u[small] ** 2) * d / math.sqrt(2.0 * math.pi)
    if np.any(~small):
        x, w = np.polynomial.hermite_e.hermegauss(80)
        w = w / math.sqrt(2.0 * math.pi)
        ub = u[~small][:, None]
        out[~small] = ub[:, 0] ** beta * np.sum(w * (1.0 + x / ub) ** beta, axis=1)
    return out


def gauss_expected_mass(mu: np.ndarray, sd: np.ndarray, t: float, alpha: float) -> np.ndarray:
    """E[(Y - t)_+^(1/(alpha-1))] for Y ~ N(mu, sd^2), per page.

    With u = (mu - t)/sd, Phi(u) = erfc(-u/sqrt 2)/2, phi(u) = exp(-u^2/2)/sqrt(2 pi):
      alpha=2   (exponent 1): (mu - t) Phi(u) + sd phi(u)
      alpha=1.5 (exponent 2): ((mu - t)^2 + sd^2) Phi(u) + (mu - t) sd phi(u)
      any other alpha (exponent e = 1/(alpha-1)): sd^e M_e(u), the truncated
        normal moment above
    and (mu - t)_+^exponent when sd = 0.
    """
    mu = np.asarray(mu, dtype=np.float64)
    sd = np.asarray(sd, dtype=np.float64)
    a = mu - t
    out = np.empty_like(mu)
    z = sd <= 0.0
    nz = ~z
    if alpha == 2.0:
        out[z] = np.maximum(a[z], 0.0)
    elif alpha == 1.5:
        out[z] = np.maximum(a[z], 0.0) ** 2
    else:
        beta = 1.0 / (alpha - 1.0)
        out[z] = np.maximum(a[z], 0.0) ** beta
        if np.any(nz):
            out[nz] = sd[nz] ** beta * truncated_normal_moment(a[nz] / sd[nz], beta)
        return out
    if np.any(nz):
        s = sd[nz]
        u = a[nz] / s
        Phi = 0.5 * erfc(-u * _INV_SQRT2)
        phi = np.exp(-0.5 * u * u) * _INV_SQRT2PI
        if alpha == 2.0:
            out[nz] = a[nz] * Phi + s * phi
        else:
            out[nz] = (a[nz] ** 2 + s * s) * Phi + a[nz] * s * phi
    return out


def gauss_tau_hat(mu: np.ndarray, sd: np.ndarray, count: np.ndarray, alpha: float,
                  iters: int = 200) -> float:
    """Solve F(t) = sum_p n_p E_p(t) = 1 by bisection.

    F is continuous and strictly decreasing where positive.  Left end
    t_lo = max_p mu_p - 1: there F >= 1 for alpha <= 2, because
    E_p(t) >= (mu_p - t)_+^e (Jensen, the integrand is convex in Y for
    e >= 1) and the top page alone gives n_p * 1 >= 1.  Right end: step
    right from t_lo, doubling, until F <= 1.
    """
    if not 1.0 < alpha <= 2.0:
        raise ValueError("the Gaussian threshold estimate needs 1 < alpha <= 2")
    mu = np.asarray(mu, dtype=np.float64)
    sd = np.asarray(sd, dtype=np.float64)
    n = np.asarray(count, dtype=np.float64)

    def F(t):
        return float(np.sum(n * gauss_expected_mass(mu, sd, t, alpha)))

    lo = float(mu.max()) - 1.0
    step = 1.0
    hi = lo + step
    while F(hi) > 1.0:
        step *= 2.0
        hi = lo + step
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        if F(mid) >= 1.0:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def gauss_margin(e_hat: np.ndarray, tau_hat: np.ndarray) -> np.ndarray:
    """max over the group's heads of e_hat[h, p] - tau_hat[h], per page."""
    e_hat = np.asarray(e_hat, dtype=np.float64)
    return np.max(e_hat - np.asarray(tau_hat, dtype=np.float64)[:, None], axis=0)


def gauss_keep_pages(e_hat: np.ndarray, tau_hat: np.ndarray, delta: float, min_pages: int = 1) -> np.ndarray:
    """e_hat: [G][n] estimated maxima of the group's heads, tau_hat: [G].
    Ascending ids of kept pages (at least min(min_pages, n))."""
    margin = gauss_margin(e_hat, tau_hat)
    keep = np.nonzero(margin > -delta)[0]
    m = min(int(min_pages), margin.size)
    if keep.size < m:
        keep = topk_pages(margin, m)  # the m largest margins, lower id first on ties
    return keep
