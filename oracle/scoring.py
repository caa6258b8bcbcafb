"""Query-aware page scoring from metadata (test infrastructure).

EntmaxKV summary section 2.A: before any key or value of a page is loaded,
the page is scored from its metadata.

Bounding box.  The pages state only that k_min/k_max give a deterministic
upper bound on the best attention score of any token in the page.  Reading:
the tightest such bound, the maximum of the linear function q.k over the box
[k_min, k_max], reached coordinate by coordinate at a vertex:
    U(q, page) = scale * sum_i max(q_i k_min_i, q_i k_max_i).
GQA reading: the KV page is shared by the group's query heads, so the page
score used for selection is the maximum of U over the group (still an upper
bound for every head in the group).

Gaussian model.  The pages state that the first and second moments let the
token scores of a page be approximated as a Gaussian random variable.
Reading (diagonal moments, scaled domain x = (alpha-1) scale q.k):
    mean_Y = (alpha-1) scale q.mu,   var_Y = (alpha-1)^2 scale^2 sum_i q_i^2 var_i,
and the page's estimated maximum score over its n_p tokens is
    e_hat = mean_Y + sd_Y sqrt(2 ln n_p)
(the classical bound on the expected maximum of n standard normals).  The
e_hat constant is "parity unpinned": the pages give no formula for it.
"""
from __future__ import annotations

import numpy as np


def bbox_bound(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray, scale: float) -> np.ndarray:
    """U[p] for one query head: scale * sum_i max(q_i kmin[p,i], q_i kmax[p,i])."""
    q = np.asarray(q, dtype=np.float64)
    return scale * np.maximum(kmin * q, kmax * q).sum(axis=1)


def bbox_page_scores(q_group: np.ndarray, kmin: np.ndarray, kmax: np.ndarray, scale: float) -> np.ndarray:
    """S[p] = max over the group's query heads of U[p]."""
    return np.max(np.stack([bbox_bound(qh, kmin, kmax, scale) for qh in q_group]), axis=0)


def gauss_page_stats(q: np.ndarray, mean: np.ndarray, var: np.ndarray, count: np.ndarray,
                     alpha: float, scale: float):
    """(mean_Y, sd_Y, e_hat) per page for one query head, scaled domain."""
    q = np.asarray(q, dtype=np.float64)
    a1 = alpha - 1.0
    mu_y = a1 * scale * (mean @ q)
    var_y = (a1 * scale) ** 2 * (var @ (q * q))
    sd_y = np.sqrt(np.maximum(var_y, 0.0))
    e_hat = mu_y + sd_y * np.sqrt(2.0 * np.log(np.asarray(count, dtype=np.float64)))
    return mu_y, sd_y, e_hat
