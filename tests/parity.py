"""GPU-vs-oracle comparison rules (test helper).

Tolerances (the decode-step bar):
  * bounding-box page scores within 1e-6 relative; the top-k set must hold
    every page scoring above U_k + eps and none below U_k - eps, where U_k is
    the oracle's k-th best score and eps = 1e-6 max(1, |U_k|), and its size
    is exactly min(k, n_b);
  * Gaussian tau_hat within 1e-5 max(1, |tau_hat|); keep decisions equal
    outside the band |margin + delta| <= 1e-5 max(1, |tau_hat|) (the page
    moments are float32 on the device);
  * entmax support: equal outside the forward-error band of an fp32 dot
    product, |x_j - tau| <= (alpha-1) scale gamma_d sum_i |q_i k_ji|
    + 1e-6 max(1, |tau|), gamma_d = d u / (1 - d u), u = 2^-24;
  * output max-abs error <= 2e-3, |sum p - 1| <= 1e-5,
    |tau - tau_oracle| <= 1e-5 max(1, |tau|).
"""
from __future__ import annotations

import numpy as np

from oracle import decode, entmax, metadata, scoring, select

U32 = 2.0 ** -24


def kv_f64(arr, kv_dtype):
    return entmax.stored_to_f64(arr, kv_dtype)


class UnitOracle:
    """Oracle view of one selection unit at current length L: a (sequence,
    KV head) whose selection the group's query heads share, or, with
    `head` given, one query head h of KV head g selecting on its own (the
    group rules with a group of one head)."""

    def __init__(self, spec, q_b, keys, vals, L, g, alpha=None, head=None):
        self.spec, self.g, self.L = spec, g, int(L)
        self.alpha = spec.alpha if alpha is None else alpha
        self.G = spec.group
        self.heads = list(range(g * self.G, (g + 1) * self.G)) if head is None else [int(head)]
        self.q = np.asarray(q_b, dtype=np.float64)
        self.k = keys[: self.L]
        self.v = vals[: self.L]
        self.md = metadata.page_metadata(self.k, self.L, spec.page_size)
        self.n_pages = metadata.page_count(self.L, spec.page_size)

    def bbox(self):
        self.S = scoring.bbox_page_scores(self.q[self.heads], self.md["kmin"], self.md["kmax"], self.spec.scale)
        return self.S

    def gauss(self):
        self.mu, self.sd, self.ehat, self.tau_hat = [], [], [], []
        for h in self.heads:
            mu, sd, eh = scoring.gauss_page_stats(self.q[h], self.md["mean"], self.md["var"], self.md["count"],
                                                  self.alpha, self.spec.scale)
            self.mu.append(mu); self.sd.append(sd); self.ehat.append(eh)
            self.tau_hat.append(select.gauss_tau_hat(mu, sd, self.md["count"], self.alpha))
        self.margin = np.max(np.array(self.ehat) - np.array(self.tau_hat)[:, None], axis=0)
        return self.margin

    def decode(self, h, tokens):
        return decode.decode_head(self.q[h], self.k, self.v, tokens, self.alpha, self.spec.scale)


def check_bbox_scores(gpu_S, S):
    err = np.abs(np.asarray(gpu_S, dtype=np.float64) - S)
    lim = 1e-6 * np.maximum(1.0, np.abs(S))
    assert np.all(err <= lim), f"bbox score error {np.max(err / lim):.3g} x tolerance"


def check_topk(gpu_sel, S, k):
    n = S.size
    kk = min(k, n)
    gpu_sel = np.asarray(gpu_sel)
    assert gpu_sel.size == kk, f"selected {gpu_sel.size} pages, expected {kk}"
    assert np.all(np.diff(gpu_sel) > 0), "selection not strictly ascending"
    if kk == n:
        assert np.array_equal(gpu_sel, np.arange(n))
        return
    Uk = np.sort(S)[::-1][kk - 1]
    eps = 1e-6 * max(1.0, abs(Uk))
    must = np.nonzero(S > Uk + eps)[0]
    never = np.nonzero(S < Uk - eps)[0]
    s = set(gpu_sel.tolist())
    assert all(int(p) in s for p in must), "a page clearly above the k-th score is missing"
    assert not any(int(p) in s for p in never), "a page clearly below the k-th score was selected"


def check_tau_hat(gpu_tau_hat, tau_hat):
    for a, b in zip(gpu_tau_hat, tau_hat):
        assert abs(a - b) <= 1e-5 * max(1.0, abs(b)), f"tau_hat {a} vs {b}"


def check_gauss_sel(gpu_sel, margin, delta, tau_hat, min_pages=1):
    """Keep rule max_h(e_hat - tau_hat) > -delta with a floor of
    min(min_pages, n) pages (the largest margins), decisions compared
    outside the band |margin + delta| <= 1e-5 max(1, |tau_hat|) and, for the
    floor, outside the same band around the oracle's m-th margin."""
    gpu_sel = np.asarray(gpu_sel)
    assert np.all(np.diff(gpu_sel) > 0), "selection not strictly ascending"
    band = 1e-5 * max(1.0, max(abs(t) for t in tau_hat))
    m = min(int(min_pages), margin.size)
    s = set(gpu_sel.tolist())
    sure_in = np.nonzero(margin + delta > band)[0]
    maybe_in = np.nonzero(margin + delta >= -band)[0]
    Mm = np.sort(margin)[::-1][m - 1] if m > 0 else np.inf
    if sure_in.size >= m:  # the rule alone decides
        clear_out = np.nonzero(margin + delta < -band)[0]
        assert all(int(p) in s for p in sure_in), "a page clearly above tau_hat - delta is missing"
        assert not any(int(p) in s for p in clear_out), "a page clearly below tau_hat - delta was kept"
        return
    if maybe_in.size < m:  # the floor decides: the m best margins
        assert gpu_sel.size == m, f"floor kept {gpu_sel.size} pages, expected {m}"
        assert all(int(p) in s for p in np.nonzero(margin > Mm + band)[0]), "a page clearly above the floor is missing"
        assert not any(int(p) in s for p in np.nonzero(margin < Mm - band)[0]), "a page clearly below the floor kept"
        return
    # rule and floor meet inside the band: at least m pages, every sure page,
    # nothing clearly below both the rule and the floor
    assert gpu_sel.size >= m
    assert all(int(p) in s for p in sure_in), "a page clearly above tau_hat - delta is missing"
    low = min(-delta, Mm) - band
    assert not any(int(p) in s for p in np.nonzero(margin < low)[0]), "a page clearly below rule and floor kept"


def check_decode(r, q_h, keys, alpha, scale, d, gpu_out, gpu_tau, gpu_psum, gpu_count, gpu_support=None):
    """r: oracle decode_head result over the same token set the GPU used."""
    err = float(np.max(np.abs(np.asarray(gpu_out, dtype=np.float64) - r["out"])))
    assert err <= 2e-3, f"output max-abs error {err}"
    assert abs(float(gpu_psum) - 1.0) <= 1e-5, f"psum {gpu_psum}"
    tau = r["tau"]
    assert abs(float(gpu_tau) - tau) <= 1e-5 * max(1.0, abs(tau)), f"tau {gpu_tau} vs {tau}"
    tokens, x = r["tokens"], r["x"]
    gam = d * U32 / (1 - d * U32)
    absdot = (alpha - 1.0) * scale * (np.abs(keys[tokens]) @ np.abs(np.asarray(q_h, dtype=np.float64)))
    eps = gam * absdot + 1e-6 * max(1.0, abs(tau))
    amb = np.abs(x - tau) <= eps
    sure_in = tokens[(x > tau) & ~amb]
    sure_out = tokens[(x <= tau) & ~amb]
    n_amb = int(np.sum(amb))
    assert len(sure_in) <= int(gpu_count) <= len(sure_in) + n_amb, \
        f"support size {gpu_count} outside [{len(sure_in)}, {len(sure_in) + n_amb}]"
    if gpu_support is not None:
        gs = set(np.asarray(gpu_support).tolist())
        assert all(int(t) in gs for t in sure_in), "a clear support token is missing"
        assert not any(int(t) in gs for t in sure_out), "a clear non-support token is in the support"
    return err
