"""Softmax attention over a token set, for the comparison the EntmaxKV pages
draw (test infrastructure: see oracle/__init__).

The summary (sec. 1 and 3) contrasts alpha-entmax with softmax: softmax
gives every token a positive weight, so dropping any token from the kept set
always leaves some output error, while entmax recovers the output exactly
once the kept set holds its support.  At the same kept set, the mass a
method drops is compared.  Here:

    z_j = scale q.k_j,  p_j = exp(z_j - max z) / sum_i exp(z_i - max z),
    lse = log sum_j exp(z_j),  o = sum_j p_j v_j,

and decoding over a kept set J renormalises over J (flash-decode style
attention over the loaded pages).  The mass the full-cache softmax puts
outside J is 1 - exp(lse_J - lse_full).
"""
from __future__ import annotations

import numpy as np


def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """z_j = scale * q.k_j, float64."""
    return scale * (np.asarray(k, dtype=np.float64) @ np.asarray(q, dtype=np.float64))


def attend(z: np.ndarray, v: np.ndarray) -> dict:
    """Softmax attention: p, output, log-normaliser."""
    z = np.asarray(z, dtype=np.float64)
    if z.size == 0:
        raise ValueError("softmax over an empty set is undefined")
    m = float(z.max())
    e = np.exp(z - m)
    s = float(e.sum())
    p = e / s
    return {"p": p, "out": p @ np.asarray(v, dtype=np.float64), "lse": m + float(np.log(s)), "psum": float(p.sum())}


def decode_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, tokens: np.ndarray, scale: float) -> dict:
    """Softmax decode of one query head over the token ids `tokens`."""
    tokens = np.asarray(tokens, dtype=np.int64)
    z = scores(q, k[tokens], scale)
    r = attend(z, v[tokens])
    r["z"] = z
    r["tokens"] = tokens
    return r


def dropped_mass(full: dict, kept_tokens: np.ndarray) -> float:
    """Full-cache softmax mass on tokens outside the kept set."""
    keep = np.isin(full["tokens"], np.asarray(kept_tokens, dtype=np.int64))
    return float(full["p"][~keep].sum())
