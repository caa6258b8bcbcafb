"""Shared driver for the GPU parity tests: run one decode step of a workload
on the device through the C ABI and compare it with the oracle."""
from __future__ import annotations

import numpy as np

import workloads as W
from oracle import decode as odecode
from parity import UnitOracle, check_bbox_scores, check_decode, check_gauss_sel, check_tau_hat, check_topk, kv_f64

SUPPORT_CAP = 4096


def policy_of(spec):
    import sparse_long_context_append_amd as ekv
    return ekv.EKV_SELECT_BBOX_TOPK if spec.policy == "bbox" else ekv.EKV_SELECT_GAUSS


def run_step(sess, spec, q_np, sparse=True, per_head=False):
    """select (when sparse) + decode on the device; returns host copies.
    per_head: one selection per query head instead of per KV head."""
    import torch
    q = torch.from_numpy(np.ascontiguousarray(q_np, dtype=np.float32)).to(sess.device)
    supp = torch.full((spec.batch, spec.n_q_heads, SUPPORT_CAP), -1, dtype=torch.int32, device=sess.device)
    if sparse:
        sess.select(q, policy=policy_of(spec), alpha=spec.alpha, scale=spec.scale, top_k=spec.top_k,
                    delta=spec.delta, per_head=per_head, min_pages=spec.min_pages)
    sess.decode(q, alpha=spec.alpha, scale=spec.scale, sparse=sparse, support_idx=supp, support_cap=SUPPORT_CAP)
    torch.cuda.synchronize()
    res = {
        "sel": sess.sel.cpu().numpy(), "cnt": sess.sel_count.cpu().numpy(),
        "out": sess.out.cpu().numpy(), "tau": sess.tau.cpu().numpy(), "psum": sess.psum.cpu().numpy(),
        "count": sess.support_count.cpu().numpy(), "supp": supp.cpu().numpy(),
        "tau_hat": sess.tau_hat.cpu().numpy(), "lens": sess.seq_lens.cpu().numpy(),
    }
    if sparse and spec.policy == "bbox":
        res["scores"] = sess.scores(q, policy=policy_of(spec), alpha=spec.alpha, scale=spec.scale,
                                    per_head=per_head).cpu().numpy()
    return res


def check_step(spec, res, q_np, units, sparse=True, kv_cache=None, heads_per_unit=None, per_head=False):
    """Compare a device step with the oracle on the given units: (b, g)
    KV-head units, or (b, h) query-head units when per_head (the selection
    rows of res are then query heads).
    kv_cache: optional dict (b, g) -> (keys_f64, vals_f64) reused across calls."""
    worst = 0.0
    for (b, u) in units:
        g = u // spec.group if per_head else u
        key = (b, g)
        if kv_cache is not None and key in kv_cache:
            keys, vals = kv_cache[key]
        else:
            keys = kv_f64(W.keys(spec, b, g), spec.kv_dtype)
            vals = kv_f64(W.values(spec, b, g), spec.kv_dtype)
            if kv_cache is not None:
                kv_cache[key] = (keys, vals)
        L = int(res["lens"][b])
        uo = UnitOracle(spec, q_np[b], keys, vals, L, g, head=u if per_head else None)
        if sparse:
            gsel = res["sel"][b, u, : res["cnt"][b, u]]
            if spec.policy == "bbox":
                S = uo.bbox()
                check_bbox_scores(res["scores"][b, u, : uo.n_pages], S)
                check_topk(gsel, S, spec.top_k)
            else:
                uo.gauss()
                check_tau_hat(res["tau_hat"][b, uo.heads], uo.tau_hat)
                check_gauss_sel(gsel, uo.margin, spec.delta, uo.tau_hat, spec.min_pages)
            tokens = odecode.pages_to_tokens(gsel, L, spec.page_size)
        else:
            tokens = np.arange(L)
        heads = uo.heads if heads_per_unit is None else uo.heads[:heads_per_unit]
        for h in heads:
            r = uo.decode(h, tokens)
            cnt = int(res["count"][b, h])
            supp = res["supp"][b, h, : min(cnt, SUPPORT_CAP)] if cnt <= SUPPORT_CAP else None
            if supp is not None:
                assert np.all(np.diff(supp) > 0), "support ids not ascending"
            err = check_decode(r, q_np[b, h], keys, spec.alpha, spec.scale, spec.head_dim,
                               res["out"][b, h], res["tau"][b, h], res["psum"][b, h], cnt, supp)
            worst = max(worst, err)
    return worst
