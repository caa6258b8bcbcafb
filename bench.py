#!/usr/bin/env python
"""Decode-step benchmark of the EntmaxKV sparse alpha-entmax path on one GPU.

One step = select_pages + entmax_decode (sparse) over one batch of the
workload; the cache is built beforehand with append_kv.  Before every timed
step the L2 caches and the Infinity Cache are evicted by streaming a read
over 1 GiB, and each step is bracketed by HIP events on the stream the
kernels run on.

Prints ONE JSON line.  `value` is the effective HBM bandwidth of the sparse
step on the million-token workload: algorithmic bytes (page metadata, the
page table, the selected K pages, the V rows of the support, q and the
output) per step over the median step time.  The 128K Gaussian workload, the
dense full-cache entmax decode, HIP-graph replay and the CPU oracle are
reported beside it.
"""
from __future__ import annotations

import os
import sys

_NCPU = len(os.sched_getaffinity(0))
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, str(_NCPU))

import argparse  # noqa: E402
import json  # noqa: E402
import statistics  # noqa: E402
import time  # noqa: E402

import numpy as np  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "sparse entmax decode µs/step and effective HBM GB/s at 128K and 1M context"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- bytes ----
def step_bytes(spec, sel, sel_count, lens, support_union, sparse=True, appends=False):
    """Algorithmic bytes of one step (what the method must move).  With
    appends, each (sequence, KV head) also reads its new K and V row, writes
    it into the cache and reads and writes its page's box and moment rows."""
    P, d, s = spec.page_size, spec.head_dim, spec.elem_bytes
    G = spec.group
    meta_rec = 2 * d * s if spec.policy == "bbox" else 2 * d * 4
    total = 0
    if appends:
        total += spec.batch * spec.n_kv_heads * (4 * d * s + 2 * (2 * d * s) + 2 * (2 * d * 4))
    for b in range(spec.batch):
        L = int(lens[b])
        n_b = -(-L // P)
        for g in range(spec.n_kv_heads):
            if sparse:
                total += n_b * meta_rec                     # page metadata
                total += n_b * 4 / spec.n_kv_heads           # page-table share
                pages = sel[b, g, : int(sel_count[b, g])].astype(np.int64)
                valid = np.minimum(P, L - pages * P)
                total += int(valid.sum()) * d * s            # valid K rows of the selected pages
            else:
                total += L * d * s                           # every K row
                total += n_b * 4 / spec.n_kv_heads
            total += int(support_union[b][g]) * d * s        # V rows of the support union
            total += G * d * 4 * 2                           # q and output
    return float(total)


def support_union_sizes(spec, supp, count):
    """Per (b, g): number of distinct tokens in the group's supports."""
    G = spec.group
    out = []
    for b in range(spec.batch):
        row = []
        for g in range(spec.n_kv_heads):
            toks = set()
            exact = True
            for h in range(g * G, (g + 1) * G):
                c = int(count[b, h])
                if c > supp.shape[2]:
                    exact = False
                    c = supp.shape[2]
                toks.update(supp[b, h, :c].tolist())
            row.append(len(toks) if exact else sum(int(count[b, h]) for h in range(g * G, (g + 1) * G)))
        out.append(row)
    return out


# ---------------------------------------------------------------- timing ---
class Timer:
    """Per-step HIP-event timing on torch's current stream.  Before every
    step the L2 caches and the 256 MB Infinity Cache are evicted by streaming
    a read over a 1 GiB buffer (written once here).  A read leaves only clean
    lines behind; a write-based flush would leave hundreds of MB of dirty
    lines whose write-back the timed step would then pay for."""

    def __init__(self, torch, flush_bytes=1 << 30):
        self.torch = torch
        self.flush = torch.ones(flush_bytes // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.empty((), dtype=torch.float32, device="cuda")

    def evict(self):
        self.torch.sum(self.flush, dim=0, out=self.sink)

    def run(self, fn, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.evict()
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for e0, e1 in ev:
            self.evict()
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = [e0.elapsed_time(e1) for e0, e1 in ev]
        return ms, wall


def score_kernel_ms(sess, spec, q, pol, scores, torch, timer, reps, copies=8):
    """Average duration of one launch of the page-scoring kernel on cold
    data: `copies` copies of the page metadata are scored back to back
    between two events (each copy was last read copies-1 launches earlier,
    more bytes ago than the last-level cache holds), after an eviction.
    Returns ms per launch, one value per repetition."""
    import dataclasses
    import sparse_long_context_append_amd as ekv
    field = "k_box" if pol == ekv.EKV_SELECT_BBOX_TOPK else "k_moments"
    caches = [dataclasses.replace(sess.cache, **{field: getattr(sess.cache, field).clone()}) for _ in range(copies)]

    def launch(c):
        ekv.score_pages(c, sess.seqs, q, spec.n_q_heads, policy=pol, alpha=spec.alpha, scale=spec.scale,
                        scores=scores, ws=sess.ws)

    for c in caches:
        launch(c)
    out = []
    for _ in range(reps):
        timer.evict()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for c in caches:
            launch(c)
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / copies)
    del caches
    return out


def read_ceiling(nbytes, torch, timer, reps=5):
    """Best plain streaming-read rate (GB/s) over a buffer of the step's
    size, after the same eviction as the timed steps: the library's read
    probe at 4, 8 and 16 blocks per compute unit, best of `reps` each."""
    import sparse_long_context_append_amd as ekv
    n = max(16, (int(nbytes) + 15) // 16 * 16)
    buf = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    best = 0.0
    for per_cu in (4, 8, 16):
        for _ in range(reps):
            timer.evict()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            ekv.stream_read(buf, sink, blocks=per_cu * cus)
            e1.record()
            torch.cuda.synchronize()
            best = max(best, n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    return best


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(round(q * (len(xs) - 1))))]


def measure(spec, steps, warmup, torch, timer, do_dense=True, do_graph=True):
    import sparse_long_context_append_amd as ekv
    from workloads.upload import build_session, queries_device
    from workloads.upload import step_tokens
    t0 = time.perf_counter()
    sess, appended = build_session(spec)
    log(f"{spec.name}: cache built in {time.perf_counter() - t0:.1f}s")
    q = queries_device(spec)
    pol = ekv.EKV_SELECT_BBOX_TOPK if spec.policy == "bbox" else ekv.EKV_SELECT_GAUSS
    SC = 4096
    supp = torch.full((spec.batch, spec.n_q_heads, SC), -1, dtype=torch.int32, device="cuda")
    # workloads with decode-time appends (c5): every step first appends one
    # token per sequence (its metadata update is part of the step); the
    # tokens sit on the device beforehand, and after the last one the lengths
    # go back to the prefilled ones (the same tokens are then written again)
    toks = [step_tokens(spec, appended, s) for s in range(spec.steps)]
    lens0 = sess.seq_lens.clone()
    n_app = [0]

    def sparse_step():
        if toks:
            if n_app[0] == len(toks):
                sess.seq_lens.copy_(lens0)
                n_app[0] = 0
            sess.append(*toks[n_app[0]])
            n_app[0] += 1
        sess.select(q, policy=pol, alpha=spec.alpha, scale=spec.scale, top_k=spec.top_k, delta=spec.delta)
        sess.decode(q, alpha=spec.alpha, scale=spec.scale, sparse=True)

    def dense_step():
        sess.decode(q, alpha=spec.alpha, scale=spec.scale, sparse=False)

    scores = torch.empty((spec.batch, spec.n_kv_heads if pol == 0 else spec.n_q_heads, sess.max_pages)
                         + (() if pol == 0 else (4,)), dtype=torch.float32, device="cuda")

    res = {}
    ms, wall = timer.run(sparse_step, steps, warmup)
    res["sparse_ms"] = ms
    res["sparse_wall_s"] = wall
    # diagnostics of the step just timed (same inputs every step)
    sess.decode(q, alpha=spec.alpha, scale=spec.scale, sparse=True, support_idx=supp, support_cap=SC)
    torch.cuda.synchronize()
    cnt = sess.sel_count.cpu().numpy()
    sel = sess.sel.cpu().numpy()
    lens = sess.seq_lens.cpu().numpy()
    sc = sess.support_count.cpu().numpy()
    union = support_union_sizes(spec, supp.cpu().numpy(), sc)
    res["bytes"] = step_bytes(spec, sel, cnt, lens, union, sparse=True, appends=bool(toks))
    res["pages_selected"] = int(cnt.sum())
    res["pages_total"] = int(sum(-(-int(L) // spec.page_size) for L in lens) * spec.n_kv_heads)
    res["support_mean"] = float(sc.mean())
    res["psum_err"] = float(np.abs(sess.psum.cpu().numpy() - 1.0).max())
    sparse_out = sess.out.clone()
    res["score_ms"] = score_kernel_ms(sess, spec, q, pol, scores, torch, timer, reps=max(5, steps // 4))
    npages = res["pages_total"]
    rec = 2 * spec.head_dim * (spec.elem_bytes if pol == 0 else 4)
    # one fp32 score per (page, KV head); Gaussian: (mean, sd) + estimate + float4 stats per (page, query head)
    out_b = 4 if pol == 0 else 28 * spec.group
    res["score_bytes"] = float(npages * (rec + out_b))
    if do_graph and not toks:  # (a captured append would advance the lengths on every replay)
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            sparse_step()  # warm on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            sparse_step()
        ms_g, _ = timer.run(g.replay, steps, warmup)
        res["graph_ms"] = ms_g
        torch.cuda.synchronize()
        # graph replays must give the eager result
        assert torch.equal(sess.out, sparse_out), "graph replay differs from eager"
    if do_dense:
        ms_d, _ = timer.run(dense_step, max(5, steps // 3), 2)
        res["dense_ms"] = ms_d
        sess.decode(q, alpha=spec.alpha, scale=spec.scale, sparse=False, support_idx=supp, support_cap=SC)
        torch.cuda.synchronize()
        sc_d = sess.support_count.cpu().numpy()
        union_d = support_union_sizes(spec, supp.cpu().numpy(), sc_d)
        res["dense_bytes"] = step_bytes(spec, sel, cnt, lens, union_d, sparse=False)
        res["dense_kv_bytes"] = float(sum(int(L) for L in lens) * spec.n_kv_heads * spec.head_dim
                                      * spec.elem_bytes * 2)
    status = sess.device_status()
    assert status == 0, f"device status {status:#x}"
    del sess
    torch.cuda.empty_cache()
    res["read_ceiling_gbs"] = read_ceiling(res["bytes"], torch, timer)
    return res


# ------------------------------------------------------------ CPU oracle ---
def cpu_baseline(spec, units, reps=3, dense_units=()):
    """Time the float64 oracle on the host: its sparse step (page scoring from
    prebuilt metadata, selection, exact entmax over the kept pages) on each
    unit (b, g) in `units`, and its full-cache entmax on `dense_units`.
    Inputs and metadata are prepared outside the timed region, one unit at a
    time.  Returns (sparse seconds summed over units, dense seconds summed
    over dense_units), each unit's time the median of `reps` runs."""
    from oracle import decode as odecode
    from oracle import entmax, metadata, scoring, select

    q = W.queries(spec).astype(np.float64)
    G = spec.group
    lens = W.seq_lens(spec)

    def sparse_pass(b, g, k, v, L, md):
        heads = range(g * G, (g + 1) * G)
        if spec.policy == "bbox":
            S = scoring.bbox_page_scores(q[b, heads], md["kmin"], md["kmax"], spec.scale)
            pages = select.topk_pages(S, spec.top_k)
        else:
            eh, th = [], []
            for h in heads:
                mu, sd, e = scoring.gauss_page_stats(q[b, h], md["mean"], md["var"], md["count"],
                                                     spec.alpha, spec.scale)
                eh.append(e)
                th.append(select.gauss_tau_hat(mu, sd, md["count"], spec.alpha))
            pages = select.gauss_keep_pages(np.array(eh), np.array(th), spec.delta)
        toks = odecode.pages_to_tokens(pages, L, spec.page_size)
        for h in heads:
            odecode.decode_head(q[b, h], k, v, toks, spec.alpha, spec.scale)

    def dense_pass(b, g, k, v, L):
        toks = np.arange(L)
        for h in range(g * G, (g + 1) * G):
            odecode.decode_head(q[b, h], k, v, toks, spec.alpha, spec.scale)

    def timed(fn, n):
        ts = []
        for _ in range(n):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts)

    sparse_s = dense_s = 0.0
    for (b, g) in sorted(set(units) | set(dense_units)):
        k = entmax.stored_to_f64(W.keys(spec, b, g), spec.kv_dtype)
        v = entmax.stored_to_f64(W.values(spec, b, g), spec.kv_dtype)
        L = int(lens[b])
        if (b, g) in units:
            md = metadata.page_metadata(k, L, spec.page_size)
            sparse_s += timed(lambda: sparse_pass(b, g, k, v, L, md), reps)
            del md
        if (b, g) in dense_units:
            dense_s += timed(lambda: dense_pass(b, g, k, v, L), 1)
        del k, v
    return sparse_s, dense_s


# -------------------------------------------------------------------- main -
def summarize(spec, r):
    med = statistics.median(r["sparse_ms"]) * 1e3  # us
    out = {
        "workload": spec.name,
        "us_per_step": round(med, 2),
        "us_p10": round(pct(r["sparse_ms"], 0.1) * 1e3, 2),
        "us_p90": round(pct(r["sparse_ms"], 0.9) * 1e3, 2),
        "bytes_per_step": int(r["bytes"]),
        "effective_gbs": round(r["bytes"] / (med * 1e-6) / 1e9, 1),
        "hbm_fraction": round(r["bytes"] / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "read_ceiling_gbs": round(r["read_ceiling_gbs"], 1),
        "fraction_of_read_ceiling": round(r["bytes"] / (med * 1e-6) / 1e9 / r["read_ceiling_gbs"], 4),
        "pages_selected": r["pages_selected"],
        "pages_total": r["pages_total"],
        "support_mean": round(r["support_mean"], 2),
        "max_abs_psum_error": r["psum_err"],
    }
    if "graph_ms" in r:
        gm = statistics.median(r["graph_ms"]) * 1e3
        out["graph_us_per_step"] = round(gm, 2)
        out["graph_effective_gbs"] = round(r["bytes"] / (gm * 1e-6) / 1e9, 1)
    if "dense_ms" in r:
        dm = statistics.median(r["dense_ms"]) * 1e3
        out["dense_us_per_step"] = round(dm, 2)
        out["dense_bytes_per_step"] = int(r["dense_bytes"])
        out["dense_effective_gbs"] = round(r["dense_bytes"] / (dm * 1e-6) / 1e9, 1)
        out["dense_full_kv_bytes"] = int(r["dense_kv_bytes"])
        out["speedup_vs_dense"] = round(dm / med, 2)
    sm = statistics.mean(r["score_ms"]) * 1e3
    out["score_kernel_us"] = round(sm, 2)
    out["score_kernel_gbs"] = round(r["score_bytes"] / (sm * 1e-6) / 1e9, 1)
    return out


def run_sweep(args, torch, timer):
    """Sparse step and full-cache decode of one sequence (32/8 heads, d=128,
    pages of 64) at contexts 32K..1M: top-k on the bounding-box bound with a
    2% page budget (isotropic keys with needles), and the Gaussian selector
    (clustered keys)."""
    import math
    rows = []
    for name in ("c4", "c4g"):
        for ctx in (1 << 15, 1 << 16, 1 << 17, 1 << 18, 1 << 19, 1 << 20):
            over = {"context": ctx}
            if name == "c4":
                over["top_k"] = math.ceil(0.02 * ctx / 64)
            spec = W.make_spec(name, **over)
            r = measure(spec, args.steps, args.warmup, torch, timer, do_dense=True, do_graph=False)
            s = summarize(spec, r)
            rows.append({"selector": spec.policy, "context": ctx, "top_k": spec.top_k if spec.policy == "bbox" else None,
                         **{k: s[k] for k in ("us_per_step", "us_p10", "us_p90", "bytes_per_step", "effective_gbs",
                                              "pages_selected", "pages_total", "support_mean", "dense_us_per_step",
                                              "speedup_vs_dense")}})
            log(f"sweep {spec.policy} {ctx}: {s['us_per_step']} us, dense {s['dense_us_per_step']} us")
    print(json.dumps({"metric": METRIC, "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "data": "synthetic", "sweep": rows}), flush=True)


def run_selectors(args, torch, timer):
    """Both selectors on the same clustered keys: one sequence of c4g's
    clustered keys (32/8 heads, d=128, pages of 64, alpha 1.5) at contexts
    32K..1M; the Gaussian selector (margin 0.5), and bounding-box top-k with
    a budget of 2% of the pages and with the Gaussian selector's mean kept
    page count per KV head.  Per variant: step time (select + decode), pages
    kept, the full-cache entmax mass outside the kept pages (dropped mass)
    and the share of the full-cache support kept."""
    import math
    import sparse_long_context_append_amd as ekv
    from workloads.upload import build_session, queries_device
    rows = []
    SC = 1 << 14
    for ctx in (1 << 15, 1 << 16, 1 << 17, 1 << 18, 1 << 19, 1 << 20):
        spec = W.make_spec("c4g", context=ctx)
        sess, _ = build_session(spec)
        q = queries_device(spec)
        B, Hq, G = spec.batch, spec.n_q_heads, spec.group
        n_pages = -(-ctx // spec.page_size)
        sidx = torch.full((B, Hq, SC), -1, dtype=torch.int32, device="cuda")
        sp = torch.zeros((B, Hq, SC), dtype=torch.float32, device="cuda")
        dense_ms, _ = timer.run(lambda: sess.decode(q, alpha=spec.alpha, scale=spec.scale, sparse=False), 3, 1)
        sess.decode(q, alpha=spec.alpha, scale=spec.scale, sparse=False, support_idx=sidx, support_p=sp,
                    support_cap=SC)
        torch.cuda.synchronize()
        cnt, ids, ps = sess.support_count.cpu().numpy(), sidx.cpu().numpy(), sp.cpu().numpy()

        def variant(label, policy, k):
            def step():
                sess.select(q, policy=policy, alpha=spec.alpha, scale=spec.scale, top_k=k, delta=spec.delta)
                sess.decode(q, alpha=spec.alpha, scale=spec.scale, sparse=True)
            ms, _ = timer.run(step, args.steps, args.warmup)
            step()
            torch.cuda.synchronize()
            sel, scnt = sess.sel.cpu().numpy(), sess.sel_count.cpu().numpy()
            d_ent, keep = _selection_quality(spec, sel, scnt, False, ids, ps, cnt, SC)
            row = {"context": ctx, "selector": label, "top_k": k if policy == ekv.EKV_SELECT_BBOX_TOPK else None,
                   "us_per_step": round(statistics.median(ms) * 1e3, 2),
                   "pages_per_kv_head_mean": round(float(scnt.mean()), 1), "pages_per_kv_head": n_pages,
                   "dropped_mass_mean": float(d_ent.mean()), "dropped_mass_max": float(d_ent.max()),
                   "support_retention_mean": float(keep.mean()),
                   "heads_with_full_support": int((keep == 1.0).sum()), "heads": int(keep.size),
                   "dense_us": round(statistics.median(dense_ms) * 1e3, 2)}
            log(f"selectors {ctx} {label}: {row['us_per_step']} us, {row['pages_per_kv_head_mean']} pages, "
                f"dropped {row['dropped_mass_mean']:.4f}, retention {row['support_retention_mean']:.3f}")
            return row, scnt
        r_g, scnt_g = variant("gaussian", ekv.EKV_SELECT_GAUSS, 0)
        rows.append(r_g)
        rows.append(variant("topk_2pct", ekv.EKV_SELECT_BBOX_TOPK, math.ceil(0.02 * n_pages))[0])
        rows.append(variant("topk_matched", ekv.EKV_SELECT_BBOX_TOPK, max(1, int(round(float(scnt_g.mean())))))[0])
        del sess
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "bounding-box top-k vs the Gaussian selector on the same clustered keys",
                      "n_gpus": 1, "data": "synthetic", "steps": args.steps, "warmup": args.warmup,
                      "selectors": rows}), flush=True)


def compare_one(spec, args, torch, timer):
    """Entmax and softmax decode over the same selected pages and over the
    whole cache: per query head, the full-cache mass outside the selection
    (entmax: from the full-cache support weights; softmax: 1 - exp(lse_J -
    lse_full)), the share of the entmax support the selection keeps, and the
    relative output error of the selection against the full cache."""
    import sparse_long_context_append_amd as ekv
    from workloads.upload import build_session, queries_device
    sess, _ = build_session(spec)
    q = queries_device(spec)
    pol = ekv.EKV_SELECT_BBOX_TOPK if spec.policy == "bbox" else ekv.EKV_SELECT_GAUSS
    B, Hq, d = spec.batch, spec.n_q_heads, spec.head_dim
    f32 = dict(dtype=torch.float32, device="cuda")
    SC = 1 << 14
    sidx = torch.full((B, Hq, SC), -1, dtype=torch.int32, device="cuda")
    sp = torch.zeros((B, Hq, SC), **f32)
    o_soft_s, o_soft_f = torch.zeros((B, Hq, d), **f32), torch.zeros((B, Hq, d), **f32)
    lse_s, lse_f = torch.zeros((B, Hq), **f32), torch.zeros((B, Hq), **f32)

    def select():
        sess.select(q, policy=pol, alpha=spec.alpha, scale=spec.scale, top_k=spec.top_k, delta=spec.delta)

    select()
    t = {}
    t["entmax_sparse_us"] = statistics.median(timer.run(
        lambda: sess.decode(q, alpha=spec.alpha, scale=spec.scale, sparse=True), args.steps, args.warmup)[0]) * 1e3
    t["entmax_full_us"] = statistics.median(timer.run(
        lambda: sess.decode(q, alpha=spec.alpha, scale=spec.scale, sparse=False), max(3, args.steps // 3), 1)[0]) * 1e3
    t["softmax_sparse_us"] = statistics.median(timer.run(
        lambda: sess.decode_softmax(q, scale=spec.scale, sparse=True, out=o_soft_s, lse=lse_s), args.steps,
        args.warmup)[0]) * 1e3
    t["softmax_full_us"] = statistics.median(timer.run(
        lambda: sess.decode_softmax(q, scale=spec.scale, sparse=False, out=o_soft_f, lse=lse_f),
        max(3, args.steps // 3), 1)[0]) * 1e3
    sess.decode(q, alpha=spec.alpha, scale=spec.scale, sparse=True)
    o_ent_s = sess.out.clone()
    sess.decode(q, alpha=spec.alpha, scale=spec.scale, sparse=False, support_idx=sidx, support_p=sp, support_cap=SC)
    o_ent_f = sess.out.clone()
    torch.cuda.synchronize()
    cnt = sess.support_count.cpu().numpy()
    ids, ps = sidx.cpu().numpy(), sp.cpu().numpy()
    sel, scnt, lens = sess.sel.cpu().numpy(), sess.sel_count.cpu().numpy(), sess.seq_lens.cpu().numpy()
    rel = lambda a, b: (torch.linalg.vector_norm(a - b, dim=-1) / torch.linalg.vector_norm(b, dim=-1)).cpu().numpy()
    err_e, err_s = rel(o_ent_s, o_ent_f), rel(o_soft_s, o_soft_f)
    d_soft = 1.0 - np.exp(lse_s.cpu().numpy().astype(np.float64) - lse_f.cpu().numpy().astype(np.float64))
    d_ent, keep = [], []
    P = spec.page_size
    for b in range(B):
        for g in range(spec.n_kv_heads):
            pages = sel[b, g, : scnt[b, g]].astype(np.int64)
            for h in range(g * spec.group, (g + 1) * spec.group):
                n = min(int(cnt[b, h]), SC)
                tok = ids[b, h, :n].astype(np.int64)
                kept = np.isin(tok // P, pages)
                d_ent.append(float(ps[b, h, :n][~kept].sum()))
                keep.append(float(kept.mean()) if n else 1.0)
    d_ent, keep = np.array(d_ent), np.array(keep)
    pages_frac = float(scnt.sum()) / float(sum(-(-int(L) // P) for L in lens) * spec.n_kv_heads)
    row = {"workload": spec.name, "selector": spec.policy, "alpha": spec.alpha, "pages_kept_frac": round(pages_frac, 4),
           "entmax": {"dropped_mass_mean": float(d_ent.mean()), "dropped_mass_max": float(d_ent.max()),
                      "support_retention_mean": float(keep.mean()),
                      "heads_with_full_support": int((keep == 1.0).sum()), "heads": int(keep.size),
                      "rel_out_err_mean": float(err_e.mean()), "rel_out_err_max": float(err_e.max())},
           "softmax": {"dropped_mass_mean": float(d_soft.mean()), "dropped_mass_max": float(d_soft.max()),
                       "rel_out_err_mean": float(err_s.mean()), "rel_out_err_max": float(err_s.max())},
           **{k: round(v, 2) for k, v in t.items()}}
    del sess
    torch.cuda.empty_cache()
    return row


def run_compare(args, torch, timer):
    rows = []
    for name in ("c2", "c3", "c4"):
        spec = W.make_spec(name)
        rows.append(compare_one(spec, args, torch, timer))
        log(f"compare {name}: entmax dropped {rows[-1]['entmax']['dropped_mass_mean']:.4f}, softmax dropped "
            f"{rows[-1]['softmax']['dropped_mass_mean']:.4f}")
    print(json.dumps({"metric": "entmax vs softmax at the same selected pages", "n_gpus": 1, "data": "synthetic",
                      "steps": args.steps, "warmup": args.warmup, "compare": rows}), flush=True)


def _selection_quality(spec, sel, scnt, per_head, ids, ps, cnt, SC):
    """Per query head: full-cache entmax mass outside the head's page list
    and the share of the full-cache support inside it."""
    P = spec.page_size
    d_ent, keep = [], []
    for b in range(spec.batch):
        for h in range(spec.n_q_heads):
            r = h if per_head else h // spec.group
            pages = sel[b, r, : scnt[b, r]].astype(np.int64)
            n = min(int(cnt[b, h]), SC)
            tok = ids[b, h, :n].astype(np.int64)
            kept = np.isin(tok // P, pages)
            d_ent.append(float(ps[b, h, :n][~kept].sum()))
            keep.append(float(kept.mean()) if n else 1.0)
    return np.array(d_ent), np.array(keep)


def gqa_one(spec, args, torch, timer):
    """Shared (one page set per KV head, used by its query group) against
    per-query-head selection, at the same per-head budget and, for top-k, at
    the same pages read per KV head (k/G per query head)."""
    import sparse_long_context_append_amd as ekv
    from workloads.upload import build_session, queries_device
    sess, _ = build_session(spec)
    q = queries_device(spec)
    pol = ekv.EKV_SELECT_BBOX_TOPK if spec.policy == "bbox" else ekv.EKV_SELECT_GAUSS
    B, Hq, G = spec.batch, spec.n_q_heads, spec.group
    SC = 1 << 14
    sidx = torch.full((B, Hq, SC), -1, dtype=torch.int32, device="cuda")
    sp = torch.zeros((B, Hq, SC), dtype=torch.float32, device="cuda")
    sess.decode(q, alpha=spec.alpha, scale=spec.scale, sparse=False, support_idx=sidx, support_p=sp, support_cap=SC)
    o_full = sess.out.clone()
    torch.cuda.synchronize()
    cnt, ids, ps = sess.support_count.cpu().numpy(), sidx.cpu().numpy(), sp.cpu().numpy()
    variants = [("shared", False, spec.top_k), ("per_head", True, spec.top_k)]
    if spec.policy == "bbox":
        variants.append(("per_head_matched_bytes", True, max(1, spec.top_k // G)))
    page_bytes = spec.page_size * spec.head_dim * (2 if spec.kv_dtype == "bf16" else 4)
    rows = []
    for label, per_head, k in variants:
        def step():
            sess.select(q, policy=pol, alpha=spec.alpha, scale=spec.scale, top_k=k, delta=spec.delta,
                        per_head=per_head)
            sess.decode(q, alpha=spec.alpha, scale=spec.scale, sparse=True)
        ms, _ = timer.run(step, args.steps, args.warmup)
        step()
        torch.cuda.synchronize()
        sel, scnt = sess.sel.cpu().numpy(), sess.sel_count.cpu().numpy()
        d_ent, keep = _selection_quality(spec, sel, scnt, per_head, ids, ps, cnt, SC)
        err = (torch.linalg.vector_norm(sess.out - o_full, dim=-1) / torch.linalg.vector_norm(o_full, dim=-1))
        err = err.cpu().numpy()
        # K pages the gather reads: once per KV head for a shared list, once per query head otherwise
        pages_read = int(scnt.sum())
        distinct = 0
        for b in range(B):
            for g in range(spec.n_kv_heads):
                rr = range(g * G, (g + 1) * G) if per_head else [g]
                distinct += len(set(np.concatenate([sel[b, r, : scnt[b, r]] for r in rr]).tolist()))
        rows.append({"selection": label, "top_k": k if spec.policy == "bbox" else None,
                     "pages_per_query_head_mean": round(float(scnt.mean()), 2),
                     "k_pages_read": pages_read, "k_bytes_read": pages_read * page_bytes,
                     "distinct_pages_per_kv_head_mean": round(distinct / (B * spec.n_kv_heads), 2),
                     "dropped_mass_mean": float(d_ent.mean()), "dropped_mass_max": float(d_ent.max()),
                     "support_retention_mean": float(keep.mean()),
                     "heads_with_full_support": int((keep == 1.0).sum()), "heads": int(keep.size),
                     "rel_out_err_mean": float(err.mean()), "rel_out_err_max": float(err.max()),
                     "step_us": round(statistics.median(ms) * 1e3, 2)})
        log(f"gqa {spec.name} {label}: dropped {rows[-1]['dropped_mass_mean']:.4f}, retention "
            f"{rows[-1]['support_retention_mean']:.4f}, {rows[-1]['step_us']} us")
    del sess
    torch.cuda.empty_cache()
    return {"workload": spec.name, "selector": spec.policy, "alpha": spec.alpha, "group": G, "rows": rows}


def run_gqa(args, torch, timer):
    out = [gqa_one(W.make_spec(name), args, torch, timer) for name in ("c2", "c3", "c4")]
    print(json.dumps({"metric": "shared vs per-query-head page selection under grouped-query attention",
                      "n_gpus": 1, "data": "synthetic", "steps": args.steps, "warmup": args.warmup,
                      "gqa": out}), flush=True)


def run_prefill(args, torch, timer):
    """Bulk prefill: one append_kv call writes a whole sequence (K and V
    rows) and builds its page metadata (box and moments) from scratch.
    Bytes per call: new K and V read, K and V written, box and moment
    records written."""
    import sparse_long_context_append_amd as ekv
    from sparse_long_context_append_amd.runtime import DecodeSession
    rows = []
    for name in ("c4", "c3"):
        spec = W.make_spec(name)
        B, Hkv, d, P = 1, spec.n_kv_heads, spec.head_dim, spec.page_size
        n = spec.context
        n_pages = -(-n // P)
        table = np.arange(n_pages, dtype=np.int32)[None, :]
        sess = DecodeSession(batch=B, n_kv_heads=Hkv, n_q_heads=spec.n_q_heads, head_dim=d, page_size=P,
                             kv_dtype=ekv.EKV_BF16, n_phys_pages=n_pages, page_table=table, cap=1)
        g = torch.Generator(device="cuda").manual_seed(7)
        k_new = torch.randn((B, n, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
        v_new = torch.randn((B, n, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)

        def call():
            sess.seq_lens.zero_()
            ekv.append_kv(sess.cache, sess.seqs, k_new, v_new, n, sess.ws)

        ms, _ = timer.run(call, args.steps, args.warmup)
        med = statistics.median(ms)
        kv_bytes = 2 * B * n * Hkv * d * 2
        meta_bytes = B * n_pages * Hkv * (2 * d * 2 + 2 * d * 4)
        total = 2 * kv_bytes + meta_bytes
        rows.append({"workload": f"{name} prefill: {n} tokens, {Hkv} KV heads, d={d}, page={P}, bf16",
                     "us_per_call": round(med * 1e3, 2), "bytes": total,
                     "gbs": round(total / (med * 1e-3) / 1e9, 1),
                     "hbm_fraction": round(total / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "tokens_per_s": round(B * n / (med * 1e-3), 1)})
        log(f"prefill {name}: {rows[-1]['us_per_call']} us, {rows[-1]['gbs']} GB/s")
        del sess, k_new, v_new
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "bulk prefill: K/V write and page metadata build", "n_gpus": 1,
                      "data": "synthetic", "steps": args.steps, "warmup": args.warmup, "prefill": rows}), flush=True)


def copy_probe(mib):
    """A plain copy kernel of known size: HBM read and write counters of its
    dispatches calibrate the counters of the path's kernels."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "dispatches": 5}), flush=True)


def traffic_from_profile(kernel, workload):
    """HBM bytes per dispatch of `kernel` on `workload` from the committed
    counter summary, if the kernel source it was taken on is unchanged."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.strip().lstrip("-").strip()
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in ("ekv_select.hip", "ekv_common.h", "ekv_kernels.h"):
        h.update(open(os.path.join(ROOT, "sparse_long_context_append_amd", "csrc", f), "rb").read())
    if vals.get("kernel_source_sha256") != h.hexdigest():
        return None
    try:
        return int(float(vals["hbm_bytes_per_dispatch"]))
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c4", help="workload the headline value is measured on")
    ap.add_argument("--also", default="c3,c5,c4g,c2,c1",
                    help="comma-separated workloads reported beside the headline one in the same line ('' for none)")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--context", type=int, default=0, help="override the workload's context (scaling sweeps)")
    ap.add_argument("--alpha", type=float, default=0.0, help="override the workload's entmax alpha")
    ap.add_argument("--q-heads", type=int, default=0,
                    help="override the workload's query-head count (query groups of other sizes)")
    ap.add_argument("--cpu-units", type=int, default=8, help="(sequence, KV head) units the CPU oracle is timed on")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the headline line: context sweep 32K..1M of the top-2%% and Gaussian "
                         "million-token workloads (one JSON line with a 'sweep' list)")
    ap.add_argument("--compare", action="store_true",
                    help="instead of the headline line: entmax vs softmax at the same selected pages (dropped "
                         "mass, support retention, output error, decode times) on c2, c3, c4")
    ap.add_argument("--gqa", action="store_true",
                    help="instead of the headline line: shared vs per-query-head selection (dropped mass, "
                         "support retention, output error, pages read, step time) on c2, c3, c4")
    ap.add_argument("--selectors", action="store_true",
                    help="instead of the headline line: bounding-box top-k (2%% of pages, and the Gaussian "
                         "selector's kept-page count) beside the Gaussian selector on the same clustered "
                         "million-token keys, contexts 32K..1M")
    ap.add_argument("--prefill", action="store_true",
                    help="instead of the headline line: bulk prefill throughput of append_kv (one call per "
                         "sequence: K/V rows and page metadata) at the c4 and c3 shapes")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (counter calibration)")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the decode path is a single-GPU path and no multi-GPU mode exists",
              file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    timer = Timer(torch)
    if args.sweep:
        run_sweep(args, torch, timer)
        return
    if args.compare:
        run_compare(args, torch, timer)
        return
    if args.gqa:
        run_gqa(args, torch, timer)
        return
    if args.prefill:
        run_prefill(args, torch, timer)
        return
    if args.selectors:
        run_selectors(args, torch, timer)
        return
    over = {"context": args.context} if args.context else {}
    if args.q_heads:
        over["n_q_heads"] = args.q_heads
    if args.alpha:
        over["alpha"] = args.alpha
    spec = W.make_spec(args.workload, **over)
    log(f"device {torch.cuda.get_device_name(0)}; workload {spec.name}")
    r = measure(spec, args.steps, args.warmup, torch, timer, not args.no_dense, not args.no_graph)
    main_sum = summarize(spec, r)
    extra = []
    for name in [n for n in args.also.split(",") if n]:
        spec2 = W.make_spec(name)
        r2 = measure(spec2, args.steps, args.warmup, torch, timer, not args.no_dense, not args.no_graph)
        extra.append(summarize(spec2, r2))
        log(f"{name}: {extra[-1]['us_per_step']} us/step")
    cpu = None
    if not args.no_cpu:
        n_units = spec.batch * spec.n_kv_heads
        units = [(b, g) for b in range(spec.batch) for g in range(spec.n_kv_heads)][: args.cpu_units]
        t0 = time.perf_counter()
        dense_units = units[:2]
        sparse_s, dense_s = cpu_baseline(spec, units, dense_units=dense_units)
        log(f"cpu oracle: {time.perf_counter() - t0:.1f}s including input preparation")
        cpu_us = sparse_s / len(units) * n_units * 1e6
        cpu = {
            "value": round(r["bytes"] / (cpu_us * 1e-6) / 1e9, 3),
            "unit": "GB/s",
            "us_per_step": round(cpu_us, 1),
            "dense_us_per_step": round(dense_s / len(dense_units) * n_units * 1e6, 1),
            "cores": int(os.environ.get("OMP_NUM_THREADS", _NCPU)),
            "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": (f"float64 numpy oracle on the host, inputs prepared outside the timing: sparse step "
                       f"({spec.policy} scoring from prebuilt page metadata, selection, exact entmax over the "
                       f"kept pages) on " + (f"all {n_units}" if len(units) == n_units else f"{len(units)} of {n_units}")
                       + f" (sequence, KV head) units of {spec.name}, median of 3 per unit"
                       + ("" if len(units) == n_units else ", scaled to all units")
                       + f"; full-cache entmax on {len(dense_units)} units, scaled"),
        }
    med_us = main_sum["us_per_step"]
    sm_us = main_sum["score_kernel_us"]
    line = {
        "metric": METRIC,
        "value": main_sum["effective_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med_us / 1e3, 5),
        "wall_ms_per_step_incl_flush": round(r["sparse_wall_s"] / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.kv_dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{spec.name}: B={spec.batch}, Hq/Hkv={spec.n_q_heads}/{spec.n_kv_heads}, "
                               f"d={spec.head_dim}, context={spec.context}, page={spec.page_size}, "
                               f"{spec.policy} select, alpha={spec.alpha}",
                   "global_batch": spec.batch, "seq_len": spec.context, "parallelism": "none"},
        "us_per_step": med_us,
        "hbm_fraction": main_sum["hbm_fraction"],
        "read_ceiling_gbs": main_sum["read_ceiling_gbs"],
        "fraction_of_read_ceiling": main_sum["fraction_of_read_ceiling"],
        "detail": main_sum,
        "roofline": {
            "scope": "dominant kernel of the step, per launch (the step-level fraction is hbm_fraction)",
            "bound": "hbm",
            "kernel": "score_bbox" if spec.policy == "bbox" else "score_gauss",
            "achieved": main_sum["score_kernel_gbs"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(main_sum["score_kernel_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profile("score_bbox" if spec.policy == "bbox" else "score_gauss", spec.name),
            "kernel_us": sm_us,
            "algorithmic_bytes": int(r["score_bytes"]),
        },
        "cpu_baseline": cpu,
    }
    if extra:
        line["also"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
