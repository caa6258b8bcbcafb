"""GPU parity of the per-query-head selection mode against the float64
oracle.  The EntmaxKV summary does not say how the query heads of a
grouped-query KV head share a page selection; besides the shared selection
(the group maximum of the box bound, the union of the Gaussian keep sets)
the library offers one selection per query head, which the oracle defines as
the group rules with a group of one head."""
import numpy as np
import pytest

import workloads as W
from gpu_common import check_step, run_step
from oracle import decode as odecode
from oracle import softmax as osoft
from parity import UnitOracle, kv_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _session(spec):
    from workloads.upload import build_session
    print(f"[case] per-head {spec.name} B={spec.batch} Hq={spec.n_q_heads} Hkv={spec.n_kv_heads} "
          f"P={spec.page_size} kv={spec.kv_dtype} policy={spec.policy}", flush=True)
    return build_session(spec)


def _q_units(spec):
    return [(b, h) for b in range(spec.batch) for h in range(spec.n_q_heads)]


@pytest.mark.parametrize("hq,hkv,kv", [(8, 2, "bf16"), (16, 2, "bf16"), (8, 2, "f32")])
def test_bbox_per_head(hq, hkv, kv):
    """Per-head box bounds and top-k (matrix-core scoring for groups of 4,
    vector scoring for groups of 8 and float32 records), then each head's
    decode over its own pages; the shared score is the maximum of the
    group's per-head scores, bit for bit (same products, same sums)."""
    spec = W.make_spec("c2", context=4099, page_size=16, top_k=24, n_q_heads=hq, n_kv_heads=hkv, n_needles=16,
                       kv_dtype=kv)
    sess, _ = _session(spec)
    q = W.queries(spec)
    res = run_step(sess, spec, q, per_head=True)
    assert res["sel"].shape[1] == hq
    check_step(spec, res, q, _q_units(spec), per_head=True)
    shared = run_step(sess, spec, q)
    assert shared["sel"].shape[1] == hkv
    G = spec.group
    n = int(np.ceil(res["lens"][0] / spec.page_size))
    per = res["scores"][0, :, :n].reshape(hkv, G, n)
    assert np.array_equal(shared["scores"][0, :, :n], per.max(axis=1))
    assert sess.device_status() == 0


def test_gauss_per_head_and_union():
    """Per-head threshold estimates and keep sets; the union of a group's
    per-head sets is the shared set wherever no head's decision is within
    the rounding band."""
    spec = W.make_spec("c3", batch=2, context=8192 + 40, n_q_heads=8, n_kv_heads=2)
    sess, _ = _session(spec)
    q = W.queries(spec)
    cache = {}
    res = run_step(sess, spec, q, per_head=True)
    check_step(spec, res, q, _q_units(spec), per_head=True, kv_cache=cache)
    shared = run_step(sess, spec, q)
    G = spec.group
    for b in range(spec.batch):
        L = int(shared["lens"][b])
        for g in range(spec.n_kv_heads):
            keys, vals = cache[(b, g)]
            uo = UnitOracle(spec, q[b], keys, vals, L, g)
            uo.gauss()
            margin_h = np.array(uo.ehat) - np.array(uo.tau_hat)[:, None]  # [G][n]
            if not np.any(margin_h > -spec.delta):
                continue  # the one-page floor applies per head and per group differently
            band = 1e-5 * max(1.0, np.abs(uo.tau_hat).max())
            near = np.any(np.abs(margin_h + spec.delta) <= band, axis=0)
            union = set()
            for h in range(g * G, (g + 1) * G):
                union |= set(res["sel"][b, h, : res["cnt"][b, h]].tolist())
            sh = set(shared["sel"][b, g, : shared["cnt"][b, g]].tolist())
            diff = union ^ sh
            assert all(near[p] for p in diff), f"union of per-head sets differs from the shared set at {sorted(diff)[:8]}"
    assert sess.device_status() == 0


def test_softmax_per_head_pages():
    """Softmax attention over each head's own page list."""
    spec = W.make_spec("c2", context=3001, page_size=16, top_k=20, n_q_heads=8, n_kv_heads=2, n_needles=16)
    sess, _ = _session(spec)
    q = W.queries(spec)
    res = run_step(sess, spec, q, per_head=True)
    out = torch.zeros((1, 8, spec.head_dim), dtype=torch.float32, device=sess.device)
    lse = torch.zeros((1, 8), dtype=torch.float32, device=sess.device)
    sess.decode_softmax(torch.from_numpy(q).to(sess.device), scale=spec.scale, sparse=True, out=out, lse=lse)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    L = int(res["lens"][0])
    for g in range(2):
        keys = kv_f64(W.keys(spec, 0, g), spec.kv_dtype)[:L]
        vals = kv_f64(W.values(spec, 0, g), spec.kv_dtype)[:L]
        for h in range(g * 4, g * 4 + 4):
            toks = odecode.pages_to_tokens(res["sel"][0, h, : res["cnt"][0, h]], L, spec.page_size)
            r = osoft.decode_head(q[0, h], keys, vals, toks, spec.scale)
            assert np.abs(o[0, h] - r["out"]).max() <= 2e-3
            assert abs(l[0, h] - r["lse"]) <= 1e-4 * max(1.0, abs(r["lse"]))
    assert sess.device_status() == 0


def test_per_head_batched_permuted_pages():
    """Several sequences of different lengths on permuted physical pages,
    Gaussian selection per query head, one appended token per step."""
    from workloads.upload import step_tokens
    spec = W.make_spec("c5", batch=3, ctx_lo=700, ctx_hi=2500, steps=3, n_q_heads=8, n_kv_heads=2)
    sess, appended = _session(spec)
    for s in range(spec.steps):
        k1, v1 = step_tokens(spec, appended, s)
        sess.append(k1, v1)
        q = W.queries(spec, s)
        res = run_step(sess, spec, q, per_head=True)
        if s == spec.steps - 1:
            check_step(spec, res, q, _q_units(spec), per_head=True)
    assert sess.device_status() == 0
