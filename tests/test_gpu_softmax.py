"""GPU parity of the softmax comparison path and of the entmax support
weights, against the float64 oracle: softmax attention over the selected
pages and over the whole cache (flash-decode split), its log-normaliser, and
the dropped-mass comparison the EntmaxKV summary draws (sec. 1 and 3)."""
import numpy as np
import pytest

import workloads as W
from gpu_common import run_step
from oracle import decode as odecode
from oracle import softmax as osoft
from parity import kv_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _session(spec):
    from workloads.upload import build_session
    print(f"[case] softmax {spec.name} B={spec.batch} Hq={spec.n_q_heads} Hkv={spec.n_kv_heads} "
          f"d={spec.head_dim} P={spec.page_size} ctx={spec.context}", flush=True)
    return build_session(spec)


def _softmax_step(sess, spec, q, sparse):
    out = torch.zeros((spec.batch, spec.n_q_heads, spec.head_dim), dtype=torch.float32, device=sess.device)
    lse = torch.zeros((spec.batch, spec.n_q_heads), dtype=torch.float32, device=sess.device)
    qd = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32)).to(sess.device)
    sess.decode_softmax(qd, scale=spec.scale, sparse=sparse, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _check_softmax(spec, q, units, out, lse, sel=None, cnt=None, lens=None, kv=None):
    for (b, g) in units:
        keys, vals = kv[(b, g)] if kv is not None and (b, g) in kv else (
            kv_f64(W.keys(spec, b, g), spec.kv_dtype), kv_f64(W.values(spec, b, g), spec.kv_dtype))
        if kv is not None:
            kv[(b, g)] = (keys, vals)
        L = int(lens[b])
        if sel is None:
            toks = np.arange(L)
        else:
            toks = odecode.pages_to_tokens(sel[b, g, : cnt[b, g]], L, spec.page_size)
        for h in range(g * spec.group, (g + 1) * spec.group):
            r = osoft.decode_head(q[b, h], keys[:L], vals[:L], toks, spec.scale)
            err = np.abs(out[b, h] - r["out"]).max()
            assert err <= 2e-3, f"softmax output error {err} (b={b}, h={h})"
            assert abs(lse[b, h] - r["lse"]) <= 1e-4 * max(1.0, abs(r["lse"])), f"lse {lse[b, h]} vs {r['lse']}"


@pytest.mark.parametrize("hkv,d", [(2, 128), (8, 128), (4, 64), (1, 128)])
def test_softmax_sparse_and_full(hkv, d):
    """Groups of 4, 1, 2 and 8 query heads (8: two half-group units per KV
    head, each reading the shared page list)."""
    spec = W.make_spec("c2", context=4099, page_size=16, top_k=40, n_q_heads=8, n_kv_heads=hkv, head_dim=d,
                       n_needles=16)
    sess, _ = _session(spec)
    q = W.queries(spec)
    res = run_step(sess, spec, q)  # selection (top-k on the bounding-box bound)
    units = [(0, g) for g in range(hkv)]
    kv = {}
    out, lse = _softmax_step(sess, spec, q, sparse=True)
    _check_softmax(spec, q, units, out, lse, res["sel"], res["cnt"], res["lens"], kv)
    out_f, lse_f = _softmax_step(sess, spec, q, sparse=False)
    _check_softmax(spec, q, units, out_f, lse_f, lens=res["lens"], kv=kv)
    # the kept set loses mass under softmax: lse over the set is below the full one
    assert np.all(lse <= lse_f + 1e-5)
    assert sess.device_status() == 0


def test_softmax_clustered_batch_and_permuted_pages():
    spec = W.make_spec("c5", batch=3, ctx_lo=700, ctx_hi=2500, steps=0, n_q_heads=8, n_kv_heads=2)
    sess, _ = _session(spec)
    q = W.queries(spec)
    res = run_step(sess, spec, q)
    units = [(b, g) for b in range(3) for g in range(2)]
    kv = {}
    out, lse = _softmax_step(sess, spec, q, sparse=True)
    _check_softmax(spec, q, units, out, lse, res["sel"], res["cnt"], res["lens"], kv)
    out_f, lse_f = _softmax_step(sess, spec, q, sparse=False)
    _check_softmax(spec, q, units, out_f, lse_f, lens=res["lens"], kv=kv)


def test_softmax_empty_and_single_token():
    from sparse_long_context_append_amd.runtime import DecodeSession
    import sparse_long_context_append_amd as ekv
    d, P = 128, 16
    table = np.array([[0, 1], [2, 3]], dtype=np.int32)
    sess = DecodeSession(batch=2, n_kv_heads=1, n_q_heads=2, head_dim=d, page_size=P, kv_dtype=ekv.EKV_BF16,
                         n_phys_pages=4, page_table=table, cap=2)
    rng = np.random.default_rng(3)
    k = torch.from_numpy(rng.standard_normal((1, 1, 1, d)).astype(np.float32)).cuda().to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((1, 1, 1, d)).astype(np.float32)).cuda().to(torch.bfloat16)
    sess.append(k, v, seq=1)  # sequence 0 stays empty, sequence 1 holds one token
    q = torch.from_numpy(rng.standard_normal((2, 2, d)).astype(np.float32)).cuda()
    out = torch.full((2, 2, d), 7.0, device="cuda")
    lse = torch.zeros((2, 2), device="cuda")
    sess.decode_softmax(q, scale=d ** -0.5, sparse=False, out=out, lse=lse)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse.cpu().numpy()[0]))
    np.testing.assert_allclose(o[1], np.tile(v[0, 0, 0].float().cpu().numpy(), (2, 1)), atol=1e-6)
    zq = (q[1].cpu().numpy() @ k[0, 0, 0].float().cpu().numpy()) * d ** -0.5
    np.testing.assert_allclose(lse.cpu().numpy()[1], zq, atol=1e-4)


def test_entmax_support_weights_and_dropped_mass():
    """The decode's per-token support weights match the oracle's p; the
    full-cache support lets the dropped mass of a selection be measured, and
    it compares with softmax's as the pages describe."""
    spec = W.make_spec("c2", context=3000, page_size=16, top_k=48, n_q_heads=8, n_kv_heads=2, n_needles=16)
    sess, _ = _session(spec)
    q = W.queries(spec)
    res = run_step(sess, spec, q)
    SC = 4096
    sidx = torch.full((1, 8, SC), -1, dtype=torch.int32, device="cuda")
    sp = torch.zeros((1, 8, SC), dtype=torch.float32, device="cuda")
    qd = torch.from_numpy(q).cuda()
    sess.decode(qd, alpha=spec.alpha, scale=spec.scale, sparse=False, support_idx=sidx, support_p=sp,
                support_cap=SC)
    torch.cuda.synchronize()
    cnt_full = sess.support_count.cpu().numpy()
    ids, ps = sidx.cpu().numpy(), sp.cpu().numpy()
    out_s, lse_s = _softmax_step(sess, spec, q, sparse=True)
    out_f, lse_f = _softmax_step(sess, spec, q, sparse=False)
    L = int(res["lens"][0])
    for g in range(2):
        keys = kv_f64(W.keys(spec, 0, g), spec.kv_dtype)[:L]
        vals = kv_f64(W.values(spec, 0, g), spec.kv_dtype)[:L]
        kept = odecode.pages_to_tokens(res["sel"][0, g, : res["cnt"][0, g]], L, spec.page_size)
        for h in range(g * 4, g * 4 + 4):
            full = odecode.decode_head(q[0, h], keys, vals, np.arange(L), spec.alpha, spec.scale)
            n = int(cnt_full[0, h])
            pf = dict(zip(full["tokens"][full["p"] > 0].tolist(), full["p"][full["p"] > 0].tolist()))
            for t, p in zip(ids[0, h, :n].tolist(), ps[0, h, :n].tolist()):
                assert abs(p - pf.get(t, 0.0)) <= 2e-3
            assert abs(ps[0, h, :n].sum() - 1.0) <= 1e-4
            # dropped mass of the selection, device vs oracle, entmax and softmax
            d_ent = float(ps[0, h, :n][~np.isin(ids[0, h, :n], kept)].sum())
            assert abs(d_ent - odecode.dropped_mass(full, kept)) <= 2e-3
            fs = osoft.decode_head(q[0, h], keys, vals, np.arange(L), spec.scale)
            d_soft = 1.0 - np.exp(lse_s[0, h] - lse_f[0, h])
            assert abs(d_soft - osoft.dropped_mass(fs, kept)) <= 1e-4
            assert d_soft > 0.0
