"""ekv_entmax_decode_noalloc (the decode on the library's fixed device
scratch) against ekv_entmax_decode (the same decode on a caller workspace):
two calls in a row through the C ABI, the second on a smaller input, each
giving the same outputs bit for bit, and the same again after a full-cache
call; plus the oracle bar on the sparse result."""
import numpy as np
import pytest

import workloads as W
from gpu_common import check_step

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(sess, spec, q, sparse):
    """(workspace decode, no-alloc decode) outputs of one step."""
    import sparse_long_context_append_amd as ekv
    SC = 1024
    outs = []
    for noalloc in (False, True):
        o = torch.full_like(sess.out, float("nan"))
        tau = torch.full_like(sess.tau, float("nan"))
        cnt = torch.full_like(sess.support_count, -7)
        ps = torch.full_like(sess.psum, float("nan"))
        sidx = torch.full((spec.batch, spec.n_q_heads, SC), -1, dtype=torch.int32, device="cuda")
        kw = dict(alpha=spec.alpha, scale=spec.scale, sel=sess.sel if sparse else None,
                  sel_count=sess.sel_count if sparse else None, cap=sess.cap if sparse else 0,
                  sel_heads=sess.sel_heads, out=o, tau=tau, support_count=cnt, psum=ps, support_idx=sidx,
                  support_cap=SC)
        if noalloc:
            st = torch.zeros(1, dtype=torch.int32, device="cuda")
            ekv.entmax_decode_noalloc(sess.cache, sess.seqs, q, spec.n_q_heads, dev_status=st, **kw)
        else:
            ekv.entmax_decode(sess.cache, sess.seqs, q, spec.n_q_heads, ws=sess.ws, **kw)
        torch.cuda.synchronize()
        if noalloc:
            assert int(st.item()) == 0
        outs.append({"out": o.cpu().numpy(), "tau": tau.cpu().numpy(), "count": cnt.cpu().numpy(),
                     "psum": ps.cpu().numpy(), "supp": sidx.cpu().numpy()})
    a, b = outs
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    return a


def _case(spec, dense_too):
    from workloads.upload import build_session, queries_device
    print(f"[case] no-alloc {spec.name} B={spec.batch} ctx={spec.context} policy={spec.policy}", flush=True)
    sess, _ = build_session(spec)
    q = queries_device(spec)
    import sparse_long_context_append_amd as ekv
    pol = ekv.EKV_SELECT_BBOX_TOPK if spec.policy == "bbox" else ekv.EKV_SELECT_GAUSS
    sess.select(q, policy=pol, alpha=spec.alpha, scale=spec.scale, top_k=spec.top_k, delta=spec.delta)
    r = _both(sess, spec, q, sparse=True)
    assert np.all(np.abs(r["psum"] - 1.0) <= 1e-5)
    res = dict(r, sel=sess.sel.cpu().numpy(), cnt=sess.sel_count.cpu().numpy(), lens=sess.seq_lens.cpu().numpy(),
               tau_hat=sess.tau_hat.cpu().numpy())
    if spec.policy == "bbox":
        res["scores"] = sess.scores(q, policy=pol, alpha=spec.alpha, scale=spec.scale).cpu().numpy()
    check_step(spec, res, W.queries(spec), [(b, g) for b in range(spec.batch) for g in range(spec.n_kv_heads)])
    if dense_too:
        _both(sess, spec, q, sparse=False)
    assert sess.device_status() == 0


def test_noalloc_matches_workspace_decode_twice():
    # first call: two sequences, bbox top-k; second: one shorter sequence,
    # Gaussian selection (a smaller input on the same scratch)
    _case(W.make_spec("c2", batch=2, context=16 * 300 + 7, n_q_heads=8, n_kv_heads=2, n_needles=8, top_k=24),
          dense_too=True)
    _case(W.make_spec("c3", batch=1, context=32 * 60 + 5, n_q_heads=8, n_kv_heads=2), dense_too=False)


def test_noalloc_rejects_oversized_lists():
    import sparse_long_context_append_amd as ekv
    from sparse_long_context_append_amd.runtime import DecodeSession
    table = np.zeros((1, 4096), dtype=np.int32)  # only the shape matters: nothing is launched
    sess = DecodeSession(batch=1, n_kv_heads=8, n_q_heads=64, head_dim=128, page_size=64,
                         kv_dtype=ekv.EKV_BF16, n_phys_pages=1, page_table=table, cap=4096, full_decode=False)
    q = torch.zeros((1, 64, 128), dtype=torch.float32, device="cuda")
    # the full cache: 64 heads x 4096 items x 1552 bytes, above 64 MiB
    with pytest.raises(ekv.EntmaxKVError) as e:
        ekv.entmax_decode_noalloc(sess.cache, sess.seqs, q, 64, alpha=1.5, scale=0.1, out=sess.out)
    assert e.value.status == ekv.EKV_ERR_WORKSPACE and "scratch" in str(e.value)
