"""GPU parity at the workloads' full sizes, in the configuration bench.py
times (DecodeSession select + decode on the default stream), checked against
the float64 oracle on sampled (sequence, KV head) units: the oracle rebuilds
the sampled units' metadata, scores, selection, threshold, support and output
from the raw keys one unit at a time.  Every step's probability sums and
device status are checked on all units."""
import numpy as np
import pytest

import workloads as W
from gpu_common import check_step, run_step

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _session(spec):
    from workloads.upload import build_session
    print(f"[case] full-size {spec.name} B={spec.batch} Hq={spec.n_q_heads} Hkv={spec.n_kv_heads} "
          f"P={spec.page_size}", flush=True)
    return build_session(spec)


def _all_units_sane(res):
    """Properties that hold on every unit at any size."""
    assert np.all(np.abs(res["psum"] - 1.0) <= 1e-5), "probability sum off on some head"
    assert np.all(res["count"] >= 1)
    assert np.all(np.isfinite(res["out"]))


def test_c4_full_million_tokens():
    spec = W.make_spec("c4")
    sess, _ = _session(spec)
    q = W.queries(spec)
    res = run_step(sess, spec, q)
    _all_units_sane(res)
    assert np.all(res["cnt"] == spec.top_k)
    cache = {}
    check_step(spec, res, q, [(0, 5)], kv_cache=cache)
    dense = run_step(sess, spec, q, sparse=False)
    _all_units_sane(dense)
    check_step(spec, dense, q, [(0, 5)], sparse=False, kv_cache=cache, heads_per_unit=1)
    assert sess.device_status() == 0


def test_c3_full_gaussian_128k():
    spec = W.make_spec("c3")
    sess, _ = _session(spec)
    q = W.queries(spec)
    res = run_step(sess, spec, q)
    _all_units_sane(res)
    check_step(spec, res, q, [(0, 0), (3, 6)])
    assert sess.device_status() == 0


def test_c4g_full_gaussian_million_tokens():
    """The million-token shape with clustered keys and the Gaussian selector."""
    spec = W.make_spec("c4g")
    sess, _ = _session(spec)
    q = W.queries(spec)
    res = run_step(sess, spec, q)
    _all_units_sane(res)
    check_step(spec, res, q, [(0, 3)])
    assert sess.device_status() == 0


def test_c5_full_batched_appends():
    """16 sequences of 16K-64K tokens on permuted pages, one token appended
    per sequence per step for 64 steps; sampled units checked at the first,
    a middle and the last step."""
    from workloads.upload import step_tokens
    spec = W.make_spec("c5")
    sess, appended = _session(spec)
    checked = {0: [(2, 1)], 31: [(9, 4)], spec.steps - 1: [(2, 1), (15, 7)]}
    for s in range(spec.steps):
        k1, v1 = step_tokens(spec, appended, s)
        sess.append(k1, v1)
        q = W.queries(spec, s)
        res = run_step(sess, spec, q)
        _all_units_sane(res)
        if s in checked:
            print(f"[step {s}] checking {checked[s]}", flush=True)
            check_step(spec, res, q, checked[s])
    assert sess.device_status() == 0
