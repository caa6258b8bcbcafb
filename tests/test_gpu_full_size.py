"""GPU parity at the workloads' full sizes, in the configuration bench.py
times (DecodeSession select + decode on the default stream), checked against
the float64 oracle on every (sequence, KV head) unit: the oracle rebuilds
each unit's metadata, scores, selection, threshold, support and output from
the raw keys, one unit at a time (its float64 copies are dropped before the
next unit).  The full-cache decode is checked on one query head of every
unit at 1M tokens and on all heads of two units at 4 x 128K."""
import time

import numpy as np
import pytest

import workloads as W
from gpu_common import check_step, run_step

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

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


def _check_every_unit(spec, q, sparse, dense=None, dense_units=(), dense_heads=None):
    """Sparse result checked on every unit; the dense result (if given) on
    dense_units ('all' for every unit), dense_heads heads each."""
    t0 = time.perf_counter()
    units = [(b, g) for b in range(spec.batch) for g in range(spec.n_kv_heads)]
    worst = 0.0
    for i, u in enumerate(units):
        cache = {}
        worst = max(worst, check_step(spec, sparse, q, [u], kv_cache=cache))
        if dense is not None and (dense_units == "all" or u in dense_units):
            worst = max(worst, check_step(spec, dense, q, [u], sparse=False, kv_cache=cache,
                                          heads_per_unit=dense_heads))
        del cache
        print(f"  unit {i + 1}/{len(units)} {u} ok ({time.perf_counter() - t0:.0f}s, worst error {worst:.2e})",
              flush=True)
    return worst


def test_c4_full_million_tokens():
    spec = W.make_spec("c4")
    sess, _ = _session(spec)
    q = W.queries(spec)
    res = run_step(sess, spec, q)
    _all_units_sane(res)
    assert np.all(res["cnt"] == spec.top_k)
    dense = run_step(sess, spec, q, sparse=False)
    _all_units_sane(dense)
    assert sess.device_status() == 0
    del sess
    _check_every_unit(spec, q, res, dense, dense_units="all", dense_heads=1)


def test_c3_full_gaussian_128k():
    spec = W.make_spec("c3")
    sess, _ = _session(spec)
    q = W.queries(spec)
    res = run_step(sess, spec, q)
    _all_units_sane(res)
    dense = run_step(sess, spec, q, sparse=False)
    _all_units_sane(dense)
    assert sess.device_status() == 0
    del sess
    _check_every_unit(spec, q, res, dense, dense_units=((0, 0), (3, 6)))


def test_c4g_full_gaussian_million_tokens():
    """The million-token shape with clustered keys and the Gaussian selector."""
    spec = W.make_spec("c4g")
    sess, _ = _session(spec)
    q = W.queries(spec)
    res = run_step(sess, spec, q)
    _all_units_sane(res)
    assert sess.device_status() == 0
    del sess
    _check_every_unit(spec, q, res)


def test_c5_full_batched_appends():
    """16 sequences of 16K-64K tokens on permuted pages, one token appended
    per sequence per step for 64 steps; sampled units checked at the first
    and a middle step, every unit at the last step."""
    from workloads.upload import step_tokens
    spec = W.make_spec("c5")
    sess, appended = _session(spec)
    checked = {0: [(2, 1)], 31: [(9, 4)]}
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
    del sess
    print(f"[step {spec.steps - 1}] checking every unit", flush=True)
    _check_every_unit(spec, q, res)
