"""GPU parity over a seeded sweep of shapes inside the library's stated limits:
head dim 64 or 128, groups of 1, 2, 4 or 8 query heads, pages of 1 to 256
tokens, fp32 or bf16 keys, top-k or Gaussian selection, alpha 1.5, 2 or a
general value, shared or per-query-head lists, ragged and permuted caches.
Every unit's sparse step and one unit's full-cache decode are compared with
the float64 oracle to the same bar as the workload tests."""
import numpy as np
import pytest

import workloads as W
from gpu_common import check_step, run_step

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = 48


def _cases():
    rng = np.random.default_rng(20261203)
    out = []
    for i in range(N_CASES):
        policy = "bbox" if i % 2 == 0 else "gauss"
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 4, 8]))
        P = int(rng.choice([1, 4, 16, 32, 64, 128, 256]))
        kv = "f32" if rng.random() < 0.3 else "bf16"
        alpha = float(rng.choice([1.5, 2.0, 1.25 if policy == "gauss" else 1.7, 1.8]))
        batch = int(rng.integers(1, 4))
        lo = int(rng.integers(100, 3000))
        hi = lo + int(rng.integers(0, 3000))
        per_head = bool(g > 1 and rng.random() < 0.3)
        out.append(dict(policy=policy, d=d, hkv=hkv, g=g, P=P, kv=kv, alpha=alpha, batch=batch, lo=lo, hi=hi,
                        per_head=per_head, seed=3000 + i))
    return out


def _spec(c):
    common = dict(batch=c["batch"], n_q_heads=c["hkv"] * c["g"], n_kv_heads=c["hkv"], head_dim=c["d"],
                  page_size=c["P"], kv_dtype=c["kv"], alpha=c["alpha"], context=0, ctx_lo=c["lo"],
                  ctx_hi=c["hi"], permute_pages=True, steps=0, seed=c["seed"])
    if c["policy"] == "bbox":
        pages = -(-c["lo"] // c["P"])
        return W.make_spec("c2", top_k=max(1, pages // 6), n_needles=8, **common)
    return W.make_spec("c3", **common)


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("case", _cases(), ids=lambda c: (f"{c['policy']}-d{c['d']}-g{c['g']}x{c['hkv']}-P{c['P']}-"
                                                          f"{c['kv']}-a{c['alpha']}-b{c['batch']}"
                                                          f"{'-ph' if c['per_head'] else ''}"))
def test_shape_sweep(case):
    from workloads.upload import build_session
    spec = _spec(case)
    print(f"[case] {case}", flush=True)
    sess, _ = build_session(spec)
    q = W.queries(spec)
    cache = {}
    per_head = case["per_head"]
    res = run_step(sess, spec, q, per_head=per_head)
    if per_head:
        units = [(b, h) for b in range(spec.batch) for h in range(spec.n_q_heads)]
    else:
        units = [(b, g) for b in range(spec.batch) for g in range(spec.n_kv_heads)]
    check_step(spec, res, q, units, kv_cache=cache, per_head=per_head)
    dense = run_step(sess, spec, q, sparse=False)
    check_step(spec, dense, q, [(spec.batch - 1, spec.n_kv_heads - 1)], sparse=False, kv_cache=cache)
    assert sess.device_status() == 0
