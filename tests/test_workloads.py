"""The seeded generators: deterministic, per-slice independent, right shapes,
and bf16 rounding is round-to-nearest-even."""
import numpy as np

import workloads as W
from workloads.configs import max_pages, needle_positions, total_lens


def test_shapes_and_determinism():
    s = W.make_spec("c2", context=2048, n_needles=8)
    k1 = W.keys(s, 0, 3)
    k2 = W.keys(s, 0, 3)
    assert k1.dtype == np.uint16 and k1.shape == (2048, 128)
    np.testing.assert_array_equal(k1, k2)
    assert not np.array_equal(W.keys(s, 0, 2), k1)
    q = W.queries(s)
    assert q.shape == (1, 32, 128) and q.dtype == np.float32
    assert W.keys(W.make_spec("c1"), 0, 0).dtype == np.float32


def test_bf16_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    b = W.round_to_bf16_bits(x)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6... mantissa 0x02)
    assert list(b) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81]


def test_page_table_permutation_and_lengths():
    s = W.make_spec("c5", batch=4, ctx_lo=100, ctx_hi=300, steps=5)
    L = W.seq_lens(s)
    assert np.all((L >= 100) & (L <= 300))
    tab, nphys = W.page_table(s)
    assert tab.shape == (4, max_pages(s))
    used = tab[tab >= 0]
    assert sorted(used.tolist()) == list(range(nphys))
    for b in range(4):
        assert np.sum(tab[b] >= 0) == -(-int(total_lens(s)[b]) // s.page_size)


def test_needles_point_at_their_query():
    s = W.make_spec("c2", context=4096, n_needles=8)
    q = W.queries(s)[0]
    k = W.keys(s, 0, 1).astype(np.uint32) << 16
    kf = k.view(np.float32)
    pos = needle_positions(s, 0, 1)
    # every needle is close to 3 q_h/|q_h| for one head of group 1
    for p in pos:
        cos = max(float(kf[p] @ q[h]) / (np.linalg.norm(kf[p]) * np.linalg.norm(q[h])) for h in range(4, 8))
        assert cos > 0.85  # noise norm ~0.1*sqrt(128) against amplitude 3
