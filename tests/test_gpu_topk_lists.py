"""Top-k through the scoring's candidate lists (bf16 records scored 256
pages per block, shared selections; each wave lists the 8 largest scores
of its 64 pages).  Pages of one token and q = e_h make
every bounding-box score an integer, exact in bf16, fp32 and float64, so
the oracle's selection (the k highest scores, the lower page first on
ties) is compared exactly, ties included.  The cases cover the list path
(ties across blocks at the k-th score, both list widths), the two ways it
falls back to the whole score row (64 pages holding more than their list
of the k pages; equal scores everywhere), ragged and empty sequences, and a
group of four query heads."""
import numpy as np
import pytest

from oracle import metadata, scoring, select

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bf16(a):
    """float array of values exact in bf16 -> bf16 tensor on the device"""
    a = np.ascontiguousarray(a, dtype=np.float32)
    assert np.array_equal(a, (a.view(np.uint32) & 0xFFFF0000).view(np.float32)), "value not exact in bf16"
    return torch.from_numpy(a).cuda().to(torch.bfloat16)


def _select(keys, lens, top_k, group=1, label=""):
    """keys [B][n][Hkv][d] (integers |x| <= 256), lengths per sequence; runs
    the selection and compares every unit with the oracle exactly."""
    from sparse_long_context_append_amd.runtime import DecodeSession
    import sparse_long_context_append_amd as ekv
    B, n, Hkv, d = keys.shape
    Hq = Hkv * group
    print(f"[case] topk lists {label} B={B} n={n} Hkv={Hkv} G={group} lens={list(lens)} top_k={top_k}", flush=True)
    table = np.arange(B * n, dtype=np.int32).reshape(B, n)
    sess = DecodeSession(batch=B, n_kv_heads=Hkv, n_q_heads=Hq, head_dim=d, page_size=1, kv_dtype=ekv.EKV_BF16,
                         n_phys_pages=B * n, page_table=table, cap=top_k, full_decode=False)
    for b in range(B):
        if lens[b] > 0:
            kb = _bf16(keys[b:b + 1, :lens[b]])
            sess.append(kb, torch.zeros_like(kb), seq=b)
    q = np.zeros((B, Hq, d), dtype=np.float32)
    for h in range(Hq):
        q[:, h, h % group] = 1.0  # head h of a group scores dimension h
    sess.select(torch.from_numpy(q).cuda(), policy=ekv.EKV_SELECT_BBOX_TOPK, alpha=1.5, scale=1.0, top_k=top_k)
    torch.cuda.synchronize()
    sel = sess.sel.cpu().numpy()
    cnt = sess.sel_count.cpu().numpy()
    for b in range(B):
        for g in range(Hkv):
            L = int(lens[b])
            md = metadata.page_metadata(keys[b, :L, g].astype(np.float64), L, 1)
            S = scoring.bbox_page_scores(q[b, g * group:(g + 1) * group].astype(np.float64), md["kmin"], md["kmax"],
                                         1.0)
            want = select.topk_pages(S, top_k)
            assert int(cnt[b, g]) == want.size, f"unit ({b},{g}): {cnt[b, g]} pages, expected {want.size}"
            np.testing.assert_array_equal(sel[b, g, :want.size], want, err_msg=f"unit ({b},{g})")
    assert sess.device_status() == 0


def _levels(rng, shape, hi_frac, tie_frac, tie_level=20, hi=(21, 41)):
    """integer scores: most in 0..9, a tie level, a few above it"""
    u = rng.random(shape)
    x = rng.integers(0, 10, shape).astype(np.float32)
    x[u < hi_frac + tie_frac] = tie_level
    x[u < hi_frac] = rng.integers(*hi, shape)[u < hi_frac]
    return x


def _keys(rng, B, n, Hkv, d, dim0):
    k = rng.integers(-3, 4, (B, n, Hkv, d)).astype(np.float32)
    k[..., :dim0.shape[-1]] = dim0
    return k


def test_lists_with_ties_across_blocks():
    """16384 pages per KV head, 8 heads: 256 lists, 2048 entries (two per
    thread).  The k-th score lies inside a level shared by about 1.5 % of
    the pages, spread over every list, so the lower-page rule picks among
    listed pages of many lists."""
    rng = np.random.default_rng(5)
    B, n, Hkv, d = 1, 16384, 8, 64
    s = _levels(rng, (B, n, Hkv, 1), 0.01, 0.015)
    _select(_keys(rng, B, n, Hkv, d, s), [n], 300, label="ties")


def test_lists_at_max_pages():
    """65535 pages per KV head, 4 heads: 1024 lists, 8192 entries (eight
    per thread), the last list ragged; scores 0..256 with many ties."""
    rng = np.random.default_rng(6)
    B, n, Hkv, d = 1, 65535, 4, 64
    s = rng.integers(0, 257, (B, n, Hkv, 1)).astype(np.float32)
    _select(_keys(rng, B, n, Hkv, d, s), [n], 1000, label="max pages")


def test_lists_fall_back_when_one_block_holds_the_top():
    """The 256 pages of one scoring block score highest on four heads: each
    of its lists holds 64 candidates for k = 200, more than its 8, so its
    cut is among the k and the selection runs over the whole row; the other
    heads' top pages are spread (list path)."""
    rng = np.random.default_rng(7)
    B, n, Hkv, d = 1, 16384, 8, 64
    s = _levels(rng, (B, n, Hkv, 1), 0.005, 0.01)
    s[:, 512:768, :4, 0] = rng.integers(100, 200, (B, 256, 4))
    _select(_keys(rng, B, n, Hkv, d, s), [n], 200, label="one block")


def test_lists_fall_back_on_equal_scores():
    """Every score 0: each list's cut equals the listed scores, so the row
    decides, and the k lowest pages win."""
    rng = np.random.default_rng(8)
    B, n, Hkv, d = 1, 16384, 8, 64
    s = np.zeros((B, n, Hkv, 1), dtype=np.float32)
    _select(_keys(rng, B, n, Hkv, d, s), [n], 5, label="equal")


def test_lists_ragged_and_empty_sequences():
    """Three sequences of 16307, 300 and 0 pages in a table of 16384: the
    first ends inside a list; the second has 40 listed pages (five lists),
    fewer than k = 150, so its row decides; the third selects nothing.  With
    k = 400 the second keeps all its pages."""
    rng = np.random.default_rng(9)
    B, n, Hkv, d = 3, 16384, 8, 64
    s = _levels(rng, (B, n, Hkv, 1), 0.005, 0.01)
    k = _keys(rng, B, n, Hkv, d, s)
    _select(k, [n - 77, 300, 0], 150, label="ragged")
    _select(k, [n - 77, 300, 0], 400, label="ragged")


def test_lists_group_of_four():
    """Groups of four query heads: the page score is the largest of the four
    heads' bounds (head h reads dimension h), 4096 pages, 8 KV heads, 4
    sequences."""
    rng = np.random.default_rng(10)
    B, n, Hkv, d = 4, 4096, 8, 64
    s = _levels(rng, (B, n, Hkv, 4), 0.003, 0.004)
    _select(_keys(rng, B, n, Hkv, d, s), [n, n - 1, 2500, 4000], 60, group=4, label="group 4")
