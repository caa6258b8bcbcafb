"""The C ABI on a machine without a GPU: the library loads, exports every
function include/entmaxkv.h declares, sizes workspaces, and rejects invalid
arguments with the documented status before touching the device."""
import ctypes
import os
import re

import pytest

import sparse_long_context_append_amd as ekv
from sparse_long_context_append_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000  # never dereferenced: every call below fails validation first


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "entmaxkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ekv_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.lib_path):
        pytest.skip("library not built")
    return B.lib()


def test_exports_every_declared_symbol(L):
    syms = declared_symbols()
    assert len(syms) >= 9
    for s in syms:
        assert hasattr(L, s), s


def cache(**kw):
    c = dict(n_phys_pages=256, n_kv_heads=8, page_size=16, head_dim=128, kv_dtype=B.EKV_BF16, reserved=0,
             k=FAKE, v=FAKE, k_box=FAKE, k_moments=FAKE)
    c.update(kw)
    return B._Cache(**c)


def seqs(**kw):
    s = dict(batch=1, max_pages=256, page_table=FAKE, seq_lens=FAKE)
    s.update(kw)
    return B._Seqs(**s)


def ws_size(L, c=None, s=None, hq=32, cap=0):
    return L.ekv_workspace_size(ctypes.byref(c or cache()), ctypes.byref(s or seqs()), hq, cap)


def test_workspace_size(L):
    n = ws_size(L)
    # candidate lists dominate: 6 lists of B*Hq*max_pages*P 4-byte entries
    assert n >= 6 * 4 * 32 * 256 * 16
    assert ws_size(L, hq=12) == 0  # not a multiple of 8
    assert ws_size(L, c=cache(head_dim=96)) == 0
    assert ws_size(L, c=cache(page_size=24)) == 0
    assert ws_size(L, c=cache(n_kv_heads=2), hq=64) == 0  # group 32
    assert L.ekv_workspace_size(None, ctypes.byref(seqs()), 32, 0) == 0
    # sized for lists of 16 pages: the per-item regions shrink 16-fold, the
    # rest does not depend on cap; cap <= 0 or >= max_pages is the full size
    small = ws_size(L, cap=16)
    assert small < n and n - small >= 6 * 4 * 32 * (256 - 16) * 16
    assert ws_size(L, cap=-1) == n and ws_size(L, cap=256) == n and ws_size(L, cap=10 ** 6) == n
    assert ws_size(L, cap=8) < small


def sp(**kw):
    p = dict(policy=B.EKV_SELECT_BBOX_TOPK, top_k=8, alpha=1.5, scale=0.125, delta=0.5, per_head=0, min_pages=1)
    p.update(kw)
    return B._SelectParams(**p)


def call_select(L, c=None, s=None, q=FAKE, hq=32, p=None, sel=FAKE, cnt=FAKE, cap=64, ws=FAKE, wsb=1 << 40):
    return L.ekv_select_pages(ctypes.byref(c or cache()), ctypes.byref(s or seqs()), q, hq,
                              ctypes.byref(p or sp()), sel, cnt, cap, None, ws, wsb, None)


def test_select_validation(L):
    assert call_select(L, q=None) == B.EKV_ERR_INVALID_ARG
    assert call_select(L, q=FAKE + 4) == B.EKV_ERR_INVALID_ARG  # misaligned
    assert call_select(L, p=sp(top_k=0)) == B.EKV_ERR_INVALID_ARG
    assert call_select(L, p=sp(policy=7)) == B.EKV_ERR_INVALID_ARG
    assert call_select(L, p=sp(alpha=1.0)) == B.EKV_ERR_INVALID_ARG
    assert call_select(L, p=sp(scale=0.0)) == B.EKV_ERR_INVALID_ARG
    assert call_select(L, p=sp(policy=B.EKV_SELECT_GAUSS, alpha=1.05)) == B.EKV_ERR_UNSUPPORTED
    assert call_select(L, p=sp(policy=B.EKV_SELECT_GAUSS, alpha=2.5)) == B.EKV_ERR_UNSUPPORTED
    assert call_select(L, c=cache(k_box=None)) == B.EKV_ERR_INVALID_ARG
    assert call_select(L, c=cache(k_moments=None), p=sp(policy=B.EKV_SELECT_GAUSS)) == B.EKV_ERR_INVALID_ARG
    assert call_select(L, cap=4) == B.EKV_ERR_CAPACITY
    assert call_select(L, cap=64, p=sp(policy=B.EKV_SELECT_GAUSS)) == B.EKV_ERR_CAPACITY  # needs max_pages
    assert call_select(L, ws=None) == B.EKV_ERR_WORKSPACE
    assert call_select(L, wsb=1024) == B.EKV_ERR_WORKSPACE
    assert "needs" in ekv.last_error()
    assert call_select(L, s=seqs(batch=0)) == B.EKV_ERR_INVALID_ARG
    assert call_select(L, s=seqs(batch=1024)) == B.EKV_ERR_UNSUPPORTED  # 8192 units
    assert call_select(L, hq=20) == B.EKV_ERR_INVALID_ARG
    assert call_select(L, sel=None) == B.EKV_ERR_INVALID_ARG
    assert call_select(L, p=sp(per_head=2)) == B.EKV_ERR_INVALID_ARG
    # per query head the units are batch * n_q_heads: 200 * 32 = 6400 > 4096
    assert call_select(L, s=seqs(batch=200), p=sp(per_head=1)) == B.EKV_ERR_UNSUPPORTED
    # the Gaussian floor: at least one page; more than one needs the top-k block's page limit
    g = dict(policy=B.EKV_SELECT_GAUSS)
    assert call_select(L, cap=256, p=sp(min_pages=0, **g)) == B.EKV_ERR_INVALID_ARG
    big = seqs(max_pages=70000)
    assert call_select(L, s=big, cap=70000, p=sp(min_pages=2, **g)) == B.EKV_ERR_UNSUPPORTED
    # selection needs only the cap-independent part of the workspace: the
    # size for one-page lists less its per-item regions (one 64-token item
    # per query head: four per-item arrays, six per-token arrays, 256-byte
    # aligned), one byte short
    a256 = lambda x: (x + 255) // 256 * 256
    items1 = 4 * a256(4 * 32) + 6 * a256(4 * 32 * 64)
    assert call_select(L, wsb=ws_size(L, cap=1) - items1 - 1) == B.EKV_ERR_WORKSPACE


def call_decode(L, q=FAKE, alpha=1.5, scale=0.125, sel=FAKE, cnt=FAKE, cap=64, sel_heads=8, out=FAKE, sidx=None,
                scap=0, ws=FAKE, wsb=1 << 40, c=None, s=None):
    return L.ekv_entmax_decode(ctypes.byref(c or cache()), ctypes.byref(s or seqs()), q, 32, alpha, scale, sel, cnt,
                               cap, sel_heads, out, None, None, None, sidx, None, scap, ws, wsb, None)


def test_decode_validation(L):
    assert call_decode(L, out=None) == B.EKV_ERR_INVALID_ARG
    assert call_decode(L, alpha=1.0) == B.EKV_ERR_INVALID_ARG
    assert call_decode(L, alpha=float("nan")) == B.EKV_ERR_INVALID_ARG
    assert call_decode(L, scale=-1.0) == B.EKV_ERR_INVALID_ARG
    assert call_decode(L, cnt=None) == B.EKV_ERR_INVALID_ARG
    assert call_decode(L, cap=0) == B.EKV_ERR_INVALID_ARG
    assert call_decode(L, sidx=FAKE, scap=0) == B.EKV_ERR_INVALID_ARG
    assert call_decode(L, wsb=100) == B.EKV_ERR_WORKSPACE
    assert call_decode(L, c=cache(k=None)) == B.EKV_ERR_INVALID_ARG
    assert call_decode(L, c=cache(kv_dtype=5)) == B.EKV_ERR_INVALID_ARG
    assert call_decode(L, sel_heads=5) == B.EKV_ERR_INVALID_ARG  # neither n_kv_heads nor n_q_heads
    assert call_decode(L, sel_heads=32, s=seqs(batch=200)) == B.EKV_ERR_UNSUPPORTED
    # a workspace sized for 64-page lists serves sparse calls of cap <= 64 only,
    # and no full-cache decode
    w64 = ws_size(L, cap=64)
    assert call_decode(L, cap=65, wsb=w64) == B.EKV_ERR_WORKSPACE
    assert call_decode(L, sel=None, cnt=None, cap=0, wsb=w64) == B.EKV_ERR_WORKSPACE
    assert "cap" in ekv.last_error()


def test_softmax_validation(L):
    f = L.ekv_softmax_decode
    call = lambda c=None, sel=FAKE, cnt=FAKE, cap=64, sh=8, out=FAKE, scale=0.125, wsb=1 << 40: f(
        ctypes.byref(c or cache()), ctypes.byref(seqs()), FAKE, 32, scale, sel, cnt, cap, sh, out, None, FAKE, wsb,
        None)
    assert call(out=None) == B.EKV_ERR_INVALID_ARG
    assert call(scale=0.0) == B.EKV_ERR_INVALID_ARG
    assert call(cnt=None) == B.EKV_ERR_INVALID_ARG
    assert call(wsb=100) == B.EKV_ERR_WORKSPACE
    assert call(c=cache(kv_dtype=B.EKV_F32)) == B.EKV_ERR_UNSUPPORTED
    assert call(sh=7) == B.EKV_ERR_INVALID_ARG


def test_append_validation(L):
    f = L.ekv_append_kv
    assert f(ctypes.byref(cache()), ctypes.byref(seqs()), FAKE, FAKE, -1, FAKE, 1 << 20, None) == B.EKV_ERR_INVALID_ARG
    assert f(ctypes.byref(cache()), ctypes.byref(seqs()), None, FAKE, 4, FAKE, 1 << 20, None) == B.EKV_ERR_INVALID_ARG
    assert f(ctypes.byref(cache()), ctypes.byref(seqs()), FAKE + 8, FAKE, 4, FAKE, 1 << 20, None) == B.EKV_ERR_INVALID_ARG
    assert f(ctypes.byref(cache()), ctypes.byref(seqs()), FAKE, FAKE, 4, None, 1 << 20, None) == B.EKV_ERR_WORKSPACE
    assert f(ctypes.byref(cache()), ctypes.byref(seqs()), FAKE, FAKE, 10 ** 6, FAKE, 1 << 20, None) == B.EKV_ERR_INVALID_ARG
    # n_new == 0 is a valid no-op that launches nothing
    assert f(ctypes.byref(cache()), ctypes.byref(seqs()), None, None, 0, FAKE, 1 << 20, None) == B.EKV_OK


def test_misc(L):
    assert ekv.status_string(B.EKV_ERR_CAPACITY) == "selection capacity too small"
    assert L.ekv_workspace_init(None, 0, None) == B.EKV_ERR_WORKSPACE
    assert L.ekv_workspace_init(FAKE, 17, None) == B.EKV_ERR_WORKSPACE
    flags = ctypes.c_int32(0)
    assert L.ekv_read_device_status(None, 0, ctypes.byref(flags), None) == B.EKV_ERR_WORKSPACE
    assert L.ekv_read_device_status(FAKE, 1 << 20, None, None) == B.EKV_ERR_INVALID_ARG


def test_noalloc_decode_validation(L):
    f = L.ekv_entmax_decode_noalloc
    call = lambda s=None, sel=FAKE, cnt=FAKE, cap=64, out=FAKE, alpha=1.5: f(
        ctypes.byref(cache()), ctypes.byref(s or seqs()), FAKE, 32, alpha, 0.125, sel, cnt, cap, 8, out, None, None,
        None, None, None, 0, None, None)
    assert call(out=None) == B.EKV_ERR_INVALID_ARG
    assert call(alpha=1.0) == B.EKV_ERR_INVALID_ARG
    assert call(cnt=None) == B.EKV_ERR_INVALID_ARG
    # 32 query heads x lists of 65536 pages of 16 tokens: far above the fixed scratch
    big = seqs(max_pages=65536)
    assert call(s=big, cap=65536) == B.EKV_ERR_WORKSPACE
    assert call(s=big, sel=None, cnt=None, cap=0) == B.EKV_ERR_WORKSPACE
    assert "scratch" in ekv.last_error()
