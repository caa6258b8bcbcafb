"""ctypes binding of libentmaxkv.so.  Argument marshalling only: every step
of the decode path runs in the library's HIP kernels.  Names mirror the C
ABI in include/entmaxkv.h (without the ekv_ prefix)."""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

EKV_OK = 0
EKV_ERR_INVALID_ARG = -1
EKV_ERR_UNSUPPORTED = -2
EKV_ERR_WORKSPACE = -3
EKV_ERR_CAPACITY = -4
EKV_ERR_HIP = -5
EKV_F32 = 0
EKV_BF16 = 1
EKV_SELECT_BBOX_TOPK = 0
EKV_SELECT_GAUSS = 1

lib_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libentmaxkv.so")


class EntmaxKVError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {status} ({status_string(status)}): {msg}")
        self.status = status


class _Cache(ctypes.Structure):
    _fields_ = [
        ("n_phys_pages", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("k_box", ctypes.c_void_p), ("k_moments", ctypes.c_void_p),
    ]


class _Seqs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("max_pages", ctypes.c_int32),
        ("page_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
    ]


class _SelectParams(ctypes.Structure):
    _fields_ = [
        ("policy", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("alpha", ctypes.c_float), ("scale", ctypes.c_float),
        ("delta", ctypes.c_float), ("per_head", ctypes.c_int32),
        ("min_pages", ctypes.c_int32),
    ]


_LIB = None
_vp, _sz, _i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
_PC, _PS, _PP = ctypes.POINTER(_Cache), ctypes.POINTER(_Seqs), ctypes.POINTER(_SelectParams)
_SIGS = {
    "ekv_workspace_size": (_sz, [_PC, _PS, _i32, _i32]),
    "ekv_workspace_init": (_i32, [_vp, _sz, _vp]),
    "ekv_append_kv": (_i32, [_PC, _PS, _vp, _vp, _i32, _vp, _sz, _vp]),
    "ekv_select_pages": (_i32, [_PC, _PS, _vp, _i32, _PP, _vp, _vp, _i32, _vp, _vp, _sz, _vp]),
    "ekv_entmax_decode": (_i32, [_PC, _PS, _vp, _i32, ctypes.c_float, ctypes.c_float, _vp, _vp, _i32, _i32,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _sz, _vp]),
    "ekv_entmax_decode_noalloc": (_i32, [_PC, _PS, _vp, _i32, ctypes.c_float, ctypes.c_float, _vp, _vp, _i32,
                                         _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp]),
    "ekv_softmax_decode": (_i32, [_PC, _PS, _vp, _i32, ctypes.c_float, _vp, _vp, _i32, _i32, _vp, _vp, _vp,
                                  _sz, _vp]),
    "ekv_score_pages": (_i32, [_PC, _PS, _vp, _i32, _PP, _vp, _vp, _sz, _vp]),
    "ekv_read_device_status": (_i32, [_vp, _sz, ctypes.POINTER(_i32), _vp]),
    "ekv_stream_read": (_i32, [_vp, _sz, _vp, _i32, _vp]),
    "ekv_status_string": (ctypes.c_char_p, [_i32]),
    "ekv_last_error": (ctypes.c_char_p, []),
}


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises if it was not built)."""
    global _LIB
    if _LIB is None:
        # Load PyTorch's HIP runtime first when PyTorch is present, so the
        # library binds to the same runtime copy (and device context) as the
        # tensors it is handed.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is missing: build it with python -m sparse_long_context_append_amd._build")
        L = ctypes.CDLL(lib_path)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().ekv_status_string(status).decode()


def last_error() -> str:
    return lib().ekv_last_error().decode()


def _check(status: int, where: str):
    if status != EKV_OK:
        raise EntmaxKVError(status, where, last_error())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


@dataclass
class PagedCache:
    """Device tensors of the paged cache; see ekv_cache in include/entmaxkv.h.
    k, v: [n_phys][Hkv][P][d]; k_box: [n_phys][Hkv][2][d] (kv dtype);
    k_moments: [n_phys][Hkv][2][d] float32."""
    k: object
    v: object
    k_box: object
    k_moments: object
    n_phys_pages: int
    n_kv_heads: int
    page_size: int
    head_dim: int
    kv_dtype: int

    def c(self) -> _Cache:
        return _Cache(self.n_phys_pages, self.n_kv_heads, self.page_size, self.head_dim, self.kv_dtype, 0,
                      _ptr(self.k), _ptr(self.v), _ptr(self.k_box), _ptr(self.k_moments))


@dataclass
class Sequences:
    """page_table: int32 [B][max_pages]; seq_lens: int32 [B] (device)."""
    page_table: object
    seq_lens: object
    batch: int
    max_pages: int

    def c(self) -> _Seqs:
        return _Seqs(self.batch, self.max_pages, _ptr(self.page_table), _ptr(self.seq_lens))


def workspace_size(cache: PagedCache, seqs: Sequences, n_q_heads: int, cap: int = 0) -> int:
    """cap: largest page-list capacity of the sparse decodes served (0: the
    whole cache, as full-cache decodes need)."""
    return int(lib().ekv_workspace_size(ctypes.byref(cache.c()), ctypes.byref(seqs.c()), n_q_heads, int(cap)))


def workspace_init(ws, stream=None):
    _check(lib().ekv_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "workspace_init")


def append_kv(cache: PagedCache, seqs: Sequences, k_new, v_new, n_new: int, ws, stream=None):
    _check(lib().ekv_append_kv(ctypes.byref(cache.c()), ctypes.byref(seqs.c()), _ptr(k_new), _ptr(v_new),
                               n_new, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "append_kv")


def _params(policy, top_k, alpha, scale, delta, per_head=False, min_pages=1) -> _SelectParams:
    return _SelectParams(int(policy), int(top_k), float(alpha), float(scale), float(delta), int(bool(per_head)),
                         int(min_pages))


def _sel_heads(cache: PagedCache, sel, sel_heads):
    """Rows of `sel` per sequence: given, else read from a [B][H][cap] tensor."""
    if sel_heads is not None:
        return int(sel_heads)
    if sel is not None and hasattr(sel, "shape") and len(sel.shape) == 3:
        return int(sel.shape[1])
    return cache.n_kv_heads


def select_pages(cache: PagedCache, seqs: Sequences, q, n_q_heads: int, *, policy: int, top_k: int = 0,
                 alpha: float, scale: float, delta: float = 0.0, per_head: bool = False, min_pages: int = 1,
                 sel, sel_count, cap: int, tau_hat=None, ws, stream=None):
    p = _params(policy, top_k, alpha, scale, delta, per_head, min_pages)
    _check(lib().ekv_select_pages(ctypes.byref(cache.c()), ctypes.byref(seqs.c()), _ptr(q), n_q_heads,
                                  ctypes.byref(p), _ptr(sel), _ptr(sel_count), cap, _ptr(tau_hat), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)), "select_pages")


def score_pages(cache: PagedCache, seqs: Sequences, q, n_q_heads: int, *, policy: int, alpha: float,
                scale: float, per_head: bool = False, scores, ws, stream=None):
    p = _params(policy, 1, alpha, scale, 0.0, per_head)
    _check(lib().ekv_score_pages(ctypes.byref(cache.c()), ctypes.byref(seqs.c()), _ptr(q), n_q_heads,
                                 ctypes.byref(p), _ptr(scores), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(stream)), "score_pages")


def entmax_decode(cache: PagedCache, seqs: Sequences, q, n_q_heads: int, *, alpha: float, scale: float,
                  sel=None, sel_count=None, cap: int = 0, sel_heads=None, out, tau=None, support_count=None,
                  psum=None, support_idx=None, support_p=None, support_cap: int = 0, ws, stream=None):
    _check(lib().ekv_entmax_decode(ctypes.byref(cache.c()), ctypes.byref(seqs.c()), _ptr(q), n_q_heads,
                                   float(alpha), float(scale), _ptr(sel), _ptr(sel_count), cap,
                                   _sel_heads(cache, sel, sel_heads), _ptr(out),
                                   _ptr(tau), _ptr(support_count), _ptr(psum), _ptr(support_idx),
                                   _ptr(support_p), support_cap, _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)), "entmax_decode")


def entmax_decode_noalloc(cache: PagedCache, seqs: Sequences, q, n_q_heads: int, *, alpha: float, scale: float,
                          sel=None, sel_count=None, cap: int = 0, sel_heads=None, out, tau=None,
                          support_count=None, psum=None, support_idx=None, support_p=None, support_cap: int = 0,
                          dev_status=None, stream=None):
    """entmax_decode on the library's fixed device scratch (no workspace)."""
    _check(lib().ekv_entmax_decode_noalloc(ctypes.byref(cache.c()), ctypes.byref(seqs.c()), _ptr(q), n_q_heads,
                                           float(alpha), float(scale), _ptr(sel), _ptr(sel_count), cap,
                                           _sel_heads(cache, sel, sel_heads), _ptr(out), _ptr(tau),
                                           _ptr(support_count), _ptr(psum), _ptr(support_idx), _ptr(support_p),
                                           support_cap, _ptr(dev_status), _stream(stream)),
           "entmax_decode_noalloc")


def softmax_decode(cache: PagedCache, seqs: Sequences, q, n_q_heads: int, *, scale: float, sel=None,
                   sel_count=None, cap: int = 0, sel_heads=None, out, lse=None, ws, stream=None):
    _check(lib().ekv_softmax_decode(ctypes.byref(cache.c()), ctypes.byref(seqs.c()), _ptr(q), n_q_heads,
                                    float(scale), _ptr(sel), _ptr(sel_count), cap,
                                    _sel_heads(cache, sel, sel_heads), _ptr(out), _ptr(lse),
                                    _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "softmax_decode")


def read_device_status(ws, stream=None) -> int:
    """Status bits of the work enqueued so far on `stream` (default: torch's
    current stream), cleared afterwards; waits for that stream."""
    flags = ctypes.c_int32(0)
    _check(lib().ekv_read_device_status(_ptr(ws), ws.numel() * ws.element_size(), ctypes.byref(flags),
                                        _stream(stream)), "read_device_status")
    return flags.value


def stream_read(src, sink, blocks: int = 0, nbytes: int | None = None, stream=None):
    """Plain streaming read of `src` (measurement helper: the read-stream
    ceiling at a given size)."""
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    _check(lib().ekv_stream_read(_ptr(src), n, _ptr(sink), int(blocks), _stream(stream)), "stream_read")
