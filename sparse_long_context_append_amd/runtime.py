"""Device memory for one paged cache plus the buffers a decode step needs.

PyTorch only provides the device allocations and the stream; every
computation is a call into libentmaxkv.so through the binding."""
from __future__ import annotations

import numpy as np

from . import binding as B


def _torch():
    import torch
    return torch


class DecodeSession:
    """A paged KV cache (K, V, bounding box, moments), its page table and
    lengths, a workspace and selection buffers, all on one device.

    page_table: int32 [batch][max_pages] (host array or device tensor),
    seq_lens: int32 [batch] initial lengths (the cache starts empty: append
    fills it and advances the lengths).
    full_decode: size the workspace for full-cache decodes too (otherwise
    only for sparse decodes of lists of up to `cap` pages)."""

    def __init__(self, *, batch, n_kv_heads, n_q_heads, head_dim, page_size, kv_dtype, n_phys_pages,
                 page_table, device="cuda", with_box=True, with_moments=True, cap=None, full_decode=True):
        torch = _torch()
        self.torch = torch
        self.device = torch.device(device)
        self.batch, self.n_kv_heads, self.n_q_heads = batch, n_kv_heads, n_q_heads
        self.head_dim, self.page_size, self.n_phys_pages = head_dim, page_size, n_phys_pages
        self.kv_dtype = kv_dtype
        tdt = torch.bfloat16 if kv_dtype == B.EKV_BF16 else torch.float32
        shape = (n_phys_pages, n_kv_heads, page_size, head_dim)
        self.k = torch.zeros(shape, dtype=tdt, device=self.device)
        self.v = torch.zeros(shape, dtype=tdt, device=self.device)
        mshape = (n_phys_pages, n_kv_heads, 2, head_dim)
        self.k_box = torch.zeros(mshape, dtype=tdt, device=self.device) if with_box else None
        self.k_moments = torch.zeros(mshape, dtype=torch.float32, device=self.device) if with_moments else None
        pt = torch.as_tensor(np.asarray(page_table, dtype=np.int32)) if isinstance(page_table, np.ndarray) else page_table
        self.page_table = pt.to(self.device, torch.int32).contiguous()
        self.max_pages = int(self.page_table.shape[1])
        self.seq_lens = torch.zeros(batch, dtype=torch.int32, device=self.device)
        self.cache = B.PagedCache(self.k, self.v, self.k_box, self.k_moments, n_phys_pages, n_kv_heads,
                                  page_size, head_dim, kv_dtype)
        self.seqs = B.Sequences(self.page_table, self.seq_lens, batch, self.max_pages)
        self.cap = int(cap if cap is not None else self.max_pages)
        nbytes = B.workspace_size(self.cache, self.seqs, n_q_heads, 0 if full_decode else self.cap)
        if nbytes == 0:
            raise ValueError("invalid cache/sequence shape: " + B.last_error())
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        B.workspace_init(self.ws)
        # room for one page list per query head; the last selection decides
        # whether the rows are KV heads (shared lists) or query heads
        self._sel_buf = torch.zeros(batch * n_q_heads * self.cap, dtype=torch.int32, device=self.device)
        self._cnt_buf = torch.zeros(batch * n_q_heads, dtype=torch.int32, device=self.device)
        self.sel_heads = n_kv_heads
        self.out = torch.zeros((batch, n_q_heads, head_dim), dtype=torch.float32, device=self.device)
        self.tau = torch.zeros((batch, n_q_heads), dtype=torch.float32, device=self.device)
        self.support_count = torch.zeros((batch, n_q_heads), dtype=torch.int32, device=self.device)
        self.psum = torch.zeros((batch, n_q_heads), dtype=torch.float32, device=self.device)
        self.tau_hat = torch.zeros((batch, n_q_heads), dtype=torch.float32, device=self.device)

    # -- cache growth -------------------------------------------------------
    def _one_seq_view(self, b: int) -> B.Sequences:
        ptab = self.page_table.data_ptr() + 4 * b * self.max_pages
        plen = self.seq_lens.data_ptr() + 4 * b
        return B.Sequences(ptab, plen, 1, self.max_pages)

    def append(self, k_new, v_new, seq: int | None = None):
        """Append k_new/v_new ([B][n][Hkv][d], or [1][n][Hkv][d] for one
        sequence `seq`) and advance the lengths."""
        n = int(k_new.shape[1])
        seqs = self.seqs if seq is None else self._one_seq_view(seq)
        B.append_kv(self.cache, seqs, k_new, v_new, n, self.ws)
        if seq is None:
            self.seq_lens += n
        else:
            self.seq_lens[seq] += n

    # -- decode step --------------------------------------------------------
    @property
    def sel(self):
        """[batch][sel_heads][cap] selected logical pages of the last selection."""
        n = self.batch * self.sel_heads
        return self._sel_buf[: n * self.cap].view(self.batch, self.sel_heads, self.cap)

    @property
    def sel_count(self):
        return self._cnt_buf[: self.batch * self.sel_heads].view(self.batch, self.sel_heads)

    def select(self, q, *, policy, alpha, scale, top_k=0, delta=0.0, per_head=False, min_pages=1):
        """Page selection shared by each KV head's query group, or one
        selection per query head (per_head=True)."""
        self.sel_heads = self.n_q_heads if per_head else self.n_kv_heads
        B.select_pages(self.cache, self.seqs, q, self.n_q_heads, policy=policy, top_k=top_k, alpha=alpha,
                       scale=scale, delta=delta, per_head=per_head, min_pages=min_pages, sel=self.sel,
                       sel_count=self.sel_count, cap=self.cap, tau_hat=self.tau_hat, ws=self.ws)

    def decode(self, q, *, alpha, scale, sparse=True, support_idx=None, support_p=None, support_cap=0):
        B.entmax_decode(self.cache, self.seqs, q, self.n_q_heads, alpha=alpha, scale=scale,
                        sel=self.sel if sparse else None, sel_count=self.sel_count if sparse else None,
                        cap=self.cap if sparse else 0, sel_heads=self.sel_heads, out=self.out, tau=self.tau,
                        support_count=self.support_count, psum=self.psum, support_idx=support_idx,
                        support_p=support_p, support_cap=support_cap, ws=self.ws)

    def decode_softmax(self, q, *, scale, sparse=True, out=None, lse=None):
        """Softmax attention over the selected pages (or the whole cache);
        writes `out` (default: the session's output buffer)."""
        B.softmax_decode(self.cache, self.seqs, q, self.n_q_heads, scale=scale,
                         sel=self.sel if sparse else None, sel_count=self.sel_count if sparse else None,
                         cap=self.cap if sparse else 0, sel_heads=self.sel_heads,
                         out=self.out if out is None else out, lse=lse, ws=self.ws)

    def scores(self, q, *, policy, alpha, scale, per_head=False):
        torch = self.torch
        if policy == B.EKV_SELECT_BBOX_TOPK:
            rows = self.n_q_heads if per_head else self.n_kv_heads
            s = torch.empty((self.batch, rows, self.max_pages), dtype=torch.float32, device=self.device)
        else:
            s = torch.empty((self.batch, self.n_q_heads, self.max_pages, 4), dtype=torch.float32, device=self.device)
        B.score_pages(self.cache, self.seqs, q, self.n_q_heads, policy=policy, alpha=alpha, scale=scale,
                      per_head=per_head, scores=s, ws=self.ws)
        return s

    def device_status(self) -> int:
        return B.read_device_status(self.ws)
