"""EntmaxKV support-aware paged sparse alpha-entmax decode for MI355X.

The compute path is the HIP library libentmaxkv.so (C ABI declared in
include/entmaxkv.h); this package only marshals torch tensors into its
arguments.  Importing the package does not load the library; the first call
does, and fails loudly if it has not been built (python -m
sparse_long_context_append_amd._build)."""
from .binding import (  # noqa: F401
    EKV_OK, EKV_ERR_INVALID_ARG, EKV_ERR_UNSUPPORTED, EKV_ERR_WORKSPACE, EKV_ERR_CAPACITY, EKV_ERR_HIP,
    EKV_F32, EKV_BF16, EKV_SELECT_BBOX_TOPK, EKV_SELECT_GAUSS,
    EntmaxKVError, PagedCache, Sequences, lib, lib_path,
    workspace_size, workspace_init, append_kv, select_pages, entmax_decode, entmax_decode_noalloc,
    softmax_decode, score_pages,
    read_device_status, status_string, last_error, stream_read,
)
