"""SOCKET soft-LSH sparse-attention decode path for AMD MI355X (gfx950).

The compute lives in the HIP library ``libsocket_lsh.so`` (C ABI in
``include/socket_lsh.h``); this package only marshals torch tensors into
its entry points.  Importing the package does not load the library; the
first call does, and raises if the library has not been built.
"""
from . import layout  # noqa: F401
from ._lib import (  # noqa: F401
    SOCKET_BF16, SOCKET_F32, SocketError, alloc_ids, alloc_workspace, lib, socket_hash_keys,
    socket_dense_decode, socket_dense_decode_workspace, socket_ids_bytes, socket_score,
    socket_score_topk, socket_score_topk_workspace, socket_soft_tables, socket_sparse_decode,
    socket_sparse_decode_workspace, socket_topk, score_stride,
    alloc_codes, codes_words, socket_codes_bytes, socket_hash_codes, socket_hard_score_topk,
    socket_hard_score_topk_workspace, socket_sample_estimate, socket_decode_step,
    socket_decode_step_workspace, socket_decode_step_noalloc, NOALLOC_SCRATCH_BYTES,
)

__version__ = "0.1.0"
