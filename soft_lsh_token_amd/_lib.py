"""ctypes binding of ``libsocket_lsh.so`` (C ABI in include/socket_lsh.h).

Argument marshalling only: every function checks the tensors' shapes,
dtypes and devices, passes raw device pointers and the current HIP stream
to the library, and raises :class:`SocketError` on a non-zero status.  All
compute happens in the HIP kernels.  There is no fallback: if the library
is missing, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsocket_lsh.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "socket_lsh.h")

SOCKET_F32, SOCKET_BF16 = 0, 1
STATUS = {0: "SOCKET_OK", -1: "SOCKET_EINVAL", -2: "SOCKET_EUNSUPPORTED", -3: "SOCKET_ENOSPC",
          -4: "SOCKET_EHIP"}

_vp, _i, _i64, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "socket_status_string": (ctypes.c_char_p, [_i]),
    "socket_version": (_i, []),
    "socket_ids_bytes": (_sz, [_i, _i, _i64, _i, _i]),
    "socket_hash_keys": (_i, [_vp, _vp, _i, _i, _i, _i, _i64, _vp, _i, _vp, _i, _i, _vp, _vp, _vp]),
    "socket_score_topk_workspace": (_sz, [_i, _i, _i, _i64, _i, _i, _i]),
    "socket_score_topk": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _i, _i, _f, _vp, _vp, _vp, _i64, _vp,
                               _i, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "socket_soft_tables": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _i, _i, _f, _i64, _vp, _sz, _vp]),
    "socket_score": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _i64, _i, _i, _vp, _vp, _sz, _vp]),
    "socket_topk": (_i, [_i, _i, _i, _i, _vp, _vp, _i64, _vp, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "socket_sparse_decode_workspace": (_sz, [_i, _i, _i, _i]),
    "socket_sparse_decode": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i64, _vp, _i, _f, _vp, _vp,
                                  _sz, _vp]),
    "socket_dense_decode_workspace": (_sz, [_i, _i, _i, _i, _i64]),
    "socket_codes_bytes": (_sz, [_i, _i, _i64, _i, _i]),
    "socket_decode_step_workspace": (_sz, [_i, _i, _i, _i64, _i, _i, _i]),
    "socket_decode_step": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _i, _f, _vp, _vp, _vp,
                                _i64, _vp, _i, _i, _i, _f, _vp, _vp, _vp, _vp, _sz, _vp]),
    "socket_decode_step_noalloc": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _i, _f, _vp,
                                        _vp, _vp, _i64, _vp, _i, _i, _i, _f, _vp, _vp, _vp, _vp]),
    "socket_sample_estimate": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _i, _i, _f, _vp, _vp, _vp, _vp,
                                    _i64, _vp, _i, _vp, _vp, _vp, _vp, _sz, _vp]),
    "socket_hash_codes": (_i, [_vp, _vp, _i, _i, _i, _i, _i64, _vp, _i, _vp, _i, _i, _vp, _vp,
                               _vp]),
    "socket_hard_score_topk_workspace": (_sz, [_i, _i, _i, _i64, _i, _i, _i]),
    "socket_hard_score_topk": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _i, _i, _vp, _vp, _vp, _i64,
                                    _vp, _i, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "socket_dense_decode": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i64, _vp, _f, _vp, _vp, _sz,
                                 _vp]),
}

_lib = None


class SocketError(RuntimeError):
    def __init__(self, fn: str, status: int):
        name = STATUS.get(status, str(status))
        super().__init__(f"{fn} failed with {name} ({lib().socket_status_string(status).decode()})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m "
                               "soft_lsh_token_amd.build` (needs hipcc)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def header_functions() -> list[str]:
    """Names of the functions declared in include/socket_lsh.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(socket_\w+)\s*\(", text, re.M)))


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise SocketError(fn, rc)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SOCKET_BF16
    if t.dtype == torch.float32:
        return SOCKET_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def socket_ids_bytes(B: int, Hkv: int, n_cap: int, L: int, P: int) -> int:
    return int(lib().socket_ids_bytes(B, Hkv, n_cap, L, P))


def alloc_ids(B: int, Hkv: int, n_cap: int, L: int, P: int, device) -> torch.Tensor:
    """A zeroed bucket-ID cache (tiled layout, see soft_lsh_token_amd.layout)."""
    from .layout import ids_shape
    t = torch.zeros(ids_shape(B, Hkv, n_cap, L, P), dtype=torch.uint8, device=device)
    assert t.numel() == socket_ids_bytes(B, Hkv, n_cap, L, P)
    return t


def _ids(ids: torch.Tensor, B: int, Hkv: int, n_cap: int, L: int, P: int) -> int:
    from .layout import ids_shape
    return _dev(ids, "ids", torch.uint8, ids_shape(B, Hkv, n_cap, L, P))


def socket_hash_keys(K: torch.Tensor | None, V: torch.Tensor | None, W: torch.Tensor | None,
                     ids: torch.Tensor | None, vnorm: torch.Tensor | None, pos0: torch.Tensor,
                     count: int, L: int, P: int, stream=None) -> None:
    """Hash rows [pos0[b], pos0[b]+count) of K into ids and store ||V|| in vnorm.
    ids=None (with K, W None allowed) stores the norms only; V=vnorm=None the IDs only."""
    ref = K if K is not None else V
    B, Hkv, n_cap, d = ref.shape
    dt = _dtype_code(ref)
    rc = lib().socket_hash_keys(
        None if K is None else _dev(K, "K", ref.dtype, ref.shape),
        None if V is None else _dev(V, "V", ref.dtype, ref.shape), dt, B, Hkv, d, n_cap,
        _dev(pos0, "pos0", torch.int32, (B,)), int(count),
        None if W is None else _dev(W, "W", ref.dtype, (L * P, d)), L, P,
        None if ids is None else _ids(ids, B, Hkv, n_cap, L, P),
        None if vnorm is None else _dev(vnorm, "vnorm", torch.float32, (B, Hkv, n_cap)),
        _stream(ref, stream))
    _check("socket_hash_keys", rc)


def socket_score_topk_workspace(B: int, Hq: int, Hkv: int, n_cap: int, L: int, P: int,
                                k_max: int) -> int:
    return int(lib().socket_score_topk_workspace(B, Hq, Hkv, n_cap, L, P, k_max))


def socket_sparse_decode_workspace(B: int, Hq: int, d: int, k_max: int) -> int:
    return int(lib().socket_sparse_decode_workspace(B, Hq, d, k_max))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """A device byte buffer whose data pointer is 256-byte aligned."""
    return torch.empty(max(int(nbytes), 1) + 256, dtype=torch.uint8, device=device)


def _temp_workspace(nbytes: int, device, stream) -> torch.Tensor:
    """A workspace for one call when the caller passes none.  It is freed when
    the call returns, while its kernels may still be queued, so it is recorded
    on the stream they run on: torch's caching allocator then hands the block
    to no other stream before that work has finished."""
    ws = alloc_workspace(nbytes, device)
    if stream is not None:
        if isinstance(stream, torch.cuda.Stream):
            s = stream
        else:
            handle = int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)
            s = torch.cuda.ExternalStream(handle, device=device)
        ws.record_stream(s)
    return ws


def score_stride(n_cap: int) -> int:
    """Row stride of the score rows: n_cap rounded up to 64."""
    return (n_cap + 63) // 64 * 64


def _ws_ptr(ws: torch.Tensor, need: int) -> tuple[int, int]:
    base = _dev(ws, "ws", torch.uint8)
    off = (-base) % 256
    return base + off, ws.numel() - off


def socket_score_topk(q: torch.Tensor, W: torch.Tensor, ids: torch.Tensor, vnorm: torch.Tensor,
                      lens: torch.Tensor, ks: torch.Tensor, k_max: int, tau: float, L: int, P: int,
                      idx: torch.Tensor, scores: torch.Tensor | None = None,
                      ws: torch.Tensor | None = None, stream=None, sink: int = 0,
                      window: int = 0) -> None:
    """Soft-LSH scores of every key and the selected indices per query head: the
    top-k keys plus the first `sink` and last `window` keys of each sequence."""
    B, Hq, d = q.shape
    Hkv, n_cap = vnorm.shape[1], vnorm.shape[2]
    need = socket_score_topk_workspace(B, Hq, Hkv, n_cap, L, P, k_max)
    if ws is None:
        ws = _temp_workspace(need, q.device, stream)
    wptr, wbytes = _ws_ptr(ws, need)
    sptr = None if scores is None else _dev(scores, "scores", torch.float32,
                                            (B, Hq, score_stride(n_cap)))
    rc = lib().socket_score_topk(
        _dev(q, "q"), _dtype_code(q), B, Hq, Hkv, d, _dev(W, "W", q.dtype, (L * P, d)), L, P,
        float(tau), _ids(ids, B, Hkv, n_cap, L, P),
        _dev(vnorm, "vnorm", torch.float32, (B, Hkv, n_cap)),
        _dev(lens, "lens", torch.int32, (B,)), n_cap, _dev(ks, "ks", torch.int32, (B,)),
        int(k_max), int(sink), int(window), _dev(idx, "idx", torch.int32, (B, Hq, k_max)), sptr,
        wptr, wbytes, _stream(q, stream))
    _check("socket_score_topk", rc)


def socket_soft_tables(q: torch.Tensor, W: torch.Tensor, Hkv: int, L: int, P: int, tau: float,
                       n_cap: int, ws: torch.Tensor, stream=None) -> None:
    """Algorithm 2, first half: every table's bucket distribution (into ws)."""
    B, Hq, d = q.shape
    wptr, wbytes = _ws_ptr(ws, 0)
    rc = lib().socket_soft_tables(_dev(q, "q"), _dtype_code(q), B, Hq, Hkv, d,
                                  _dev(W, "W", q.dtype, (L * P, d)), L, P, float(tau), int(n_cap),
                                  wptr, wbytes, _stream(q, stream))
    _check("socket_soft_tables", rc)


def socket_score(ids: torch.Tensor, vnorm: torch.Tensor, lens: torch.Tensor, Hq: int, L: int,
                 P: int, scores: torch.Tensor, ws: torch.Tensor, stream=None, sink: int = 0,
                 window: int = 0) -> None:
    """Algorithm 2, second half: soft-count scores (needs socket_soft_tables on ws first)."""
    B, Hkv, n_cap = vnorm.shape
    wptr, wbytes = _ws_ptr(ws, 0)
    rc = lib().socket_score(B, Hq, Hkv, L, P, _ids(ids, B, Hkv, n_cap, L, P),
                            _dev(vnorm, "vnorm", torch.float32, (B, Hkv, n_cap)),
                            _dev(lens, "lens", torch.int32, (B,)), n_cap, int(sink), int(window),
                            _dev(scores, "scores", torch.float32, (B, Hq, score_stride(n_cap))),
                            wptr, wbytes,
                            _stream(ids, stream))
    _check("socket_score", rc)


def socket_topk(scores: torch.Tensor, lens: torch.Tensor, ks: torch.Tensor, Hkv: int, L: int,
                n_cap: int, idx: torch.Tensor, ws: torch.Tensor, stream=None, sink: int = 0,
                window: int = 0) -> None:
    """Algorithm 3: top-k per query head from scores + the histogram socket_score left in ws."""
    B, Hq, _ = scores.shape
    k_max = idx.shape[-1]
    wptr, wbytes = _ws_ptr(ws, 0)
    rc = lib().socket_topk(B, Hq, Hkv, L, _dev(scores, "scores", torch.float32,
                           (B, Hq, score_stride(n_cap))), _dev(lens, "lens",
                           torch.int32, (B,)), n_cap, _dev(ks, "ks", torch.int32, (B,)), k_max,
                           int(sink), int(window), _dev(idx, "idx", torch.int32, (B, Hq, k_max)),
                           wptr, wbytes,
                           _stream(scores, stream))
    _check("socket_topk", rc)


def socket_sparse_decode(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, idx: torch.Tensor,
                         scale: float, out: torch.Tensor, ws: torch.Tensor | None = None,
                         stream=None) -> None:
    """Exact attention of q over the keys listed in idx (-1 entries skipped)."""
    B, Hq, d = q.shape
    _, Hkv, n_cap, _ = K.shape
    k_max = idx.shape[-1]
    need = socket_sparse_decode_workspace(B, Hq, d, k_max)
    if ws is None:
        ws = _temp_workspace(need, q.device, stream)
    wptr, wbytes = _ws_ptr(ws, need)
    rc = lib().socket_sparse_decode(
        _dev(q, "q"), _dev(K, "K", q.dtype), _dev(V, "V", q.dtype, K.shape), _dtype_code(q), B, Hq,
        Hkv, d, n_cap, _dev(idx, "idx", torch.int32, (B, Hq, k_max)), k_max, float(scale),
        _dev(out, "out", torch.float32, (B, Hq, d)), wptr, wbytes, _stream(q, stream))
    _check("socket_sparse_decode", rc)


def socket_dense_decode_workspace(B: int, Hq: int, Hkv: int, d: int, n_cap: int) -> int:
    return int(lib().socket_dense_decode_workspace(B, Hq, Hkv, d, n_cap))


def socket_dense_decode(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, lens: torch.Tensor,
                        scale: float, out: torch.Tensor, ws: torch.Tensor | None = None,
                        stream=None) -> None:
    """Full attention of q over keys [0, lens[b]) of its KV head (the dense reference)."""
    B, Hq, d = q.shape
    _, Hkv, n_cap, _ = K.shape
    need = socket_dense_decode_workspace(B, Hq, Hkv, d, n_cap)
    if ws is None:
        ws = _temp_workspace(need, q.device, stream)
    wptr, wbytes = _ws_ptr(ws, need)
    rc = lib().socket_dense_decode(
        _dev(q, "q"), _dev(K, "K", q.dtype), _dev(V, "V", q.dtype, K.shape), _dtype_code(q), B, Hq,
        Hkv, d, n_cap, _dev(lens, "lens", torch.int32, (B,)), float(scale),
        _dev(out, "out", torch.float32, (B, Hq, d)), wptr, wbytes, _stream(q, stream))
    _check("socket_dense_decode", rc)


# ----------------------------------------------------------------------------- hard-LSH mode

def codes_words(L: int, P: int) -> int:
    return (L * P + 31) // 32


def socket_codes_bytes(B: int, Hkv: int, n_cap: int, L: int, P: int) -> int:
    return int(lib().socket_codes_bytes(B, Hkv, n_cap, L, P))


def alloc_codes(B: int, Hkv: int, n_cap: int, L: int, P: int, device) -> torch.Tensor:
    """A zeroed code cache for the hard-LSH mode: int32 [B, Hkv, words, n_cap]."""
    t = torch.zeros(B, Hkv, codes_words(L, P), n_cap, dtype=torch.int32, device=device)
    assert t.numel() * 4 == socket_codes_bytes(B, Hkv, n_cap, L, P)
    return t


def socket_hash_codes(K: torch.Tensor, V: torch.Tensor, W: torch.Tensor, codes: torch.Tensor,
                      vnorm: torch.Tensor, pos0: torch.Tensor, count: int, L: int, P: int,
                      stream=None) -> None:
    """Sign codes of rows [pos0[b], pos0[b]+count) of K, and ||V|| into vnorm."""
    B, Hkv, n_cap, d = K.shape
    rc = lib().socket_hash_codes(
        _dev(K, "K"), _dev(V, "V", K.dtype, K.shape), _dtype_code(K), B, Hkv, d, n_cap,
        _dev(pos0, "pos0", torch.int32, (B,)), int(count), _dev(W, "W", K.dtype, (L * P, d)),
        L, P, _dev(codes, "codes", torch.int32, (B, Hkv, codes_words(L, P), n_cap)),
        _dev(vnorm, "vnorm", torch.float32, (B, Hkv, n_cap)), _stream(K, stream))
    _check("socket_hash_codes", rc)


def socket_hard_score_topk_workspace(B: int, Hq: int, Hkv: int, n_cap: int, L: int, P: int,
                                     k_max: int) -> int:
    return int(lib().socket_hard_score_topk_workspace(B, Hq, Hkv, n_cap, L, P, k_max))


def socket_hard_score_topk(q: torch.Tensor, W: torch.Tensor, codes: torch.Tensor,
                           vnorm: torch.Tensor, lens: torch.Tensor, ks: torch.Tensor, k_max: int,
                           L: int, P: int, idx: torch.Tensor, scores: torch.Tensor | None = None,
                           ws: torch.Tensor | None = None, stream=None, sink: int = 0,
                           window: int = 0) -> None:
    """Hard collision-count scores and the selected indices per query head."""
    B, Hq, d = q.shape
    Hkv, n_cap = vnorm.shape[1], vnorm.shape[2]
    need = socket_hard_score_topk_workspace(B, Hq, Hkv, n_cap, L, P, k_max)
    if ws is None:
        ws = _temp_workspace(need, q.device, stream)
    wptr, wbytes = _ws_ptr(ws, need)
    sptr = None if scores is None else _dev(scores, "scores", torch.float32,
                                            (B, Hq, score_stride(n_cap)))
    rc = lib().socket_hard_score_topk(
        _dev(q, "q"), _dtype_code(q), B, Hq, Hkv, d, _dev(W, "W", q.dtype, (L * P, d)), L, P,
        _dev(codes, "codes", torch.int32, (B, Hkv, codes_words(L, P), n_cap)),
        _dev(vnorm, "vnorm", torch.float32, (B, Hkv, n_cap)),
        _dev(lens, "lens", torch.int32, (B,)), n_cap, _dev(ks, "ks", torch.int32, (B,)),
        int(k_max), int(sink), int(window), _dev(idx, "idx", torch.int32, (B, Hq, k_max)), sptr,
        wptr, wbytes, _stream(q, stream))
    _check("socket_hard_score_topk", rc)


# ----------------------------------------------------------------------------- sampling estimator

def socket_sample_estimate(q: torch.Tensor, W: torch.Tensor, ids: torch.Tensor,
                           vnorm: torch.Tensor, V: torch.Tensor, lens: torch.Tensor,
                           u: torch.Tensor, tau: float, L: int, P: int, out: torch.Tensor,
                           draws: torch.Tensor | None = None, scores: torch.Tensor | None = None,
                           ws: torch.Tensor | None = None, stream=None) -> None:
    """Value-aware sampling estimate T(q) of the soft-attention output, from the
    uniforms u [B, Hq, M]; the drawn key indices go to draws when given."""
    B, Hq, d = q.shape
    Hkv, n_cap = vnorm.shape[1], vnorm.shape[2]
    M = u.shape[-1]
    need = socket_score_topk_workspace(B, Hq, Hkv, n_cap, L, P, 1)
    if ws is None:
        ws = _temp_workspace(need, q.device, stream)
    wptr, wbytes = _ws_ptr(ws, need)
    dptr = None if draws is None else _dev(draws, "draws", torch.int32, (B, Hq, M))
    sptr = None if scores is None else _dev(scores, "scores", torch.float32,
                                            (B, Hq, score_stride(n_cap)))
    rc = lib().socket_sample_estimate(
        _dev(q, "q"), _dtype_code(q), B, Hq, Hkv, d, _dev(W, "W", q.dtype, (L * P, d)), L, P,
        float(tau), _ids(ids, B, Hkv, n_cap, L, P),
        _dev(vnorm, "vnorm", torch.float32, (B, Hkv, n_cap)),
        _dev(V, "V", q.dtype, (B, Hkv, n_cap, d)), _dev(lens, "lens", torch.int32, (B,)), n_cap,
        _dev(u, "u", torch.float32, (B, Hq, M)), M, _dev(out, "out", torch.float32, (B, Hq, d)),
        dptr, sptr, wptr, wbytes, _stream(q, stream))
    _check("socket_sample_estimate", rc)


# ----------------------------------------------------------------------------- fused step

def socket_decode_step_workspace(B: int, Hq: int, Hkv: int, n_cap: int, L: int, P: int,
                                 k_max: int) -> int:
    return int(lib().socket_decode_step_workspace(B, Hq, Hkv, n_cap, L, P, k_max))


def socket_decode_step(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, W: torch.Tensor,
                       ids: torch.Tensor, vnorm: torch.Tensor, lens: torch.Tensor,
                       ks: torch.Tensor, k_max: int, tau: float, L: int, P: int, scale: float,
                       idx: torch.Tensor, out: torch.Tensor, scores: torch.Tensor | None = None,
                       ws: torch.Tensor | None = None, stream=None, sink: int = 0,
                       window: int = 0) -> None:
    """One decode step: hash key lens[b] - 1, select, attend (see the header)."""
    B, Hq, d = q.shape
    _, Hkv, n_cap, _ = K.shape
    need = socket_decode_step_workspace(B, Hq, Hkv, n_cap, L, P, k_max)
    if ws is None:
        ws = _temp_workspace(need, q.device, stream)
    wptr, wbytes = _ws_ptr(ws, need)
    sptr = None if scores is None else _dev(scores, "scores", torch.float32,
                                            (B, Hq, score_stride(n_cap)))
    rc = lib().socket_decode_step(
        _dev(q, "q"), _dev(K, "K", q.dtype), _dev(V, "V", q.dtype, K.shape), _dtype_code(q), B, Hq,
        Hkv, d, _dev(W, "W", q.dtype, (L * P, d)), L, P, float(tau), _ids(ids, B, Hkv, n_cap, L, P),
        _dev(vnorm, "vnorm", torch.float32, (B, Hkv, n_cap)), _dev(lens, "lens", torch.int32, (B,)),
        n_cap, _dev(ks, "ks", torch.int32, (B,)), int(k_max), int(sink), int(window), float(scale),
        _dev(idx, "idx", torch.int32, (B, Hq, k_max)), sptr,
        _dev(out, "out", torch.float32, (B, Hq, d)), wptr, wbytes, _stream(q, stream))
    _check("socket_decode_step", rc)


NOALLOC_SCRATCH_BYTES = 64 << 20  # SOCKET_NOALLOC_SCRATCH_BYTES


def socket_decode_step_noalloc(q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
                               W: torch.Tensor, ids: torch.Tensor, vnorm: torch.Tensor,
                               lens: torch.Tensor, ks: torch.Tensor, k_max: int, tau: float, L: int,
                               P: int, scale: float, idx: torch.Tensor, out: torch.Tensor,
                               scores: torch.Tensor | None = None, stream=None, sink: int = 0,
                               window: int = 0) -> None:
    """socket_decode_step with the library's static scratch memory instead of a
    workspace: no device memory is allocated (see the header for the size limit
    and the rule that calls on one GPU must not overlap)."""
    B, Hq, d = q.shape
    _, Hkv, n_cap, _ = K.shape
    sptr = None if scores is None else _dev(scores, "scores", torch.float32,
                                            (B, Hq, score_stride(n_cap)))
    rc = lib().socket_decode_step_noalloc(
        _dev(q, "q"), _dev(K, "K", q.dtype), _dev(V, "V", q.dtype, K.shape), _dtype_code(q), B, Hq,
        Hkv, d, _dev(W, "W", q.dtype, (L * P, d)), L, P, float(tau), _ids(ids, B, Hkv, n_cap, L, P),
        _dev(vnorm, "vnorm", torch.float32, (B, Hkv, n_cap)), _dev(lens, "lens", torch.int32, (B,)),
        n_cap, _dev(ks, "ks", torch.int32, (B,)), int(k_max), int(sink), int(window), float(scale),
        _dev(idx, "idx", torch.int32, (B, Hq, k_max)), sptr,
        _dev(out, "out", torch.float32, (B, Hq, d)), _stream(q, stream))
    _check("socket_decode_step_noalloc", rc)
