"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, sizes workspaces, and rejects bad arguments before it
enqueues anything (no GPU needed: every call here returns during argument
checking)."""
from __future__ import annotations

import ctypes

import pytest

import soft_lsh_token_amd as S
from soft_lsh_token_amd import _lib

EINVAL, EUNSUP, ENOSPC = -1, -2, -3
FAKE = 0x10000  # a non-null, 256-aligned stand-in pointer; never dereferenced


def test_library_exports_every_header_function():
    lib = S.lib()
    names = _lib.header_functions()
    assert {"socket_hash_keys", "socket_score_topk", "socket_sparse_decode",
            "socket_score_topk_workspace", "socket_sparse_decode_workspace",
            "socket_status_string", "socket_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_status_strings():
    lib = S.lib()
    for code in (0, EINVAL, EUNSUP, ENOSPC, -4):
        assert lib.socket_status_string(code)
    assert lib.socket_status_string(-99) == b"unknown status"
    assert lib.socket_version() >= 100


def test_workspace_sizes():
    a = S.socket_score_topk_workspace(1, 32, 8, 32768, 64, 8, 656)
    b = S.socket_score_topk_workspace(1, 32, 8, 131072, 64, 8, 1024)
    assert 0 < a < b
    assert a % 256 == 0
    assert S.socket_score_topk_workspace(0, 32, 8, 32768, 64, 8, 656) == 0
    assert S.socket_score_topk_workspace(1, 32, 4, 32768, 64, 8, 656) > 0   # 8 heads per KV head
    assert S.socket_score_topk_workspace(1, 130, 2, 32768, 64, 8, 656) == 0  # 65: too many
    assert S.socket_score_topk_workspace(1, 32, 8, 32768, 129, 8, 656) == 0
    assert S.socket_score_topk_workspace(1, 32, 8, 32768, 65, 10, 656) == 0
    # one workspace size for both ID widths (the stage entries take no P)
    assert S.socket_score_topk_workspace(1, 32, 8, 32768, 60, 10, 656) == \
        S.socket_score_topk_workspace(1, 32, 8, 32768, 60, 8, 656)
    assert S.socket_sparse_decode_workspace(1, 32, 128, 1024) > 0
    assert S.socket_sparse_decode_workspace(1, 32, 64, 1024) == 0


def _hash(**kw):
    args = dict(K=FAKE, V=FAKE, dtype=1, B=1, Hkv=8, d=128, n_cap=1024, pos0=FAKE, count=16,
                W=FAKE, L=64, P=8, ids=FAKE, vnorm=FAKE, stream=None)
    args.update(kw)
    return S.lib().socket_hash_keys(*args.values())


def test_hash_argument_checks():
    assert _hash(K=None) == EINVAL
    assert _hash(W=None) == EINVAL
    assert _hash(vnorm=None) == EINVAL            # V without vnorm
    assert _hash(V=None) == EINVAL                # vnorm without V
    assert _hash(ids=None, vnorm=None, V=None) == EINVAL  # no output
    assert _hash(pos0=None) == EINVAL
    assert _hash(ids=None, K=None, W=None, count=0) == 0  # norms only: K and W not needed
    assert _hash(V=None, vnorm=None, count=0) == 0        # IDs only
    assert _hash(dtype=7) == EINVAL
    assert _hash(B=0) == EINVAL
    assert _hash(count=-1) == EINVAL
    assert _hash(d=64) == EUNSUP
    assert _hash(P=11) == EUNSUP
    assert _hash(P=10, L=65) == EUNSUP    # two-byte IDs: at most 64 tables
    assert _hash(L=300) == EUNSUP
    assert _hash(count=0) == 0  # nothing to do, nothing enqueued


def _score(**kw):
    B, Hq, n_cap, L, P, k_max = 1, 32, 1024, 64, 8, 32
    need = S.socket_score_topk_workspace(B, Hq, 8, n_cap, L, P, k_max)
    args = dict(q=FAKE, dtype=1, B=B, Hq=Hq, Hkv=8, d=128, W=FAKE, L=L, P=P, tau=0.5, ids=FAKE,
                vnorm=FAKE, lens=FAKE, n_cap=n_cap, ks=FAKE, k_max=k_max, sink=0, window=0, idx=FAKE,
                scores=None, ws=FAKE, ws_bytes=need, stream=None)
    args.update(kw)
    return S.lib().socket_score_topk(*args.values())


def test_score_argument_checks():
    assert _score(q=None) == EINVAL
    assert _score(ws=None) == EINVAL
    assert _score(tau=0.0) == EINVAL
    assert _score(tau=float("nan")) == EINVAL
    assert _score(tau=float("inf")) == EINVAL
    assert _score(Hkv=5) == EINVAL        # 32 % 5
    assert _score(Hq=130, Hkv=2) == EUNSUP  # 65 query heads per KV head (at most 64)
    assert S.socket_score_topk_workspace(1, 64, 8, 1024, 64, 8, 32) > 0   # 8 per KV head
    assert S.socket_score_topk_workspace(1, 24, 8, 1024, 64, 8, 32) > 0   # 3 per KV head
    assert _score(P=11) == EUNSUP
    assert _score(P=9, L=65) == EUNSUP
    assert _score(d=96) == EUNSUP
    assert _score(k_max=0) == EINVAL
    assert _score(ws=FAKE + 8) == EINVAL  # misaligned workspace
    assert _score(ws_bytes=1024) == ENOSPC
    assert _score(sink=-1) == EINVAL
    assert _score(window=-4) == EINVAL
    assert _score(sink=20, window=13) == EINVAL   # the forced keys alone overflow k_max = 32


def test_dense_decode_argument_checks():
    lib = S.lib()
    need = S.socket_dense_decode_workspace(1, 32, 8, 128, 32768)
    assert need >= 32 * 64 * 130 * 4             # 64 splits of 512 keys, (o, m, l) per head
    assert S.socket_dense_decode_workspace(1, 32, 8, 64, 32768) == 0
    assert S.socket_dense_decode_workspace(1, 32, 8, 128, 0) == 0
    assert S.socket_dense_decode_workspace(1, 32, 5, 128, 100) == 0
    args = dict(q=FAKE, K=FAKE, V=FAKE, dtype=1, B=1, Hq=32, Hkv=8, d=128, n_cap=32768, lens=FAKE,
                scale=0.088, out=FAKE, ws=FAKE, ws_bytes=need, stream=None)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return lib.socket_dense_decode(*a.values())
    assert call(lens=None) == EINVAL
    assert call(Hkv=5) == EINVAL
    assert call(Hq=130, Hkv=2) == EUNSUP       # 65 query heads per KV head (at most 64)
    assert S.socket_dense_decode_workspace(1, 64, 8, 128, 32768) > 0   # 8 per KV head
    assert call(d=96) == EUNSUP
    assert call(scale=float("nan")) == EINVAL
    assert call(ws=FAKE + 8) == EINVAL
    assert call(ws_bytes=need - 1) == ENOSPC


def test_hard_mode_argument_checks():
    lib = S.lib()
    assert S.socket_codes_bytes(1, 8, 1000, 300, 2) == 8 * 19 * 1000 * 4   # 600 bits -> 19 words
    assert S.socket_codes_bytes(1, 8, 1000, 500, 2) == 8 * 32 * 1000 * 4
    assert S.socket_codes_bytes(1, 8, 1000, 100, 3) == 0                   # P must divide 32
    assert S.socket_codes_bytes(1, 8, 1000, 4097, 1) == 0
    need = S.socket_hard_score_topk_workspace(1, 32, 8, 1024, 300, 2, 64)
    assert need > 0
    assert S.socket_hard_score_topk_workspace(1, 32, 4, 1024, 300, 2, 64) > 0   # 8 heads per KV head
    assert S.socket_hard_score_topk_workspace(1, 130, 2, 1024, 300, 2, 64) == 0  # 65: too many
    h = dict(K=FAKE, V=FAKE, dtype=1, B=1, Hkv=8, d=128, n_cap=1024, pos0=FAKE, count=16, W=FAKE,
             L=300, P=2, codes=FAKE, vnorm=FAKE, stream=None)

    def hc(**kw):
        a = dict(h)
        a.update(kw)
        return lib.socket_hash_codes(*a.values())
    assert hc(codes=None) == EINVAL
    assert hc(P=3) == EUNSUP
    assert hc(d=64) == EUNSUP
    assert hc(count=0) == 0
    a = dict(q=FAKE, dtype=1, B=1, Hq=32, Hkv=8, d=128, W=FAKE, L=300, P=2, codes=FAKE,
             vnorm=FAKE, lens=FAKE, n_cap=1024, ks=FAKE, k_max=64, sink=0, window=0, idx=FAKE,
             scores=None, ws=FAKE, ws_bytes=need, stream=None)

    def hs(**kw):
        b = dict(a)
        b.update(kw)
        return lib.socket_hard_score_topk(*b.values())
    assert hs(codes=None) == EINVAL
    assert hs(Hkv=5) == EINVAL
    assert hs(P=6) == EUNSUP
    assert hs(sink=40, window=40) == EINVAL
    assert hs(ws=FAKE + 4) == EINVAL
    assert hs(ws_bytes=need - 1) == ENOSPC


def test_codes_to_ids_bits():
    """The host view of hard-mode codes: ID bit j of table l is code bit l*P + j."""
    import numpy as np
    from soft_lsh_token_amd import layout
    rng = np.random.default_rng(4)
    for L, P in ((300, 2), (9, 4), (33, 1), (4, 16)):
        nw = (L * P + 31) // 32
        codes = rng.integers(0, 2 ** 32, size=(2, 3, nw, 5), dtype=np.uint64).astype(np.uint32)
        ids = layout.codes_to_ids(codes.view(np.int32), L, P)
        assert ids.shape == (2, 3, 5, L)
        for (b, h, i, l) in [(0, 0, 0, 0), (1, 2, 4, L - 1), (0, 1, 3, L // 2)]:
            want = 0
            for j in range(P):
                p = l * P + j
                want |= int((int(codes[b, h, p // 32, i]) >> (p % 32)) & 1) << j
            assert ids[b, h, i, l] == want


def _decode(**kw):
    B, Hq, k_max = 1, 32, 64
    need = S.socket_sparse_decode_workspace(B, Hq, 128, k_max)
    args = dict(q=FAKE, K=FAKE, V=FAKE, dtype=1, B=B, Hq=Hq, Hkv=8, d=128, n_cap=1024, idx=FAKE,
                k_max=k_max, scale=0.088, out=FAKE, ws=FAKE, ws_bytes=need, stream=None)
    args.update(kw)
    return S.lib().socket_sparse_decode(*args.values())


def test_decode_argument_checks():
    assert _decode(idx=None) == EINVAL
    assert _decode(out=None) == EINVAL
    assert _decode(dtype=3) == EINVAL
    assert _decode(Hkv=3) == EINVAL
    assert _decode(scale=float("nan")) == EINVAL
    assert _decode(d=256) == EUNSUP
    assert _decode(ws_bytes=16) == ENOSPC


def test_binding_rejects_host_tensors():
    import torch
    K = torch.zeros(1, 1, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        S.socket_hash_keys(K, K, torch.zeros(8, 128, dtype=torch.bfloat16),
                           torch.zeros(1, 1, 8, 1, dtype=torch.uint8),
                           torch.zeros(1, 1, 8), torch.zeros(1, dtype=torch.int32), 8, 1, 8)


def test_stage_argument_checks():
    lib = S.lib()
    need = S.socket_score_topk_workspace(1, 32, 8, 1024, 64, 8, 32)
    # socket_soft_tables(q, dtype, B, Hq, Hkv, d, W, L, P, tau, n_cap, ws, ws_bytes, stream)
    assert lib.socket_soft_tables(None, 1, 1, 32, 8, 128, FAKE, 64, 8, 0.5, 1024, FAKE, need, None) == EINVAL
    assert lib.socket_soft_tables(FAKE, 1, 1, 32, 8, 128, FAKE, 64, 8, -1.0, 1024, FAKE, need, None) == EINVAL
    assert lib.socket_soft_tables(FAKE, 1, 1, 32, 8, 64, FAKE, 64, 8, 0.5, 1024, FAKE, need, None) == EUNSUP
    assert lib.socket_soft_tables(FAKE, 1, 1, 32, 8, 128, FAKE, 64, 8, 0.5, 1024, FAKE, 64, None) == ENOSPC
    # socket_score(B, Hq, Hkv, L, P, ids, vnorm, lens, n_cap, sink, window, scores, ws,
    #              ws_bytes, stream)
    assert lib.socket_score(1, 32, 8, 64, 8, None, FAKE, FAKE, 1024, 0, 0, FAKE, FAKE, need, None) == EINVAL
    assert lib.socket_score(1, 32, 5, 64, 8, FAKE, FAKE, FAKE, 1024, 0, 0, FAKE, FAKE, need, None) == EINVAL
    assert lib.socket_score(1, 32, 8, 64, 8, FAKE, FAKE, FAKE, 1024, 0, 0, FAKE, None, need, None) == EINVAL
    assert lib.socket_score(1, 32, 8, 64, 8, FAKE, FAKE, FAKE, 1024, -1, 0, FAKE, FAKE, need, None) == EINVAL
    # socket_topk(B, Hq, Hkv, L, scores, lens, n_cap, ks, k_max, sink, window, idx, ws,
    #             ws_bytes, stream)
    assert lib.socket_topk(1, 32, 8, 64, FAKE, FAKE, 1024, FAKE, 0, 0, 0, FAKE, FAKE, need, None) == EINVAL
    assert lib.socket_topk(1, 32, 8, 64, FAKE, None, 1024, FAKE, 32, 0, 0, FAKE, FAKE, need, None) == EINVAL
    assert lib.socket_topk(1, 32, 8, 64, FAKE, FAKE, 1024, FAKE, 32, 0, 0, FAKE, FAKE, 16, None) == ENOSPC
    assert lib.socket_topk(1, 32, 8, 64, FAKE, FAKE, 1024, FAKE, 32, 16, 17, FAKE, FAKE, need, None) == EINVAL


@pytest.mark.parametrize("L,P", [(3, 8), (16, 8), (20, 8), (32, 8), (60, 8), (64, 8), (100, 8),
                                 (128, 8), (5, 10), (16, 9), (20, 10), (60, 10), (64, 10)])
def test_ids_layout_roundtrip_and_formula(L, P):
    """pack/unpack invert each other and place each ID's bytes where the header's formula says."""
    import numpy as np
    from soft_lsh_token_amd import layout
    rng = np.random.default_rng(L * 16 + P)
    B, Hkv, n, n_cap = 2, 3, 150, 200
    C = 2 if P > 8 else 1
    ids = rng.integers(0, 1 << P, size=(B, Hkv, n, L)).astype(np.uint16 if C == 2 else np.uint8)
    tiled = layout.pack(ids, n_cap, P)
    assert tiled.dtype == np.uint8
    assert tiled.shape == layout.ids_shape(B, Hkv, n_cap, L, P)
    assert tiled.size == S.socket_ids_bytes(B, Hkv, n_cap, L, P)
    np.testing.assert_array_equal(layout.unpack(tiled, L, n, P), ids)
    TL = layout.tables_per_word(L)
    assert 16 * TL >= L and (TL == 1 or 8 * TL < L)
    WB = TL * C
    assert layout.word_bytes(L, P) == WB
    flat = tiled.reshape(-1)
    G = (n_cap + 63) // 64
    packed = P > 8 and L > 32
    assert layout.packed(L, P) == packed
    assert layout.key_bytes(L, P) == (80 if packed else 16 * WB)
    for (b, h, i, l) in [(0, 0, 0, 0), (1, 2, 149, L - 1), (0, 1, 77, L // 2), (1, 0, 64, 0),
                         (1, 1, 100, min(L - 1, 3)), (0, 2, 15, min(L - 1, 35))]:
        r, w, cell = b * Hkv + h, l // TL, l % TL
        t = i % 64
        kg, x = t // 16, t % 16
        u = (x - w) % 16
        if packed:  # the header's packed formula: 40-bit word = 4 low bytes + 1 high byte
            base = (r * G + i // 64) * 5120
            lo = base + (u // 4) * 1024 + 16 * (16 * kg + w) + 4 * (u % 4)
            hi = base + 4096 + 16 * (16 * kg + w) + u
            word = int.from_bytes(bytes(flat[lo:lo + 4]), "little") | (int(flat[hi]) << 32)
            value = (word >> (10 * cell)) & 0x3FF
        else:
            R = 16 // WB
            off = ((r * G + i // 64) * 1024 + (u // R) * 64 * R + (16 * kg + w) * R + u % R) * WB
            off += cell * C
            value = int(flat[off]) | (int(flat[off + 1]) << 8 if C == 2 else 0)
        assert value == ids[b, h, i, l]


def test_p10_footprint():
    """At the pages' operating point (P = 10, L = 60: 600 bits a token, SOCKET Sec. 1) the
    cache stores 80 bytes of IDs and a 4-byte norm per key, 16.4% over bf16 K and V at
    d = 128 (the pages put it near 15%, Sec. 7)."""
    per_key = S.socket_ids_bytes(1, 1, 64, 60, 10) // 64
    assert per_key == 80 and per_key * 8 >= 600
    assert (per_key + 4) / (2 * 128 * 2) < 0.17


def test_ids_bytes_limits():
    """Table shapes without an ID layout are refused (size 0)."""
    assert S.socket_ids_bytes(1, 1, 10, 129, 8) == 0
    assert S.socket_ids_bytes(1, 1, 10, 65, 10) == 0
    assert S.socket_ids_bytes(1, 1, 10, 64, 11) == 0
    assert S.socket_ids_bytes(1, 1, 10, 64, 10) == 64 * 80     # packed: 80 bytes a key
    assert S.socket_ids_bytes(1, 1, 10, 60, 9) == 64 * 80
    assert S.socket_ids_bytes(1, 1, 10, 32, 10) == 64 * 16 * 4  # two-byte cells
    assert S.socket_ids_bytes(1, 1, 10, 128, 8) == 64 * 16 * 8
