"""Host-side view of the bucket-ID cache layout (include/socket_lsh.h).

The HIP library stores the bucket IDs tiled in groups of 64 keys, each key's
IDs cut into 16 words of TL tables (cells of one byte for P <= 8, two
little-endian bytes for P = 9 or 10 with L <= 32, ten bits packed four to a
40-bit word for P = 9 or 10 with 33 <= L <= 64), in a diagonal order (see the
header).
These helpers convert between that layout and a plain [B, Hkv, n, L] array
(uint8 for one-byte cells, uint16 for two-byte cells).  They are index
permutations only (for inspection, tests, and loading IDs computed
elsewhere); nothing of the method is computed here.
"""
from __future__ import annotations

import numpy as np


def tables_per_word(L: int) -> int:
    return 1 if L <= 16 else 2 if L <= 32 else 4 if L <= 64 else 8


def cell_bytes(P: int) -> int:
    return 2 if P > 8 else 1


def word_bytes(L: int, P: int = 8) -> int:
    """Bytes of an unpacked word (packed words are 5 bytes, split in 4 + 1)."""
    return tables_per_word(L) * cell_bytes(P)


def packed(L: int, P: int) -> bool:
    """Ten-bit cells, four to a word: P = 9 or 10 with 33 <= L <= 64."""
    return P > 8 and tables_per_word(L) == 4


def key_bytes(L: int, P: int = 8) -> int:
    return 80 if packed(L, P) else 16 * word_bytes(L, P)


def groups(n_cap: int) -> int:
    return (n_cap + 63) // 64


def ids_shape(B: int, Hkv: int, n_cap: int, L: int, P: int = 8) -> tuple:
    """Shape of the cache as a uint8 tensor: [B, Hkv, groups, 64 * key_bytes]."""
    return (B, Hkv, groups(n_cap), 64 * key_bytes(L, P))


def _perm(L: int, P: int):
    """Byte position inside a 64-key group of (key t, word w, byte b of the word)."""
    WB = word_bytes(L, P)
    t = np.arange(64)[:, None, None]
    w = np.arange(16)[None, :, None]
    b = np.arange(WB)[None, None, :]
    kg, x = t // 16, t % 16
    R = 16 // WB
    r = (x - w) % 16
    slot = (r // R) * 64 * R + (16 * kg + w) * R + r % R
    return slot * WB + b          # [64, 16, WB]


def _cell_dtype(P: int):
    return np.dtype("<u2") if cell_bytes(P) == 2 else np.dtype(np.uint8)


def _perm_packed():
    """Packed words: byte positions inside a 64-key group of the 4 low bytes
    [64, 16, 4] and of the high byte [64, 16] of (key t, word w)."""
    t = np.arange(64)[:, None]
    w = np.arange(16)[None, :]
    kg, x = t // 16, t % 16
    r = (x - w) % 16
    lane = 16 * kg + w
    lo = (r // 4) * 1024 + lane * 16 + (r % 4) * 4
    hi = 4096 + lane * 16 + r
    return lo[:, :, None] + np.arange(4)[None, None, :], hi


def _unpack_packed(tiled: np.ndarray, L: int, n):
    B, Hkv, G, gb = tiled.shape
    lo_pos, hi_pos = _perm_packed()
    lo = tiled[:, :, :, lo_pos].astype(np.uint64)                  # [B, Hkv, G, 64, 16, 4]
    val = (lo[..., 0] | (lo[..., 1] << 8) | (lo[..., 2] << 16) | (lo[..., 3] << 24)
           | (tiled[:, :, :, hi_pos].astype(np.uint64) << 32))       # [B, Hkv, G, 64, 16]
    cells = (val[..., None] >> (10 * np.arange(4, dtype=np.uint64))) & 0x3FF
    keys = cells.reshape(B, Hkv, G * 64, 64)[..., :L].astype(np.uint16)
    return keys if n is None else keys[:, :, :n]


def _pack_packed(ids: np.ndarray, n_cap: int) -> np.ndarray:
    B, Hkv, n, L = ids.shape
    G = groups(n_cap)
    cells = np.zeros((B, Hkv, G * 64, 64), dtype=np.uint64)
    cells[:, :, :n, :L] = ids
    cells = cells.reshape(B, Hkv, G, 64, 16, 4)
    val = (cells << (10 * np.arange(4, dtype=np.uint64))).sum(axis=-1)  # disjoint bit fields
    out = np.zeros((B, Hkv, G, 64 * 80), dtype=np.uint8)
    lo_pos, hi_pos = _perm_packed()
    for b8 in range(4):
        out[:, :, :, lo_pos[..., b8]] = ((val >> np.uint64(8 * b8)) & 0xFF).astype(np.uint8)
    out[:, :, :, hi_pos] = ((val >> np.uint64(32)) & 0xFF).astype(np.uint8)
    return out


def unpack(tiled: np.ndarray, L: int, n: int | None = None, P: int = 8) -> np.ndarray:
    """[B, Hkv, G, 64*key_bytes] tiled cache -> [B, Hkv, n, L] bucket IDs."""
    if packed(L, P):
        return _unpack_packed(tiled, L, n)
    B, Hkv, G, gb = tiled.shape
    pos = _perm(L, P).reshape(64, -1)                        # [64, 16*WB]
    keys = np.ascontiguousarray(tiled[:, :, :, pos])         # [B, Hkv, G, 64, 16*WB]
    keys = keys.view(_cell_dtype(P)).reshape(B, Hkv, G * 64, -1)[..., :L]
    keys = keys.astype(np.uint16 if cell_bytes(P) == 2 else np.uint8)
    return keys if n is None else keys[:, :, :n]


def pack(ids: np.ndarray, n_cap: int | None = None, P: int = 8) -> np.ndarray:
    """[B, Hkv, n, L] bucket IDs -> tiled cache (keys past n and tables past L are 0)."""
    B, Hkv, n, L = ids.shape
    n_cap = n if n_cap is None else n_cap
    if packed(L, P):
        return _pack_packed(ids, n_cap)
    G, TL, WB = groups(n_cap), tables_per_word(L), word_bytes(L, P)
    cells = np.zeros((B, Hkv, G * 64, 16 * TL), dtype=_cell_dtype(P))
    cells[:, :, :n, :L] = ids
    full = cells.view(np.uint8).reshape(B, Hkv, G, 64, 16 * WB)
    out = np.zeros((B, Hkv, G, 64 * 16 * WB), dtype=np.uint8)
    out[:, :, :, _perm(L, P).reshape(64, -1)] = full
    return out


def codes_to_ids(codes: np.ndarray, L: int, P: int, n: int | None = None) -> np.ndarray:
    """Hard-mode codes [B, Hkv, words, n_cap] (any 32-bit integer dtype) ->
    [B, Hkv, n, L] bucket IDs: bit j of table l's ID is code bit l*P + j."""
    c = np.asarray(codes).astype(np.uint32)
    B, Hkv, nw, n_cap = c.shape
    n = n_cap if n is None else n
    c = c[..., :n]
    p = np.arange(L * P)
    bits = (c[:, :, p // 32, :] >> (p % 32)[None, None, :, None].astype(np.uint32)) & 1
    bits = bits.reshape(B, Hkv, L, P, n).astype(np.int64)
    ids = (bits << np.arange(P)[None, None, None, :, None]).sum(axis=3)
    return np.ascontiguousarray(ids.transpose(0, 1, 3, 2))
