"""Host-side view of the bucket-ID cache layout (include/socket_lsh.h).

The HIP library stores the bucket IDs tiled in groups of 64 keys, each key's
IDs cut into 16 words of TL bytes, in a diagonal order (see the header).
These helpers convert between that layout and a plain [B, Hkv, n, L] uint8
array.  They are index permutations only (for inspection, tests, and
loading IDs computed elsewhere); nothing of the method is computed here.
"""
from __future__ import annotations

import numpy as np


def word_bytes(L: int) -> int:
    return 1 if L <= 16 else 2 if L <= 32 else 4 if L <= 64 else 8


def key_bytes(L: int) -> int:
    return 16 * word_bytes(L)


def groups(n_cap: int) -> int:
    return (n_cap + 63) // 64


def ids_shape(B: int, Hkv: int, n_cap: int, L: int) -> tuple:
    """Shape of the cache as a uint8 tensor: [B, Hkv, groups, 64 * key_bytes]."""
    return (B, Hkv, groups(n_cap), 64 * key_bytes(L))


def _perm(L: int):
    """Byte position inside a 64-key group of (key t, word w, byte b)."""
    TL = word_bytes(L)
    t = np.arange(64)[:, None, None]
    w = np.arange(16)[None, :, None]
    b = np.arange(TL)[None, None, :]
    kg, x = t // 16, t % 16
    R = 16 // TL
    r = (x - w) % 16
    slot = (r // R) * 64 * R + (16 * kg + w) * R + r % R
    return slot * TL + b          # [64, 16, TL]


def unpack(tiled: np.ndarray, L: int, n: int | None = None) -> np.ndarray:
    """[B, Hkv, G, 64*key_bytes] tiled cache -> [B, Hkv, n, L] bucket IDs."""
    B, Hkv, G, gb = tiled.shape
    pos = _perm(L).reshape(64, -1)                           # [64, 16*TL]
    keys = tiled[:, :, :, pos]                               # [B, Hkv, G, 64, 16*TL]
    keys = keys.reshape(B, Hkv, G * 64, -1)[..., :L]
    return keys if n is None else keys[:, :, :n]


def pack(ids: np.ndarray, n_cap: int | None = None) -> np.ndarray:
    """[B, Hkv, n, L] bucket IDs -> tiled cache (keys past n and tables past L are 0)."""
    B, Hkv, n, L = ids.shape
    n_cap = n if n_cap is None else n_cap
    G, TL = groups(n_cap), word_bytes(L)
    full = np.zeros((B, Hkv, G * 64, 16 * TL), dtype=np.uint8)
    full[:, :, :n, :L] = ids
    out = np.zeros((B, Hkv, G, 64 * 16 * TL), dtype=np.uint8)
    pos = _perm(L).reshape(64, -1)
    out[:, :, :, pos] = full.reshape(B, Hkv, G, 64, 16 * TL)
    return out
