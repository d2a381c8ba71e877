"""CPU oracle for the SOCKET decode path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its Python
binding) never calls it, and it shares no code with that path.

It is a plain, slow, float64 implementation of the method described in
"SOCKET: SOft Collision Kernel EsTimator for Sparse Attention"
(paperpeel.com/paper/2602.06283), Section 4.1 "The Final Algorithm":

* Algorithm 1, key hashing at prefill: every key gets one bucket per hash
  table from L random projections; bucket IDs are cached together with the
  value-vector norms (Sec. 4.1; Sec. 1 "Key Idea" names the value-norm
  weighting).  A bucket ID is the sign pattern of W^(l) k (Appendix B.2).
* Algorithm 2, query soft hashing at decode: the query induces a
  probability distribution over the buckets of each table; a key's score
  aggregates the probability mass of its own buckets (Sec. 4.1, eq. (3),
  which the extracted page lost).  The Chinese technical summary of the
  same paper (gist.science) says the distribution is a temperature
  controlled softmax of the query's projections on the random hyperplanes.
* Algorithm 3: deterministic top-k of the soft scores, then exact attention
  over that subset (Sec. 4.1; Sec. 2 "Related Work" contrasts this with
  MagicPIG's sampling).

Readings where the pages are silent (each listed in the design notes):

* Soft hashing (eq. (3) lost): the distribution over the 2^P buckets b of
  table l is softmax_b(<c(b), u_l> / tau) with u_l = W^(l) q and the
  hypercube corner c_j(b) = +1 if bit j of b is set, else -1.  Its argmax
  is the hard bucket sign(W^(l) q), so tau -> 0 recovers hard LSH as the
  paper states in Sec. 5.3.
* Score: s_i = ||v_i||_2 * sum_l p_l(b_l(i) | q) (a sum over tables, not a
  mean; a mean would not change the ranking).
* Bit j of a bucket ID is plane j of its table; z == 0 gives bit 0.
* Bucket IDs belong to KV heads and are shared by the GQA query heads that
  read that KV head (query head g reads KV head g // (Hq / Hkv)).
* Top-k ties go to the lower key index.  Attention uses scale 1/sqrt(d).
* Sink and local-window tokens (Sec. 6 setup: a small number, 64 or 128,
  always attended): the first `sink` and the last `window` keys of the
  sequence are always selected, and the top-k budget goes to the other
  keys, so a head attends min(n, k + sink + window) distinct keys.

Every input is taken as given (already rounded to its storage dtype) and
promoted to float64.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "hash_keys", "value_norms", "projections", "soft_tables", "scores", "topk", "select",
    "sparse_attention", "decode_step", "hard_collision_scores", "soft_counts",
    "sampling_distribution", "soft_attention", "inverse_cdf", "sample_estimate",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def hash_keys(K, W, L: int, P: int):
    """Algorithm 1 (SOCKET Sec. 4.1; bucket = sign pattern, App. B.2).

    K: [..., n, d]; W: [L*P, d], rows l*P .. l*P+P-1 are table l's planes.
    Returns (ids [..., n, L] int64, z [..., n, L, P] float64) where z are
    the projections whose signs give the bits.
    """
    K = _f64(K)
    W = _f64(W)
    z = K @ W.T                                   # [..., n, L*P]
    z = z.reshape(*z.shape[:-1], L, P)
    bits = (z > 0).astype(np.int64)               # z == 0 -> bit 0
    weights = (np.int64(1) << np.arange(P, dtype=np.int64))
    ids = (bits * weights).sum(axis=-1)           # [..., n, L]
    return ids, z


def value_norms(V):
    """Cached value-vector norms ||v_i||_2 (SOCKET Sec. 1 "Key Idea", Sec. 4.1)."""
    V = _f64(V)
    return np.sqrt((V * V).sum(axis=-1))


def projections(q, W, L: int, P: int):
    """u[..., l, j] = <W[l*P + j], q> in float64."""
    q = _f64(q)
    W = _f64(W)
    u = q @ W.T
    return u.reshape(*u.shape[:-1], L, P)


def _corners(P: int) -> np.ndarray:
    """c[b, j] = +1 if bit j of b is set else -1, for b in [0, 2^P)."""
    b = np.arange(1 << P)[:, None]
    j = np.arange(P)[None, :]
    return np.where((b >> j) & 1, 1.0, -1.0)


def soft_tables(q, W, L: int, P: int, tau: float):
    """Algorithm 2's per-table bucket distribution (SOCKET Sec. 4.1).

    Softmax over the 2^P buckets of the corner logits <c(b), u_l> / tau.
    Returns p[..., l, b], float64, each row summing to one.
    """
    u = projections(q, W, L, P)                   # [..., L, P]
    x = (u @ _corners(P).T) / float(tau)          # [..., L, 2^P]
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def scores(tables, ids, vnorm, lens=None):
    """Soft-count scores s_i = ||v_i|| * sum_l p_l[b_l(i)] (SOCKET Sec. 4.1, Sec. 1).

    tables: [B, Hq, L, 2^P]; ids: [B, Hkv, n, L]; vnorm: [B, Hkv, n].
    Query head g reads KV head g // (Hq / Hkv).  Positions at or beyond
    lens[b] are set to NaN (they are not keys of that sequence).
    Returns [B, Hq, n] float64.
    """
    tables = _f64(tables)
    vnorm = _f64(vnorm)
    B, Hq, L, _ = tables.shape
    Hkv, n = ids.shape[1], ids.shape[2]
    group = Hq // Hkv
    out = np.empty((B, Hq, n), dtype=np.float64)
    lidx = np.arange(L)[None, :]
    for b in range(B):
        for g in range(Hq):
            h = g // group
            mass = tables[b, g][lidx, ids[b, h]]      # [n, L]
            out[b, g] = vnorm[b, h] * mass.sum(axis=-1)
            if lens is not None:
                out[b, g, int(lens[b]):] = np.nan
    return out


def hard_collision_scores(q, W, ids, vnorm, L: int, P: int, lens=None):
    """tau -> 0 limit: ||v_i|| * #{l : b_l(i) == sign pattern of W^(l) q} (Sec. 5.3)."""
    qids, _ = hash_keys(_f64(q)[..., None, :], W, L, P)   # [B, Hq, 1, L]
    qids = qids[..., 0, :]
    B, Hq = qids.shape[:2]
    Hkv, n = ids.shape[1], ids.shape[2]
    group = Hq // Hkv
    out = np.empty((B, Hq, n))
    for b in range(B):
        for g in range(Hq):
            h = g // group
            out[b, g] = _f64(vnorm)[b, h] * (ids[b, h] == qids[b, g][None, :]).sum(axis=-1)
            if lens is not None:
                out[b, g, int(lens[b]):] = np.nan
    return out


def topk(s, k: int, n: int | None = None) -> np.ndarray:
    """Algorithm 3: the k highest scores among the first n keys; ties -> lower index.

    Returns the selected key indices sorted ascending (the set is what the
    method defines; the order is not part of it).
    """
    s = _f64(s)
    if n is None:
        n = s.shape[-1]
    order = np.argsort(-s[:n], kind="stable")
    return np.sort(order[:k])


def select(s, k: int, n: int | None = None, sink: int = 0, window: int = 0) -> np.ndarray:
    """Algorithm 3's selection with always-attended sink and local-window tokens
    (Sec. 6 setup).  Keys [0, sink) and [n - window, n) are always taken; the
    k highest scores among the remaining keys are added (ties -> lower index).

    Returns the attended key indices sorted ascending.
    """
    s = _f64(s)
    if n is None:
        n = s.shape[-1]
    forced = np.zeros(n, dtype=bool)
    forced[:min(sink, n)] = True
    forced[max(n - window, 0):] = True
    rest = np.nonzero(~forced)[0]
    order = np.argsort(-s[rest], kind="stable")        # stable: lower index first on ties
    picked = rest[order[:max(int(k), 0)]]
    return np.sort(np.concatenate([np.nonzero(forced)[0], picked]))


def sparse_attention(q, K, V, idx, scale: float):
    """Exact softmax attention of one query over the selected keys (SOCKET Sec. 2, 4.1).

    q: [d]; K, V: [n, d]; idx: selected indices.  Returns [d] float64.
    """
    q = _f64(q)
    Ks = _f64(K)[idx]
    Vs = _f64(V)[idx]
    logits = (Ks @ q) * float(scale)
    logits = logits - logits.max()
    a = np.exp(logits)
    a = a / a.sum()
    return a @ Vs


def soft_counts(tables_row, ids_rows):
    """L-table soft count of each key, s~_j = sum_l p_l(b_l(j) | q) (App. B.2).

    tables_row: [L, 2^P] of one query head; ids_rows: [n, L].  Returns [n].
    """
    t = _f64(tables_row)
    L = t.shape[0]
    return t[np.arange(L)[None, :], np.asarray(ids_rows, dtype=np.int64)].sum(axis=-1)


def sampling_distribution(tables_row, ids_rows, vnorm_row):
    """Value-aware sampling law of the estimator T(q) (Sec. 5.1; App. B.2):
    a~_j = s~_j / sum_i s~_i (soft attention weights) and
    p_j = a~_j ||v_j|| / S_1 with S_1 = sum_j a~_j ||v_j||.
    Returns (p [n], S_1, a~ [n])."""
    sc = soft_counts(tables_row, ids_rows)
    a = sc / sc.sum()
    wv = a * _f64(vnorm_row)
    S1 = wv.sum()
    return (wv / S1 if S1 > 0 else wv), S1, a


def soft_attention(tables_row, ids_rows, V_rows):
    """The soft-attention output y_{tau,L}(q) = sum_j a~_j v_j (App. B.2)."""
    _, _, a = sampling_distribution(tables_row, ids_rows, value_norms(V_rows))
    return a @ _f64(V_rows)


def inverse_cdf(p, u) -> np.ndarray:
    """Index drawn from the law p by the uniform u in [0, 1): the first j whose
    cumulative mass exceeds u (keys without mass are never drawn)."""
    cdf = np.cumsum(_f64(p))
    J = np.searchsorted(cdf, np.asarray(u, dtype=np.float64) * cdf[-1], side="right")
    last = int(np.nonzero(_f64(p) > 0)[0][-1])
    return np.minimum(J, last)


def sample_estimate(tables_row, ids_rows, V_rows, u):
    """The value-aware sampling estimator of Theorem 3 (Sec. 5.1, App. B.2):
    M draws J_m ~ p (value-aware law above), X_m = a~_J v_J / p_J =
    S_1 v_J / ||v_J||, T(q) = (1/M) sum_m X_m.  The draws come from the given
    uniforms u [M].  Returns (T [d], J [M])."""
    V = _f64(V_rows)
    vn = value_norms(V)
    p, S1, _ = sampling_distribution(tables_row, ids_rows, vn)
    if S1 <= 0:
        return np.zeros(V.shape[-1]), np.zeros(len(u), dtype=np.int64)
    J = inverse_cdf(p, u)
    X = S1 * V[J] / vn[J][:, None]
    return X.mean(axis=0), J


def decode_step(w, q=None, lens=None, ks=None, K=None, V=None, ids=None, vnorm=None,
                sink: int = 0, window: int = 0):
    """Hash (if needed), score, select and attend for every (sequence, query head).

    ``w`` is a workload from the shared input module.  Returns a dict with
    ids, vnorm, tables, scores, idx (list of arrays per (b, g)) and out
    [B, Hq, d].
    """
    q = w.q if q is None else q
    lens = w.lens if lens is None else lens
    ks = w.ks if ks is None else ks
    K = w.K if K is None else K
    V = w.V if V is None else V
    if ids is None:
        ids, _ = hash_keys(K, w.W, w.L, w.P)
    if vnorm is None:
        vnorm = value_norms(V)
    tables = soft_tables(q, w.W, w.L, w.P, w.tau)
    s = scores(tables, ids, vnorm, lens)
    group = w.Hq // w.Hkv
    out = np.empty((w.B, w.Hq, w.d))
    sel = {}
    for b in range(w.B):
        for g in range(w.Hq):
            idx = select(s[b, g], int(ks[b]), int(lens[b]), sink, window)
            sel[(b, g)] = idx
            out[b, g] = sparse_attention(q[b, g], K[b, g // group], V[b, g // group], idx,
                                         w.scale)
    return dict(ids=ids, vnorm=vnorm, tables=tables, scores=s, idx=sel, out=out)
