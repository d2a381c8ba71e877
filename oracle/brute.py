"""Pure-Python loop versions of the SOCKET steps -- TEST INFRASTRUCTURE ONLY.

Written independently of the vectorised oracle (no numpy arithmetic, only
``math``), for tiny shapes, so that the two can be checked against each
other.  Definitions follow "SOCKET: SOft Collision Kernel EsTimator for
Sparse Attention", Sec. 4.1 (Algorithms 1-3) and Appendix B.2 (bucket ID =
sign pattern of W^(l) k).  The per-bucket probability is computed here by
enumerating the 2^P buckets and normalising the exponentiated corner
logits directly.
"""
from __future__ import annotations

import math


def dot(a, b):
    s = 0.0
    for x, y in zip(a, b):
        s += float(x) * float(y)
    return s


def bucket_id(W, k, l, P):
    """Sign pattern of table l's P planes applied to k; plane j -> bit j."""
    b = 0
    for j in range(P):
        if dot(W[l * P + j], k) > 0.0:
            b |= 1 << j
    return b


def bucket_distribution(W, q, l, P, tau):
    """p(b) for b in 0..2^P-1, by explicit enumeration of the buckets."""
    u = [dot(W[l * P + j], q) for j in range(P)]
    logits = []
    for b in range(1 << P):
        x = 0.0
        for j in range(P):
            sign = 1.0 if (b >> j) & 1 else -1.0
            x += sign * u[j]
        logits.append(x / tau)
    m = max(logits)
    e = [math.exp(x - m) for x in logits]
    z = sum(e)
    return [x / z for x in e]


def score(W, q, k, v, L, P, tau):
    """||v|| * sum over tables of the query's mass on k's bucket."""
    vn = math.sqrt(sum(float(x) * float(x) for x in v))
    total = 0.0
    for l in range(L):
        p = bucket_distribution(W, q, l, P, tau)
        total += p[bucket_id(W, k, l, P)]
    return vn * total


def top_k(s, k):
    """Indices of the k largest scores; among equal scores the lower index wins."""
    chosen = []
    remaining = list(range(len(s)))
    for _ in range(k):
        best = remaining[0]
        for i in remaining[1:]:
            if s[i] > s[best]:
                best = i
        chosen.append(best)
        remaining.remove(best)
    return sorted(chosen)


def select(s, k, sink, window):
    """Attended keys of one head: the first `sink` and last `window` keys, plus
    the k best of the others (k-fold arg max, lower index first on equal
    scores)."""
    n = len(s)
    forced = [i for i in range(n) if i < sink or i >= n - window]
    others = [i for i in range(n) if i not in forced]
    chosen = []
    for _ in range(min(k, len(others))):
        best = None
        for i in others:
            if i in chosen:
                continue
            if best is None or s[i] > s[best]:
                best = i
        chosen.append(best)
    return sorted(forced + chosen)


def attention(q, Ks, Vs, scale):
    logits = [dot(kk, q) * scale for kk in Ks]
    m = max(logits)
    e = [math.exp(x - m) for x in logits]
    z = sum(e)
    d = len(Vs[0])
    out = [0.0] * d
    for w, v in zip(e, Vs):
        for t in range(d):
            out[t] += (w / z) * float(v[t])
    return out
