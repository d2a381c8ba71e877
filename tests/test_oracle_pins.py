"""Pins for the CPU oracle: it is checked against things other than itself.

* hand-derived worked examples (tests/golden/worked_examples.json),
* closed forms and algebraic identities (product of sigmoids, P = 1),
* limits the paper states (tau -> 0 gives hard LSH, SOCKET Sec. 5.3),
* library routines (torch's scaled_dot_product_attention in float64),
* brute-force loops on tiny inputs (oracle/brute.py),
* a statistical closed form (the angular collision probability
  (1 - theta/pi)^P of SOCKET App. B.2) by Monte Carlo.

Every check is a function of the implementation under test, so the
mutation tests at the bottom can plant a mistake in a copy of the oracle
and show that at least one pin catches it.
"""
from __future__ import annotations

import json
import math
import os
import types

import numpy as np
import pytest
from scipy.special import expit

from oracle import brute
from oracle import socket_oracle as SO
from soft_lsh_token_amd.inputs import make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _qexpr(exprs):
    return np.array([eval(e, {"log": math.log}) for e in exprs], dtype=np.float64)


def impl(**over):
    """The oracle as a namespace, optionally with functions replaced."""
    ns = types.SimpleNamespace(
        hash_keys=SO.hash_keys, value_norms=SO.value_norms, soft_tables=SO.soft_tables,
        scores=SO.scores, topk=SO.topk, select=SO.select, sparse_attention=SO.sparse_attention,
        hard_collision_scores=SO.hard_collision_scores, soft_counts=SO.soft_counts,
        sampling_distribution=SO.sampling_distribution, soft_attention=SO.soft_attention,
        inverse_cdf=SO.inverse_cdf, sample_estimate=SO.sample_estimate)
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


# ----------------------------------------------------------------------------- checks

def check_golden_hash(so):
    g = _golden()["hash"]
    ids, _ = so.hash_keys(np.array(g["keys"], float), np.array(g["W"], float), g["L"], g["P"])
    assert ids.tolist() == g["ids"]


def check_golden_soft_table(so):
    g = _golden()["soft_table"]
    p = so.soft_tables(_qexpr(g["q_expr"]), np.array(g["W"], float), g["L"], g["P"], g["tau"])
    np.testing.assert_allclose(p[0], g["p"], rtol=1e-13, atol=0)


def check_golden_score_topk(so):
    g = _golden()["score_topk"]
    W = np.array(g["W"], float)
    q = _qexpr(g["q_expr"])
    keys = np.array(g["keys"], float)
    vals = np.array(g["values"], float)
    for reps in (1, 2):  # L=2 with the same planes twice doubles every score
        Wr = np.concatenate([W] * reps, axis=0)
        ids, _ = so.hash_keys(keys[None, None], Wr, reps, g["P"])
        vn = so.value_norms(vals[None, None])
        t = so.soft_tables(q[None, None], Wr, reps, g["P"], g["tau"])
        s = so.scores(t, ids, vn)[0, 0]
        np.testing.assert_allclose(s, reps * np.array(g["scores"]), rtol=1e-13)
        assert so.topk(s, 2).tolist() == g["top2"]
        assert so.topk(s, 1).tolist() == g["top1"]


def check_golden_attention(so):
    g = _golden()["attention"]
    out = so.sparse_attention(_qexpr(g["q_expr"]), np.array(g["keys"], float),
                              np.array(g["values"], float), np.arange(2), g["scale"])
    np.testing.assert_allclose(out, g["out"], rtol=1e-13)


def check_tables_sum_to_one(so):
    rng = np.random.default_rng(1)
    for P in (1, 3, 8):
        W = rng.standard_normal((5 * P, 16))
        q = rng.standard_normal((3, 16))
        for tau in (0.3, 0.5, 2.0):
            p = so.soft_tables(q, W, 5, P, tau)
            assert p.shape == (3, 5, 1 << P)
            assert (p >= 0).all()
            np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)


def check_product_of_sigmoids(so):
    """softmax over corners == prod_j sigmoid(2 c_j(b) u_j / tau) (algebraic identity)."""
    rng = np.random.default_rng(2)
    L, P, d = 4, 6, 32
    W = rng.standard_normal((L * P, d))
    q = rng.standard_normal(d) * 0.3
    tau = 0.5
    p = so.soft_tables(q, W, L, P, tau)
    u = (W @ q).reshape(L, P)
    for l in range(L):
        for b in range(1 << P):
            c = np.array([1.0 if (b >> j) & 1 else -1.0 for j in range(P)])
            expect = np.prod(expit(2.0 * c * u[l] / tau))
            assert abs(p[l, b] - expect) <= 1e-13 * max(expect, 1e-300) + 1e-300


def check_tau_to_zero(so):
    """tau -> 0: one-hot at the query's hard bucket; scores -> ||v|| * collision count."""
    rng = np.random.default_rng(3)
    L, P, d, n = 6, 4, 16, 40
    for _ in range(20):
        W = rng.standard_normal((L * P, d))
        q = rng.standard_normal(d)
        if np.abs(W @ q).min() > 1e-2:
            break
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    tau = 1e-4
    p = so.soft_tables(q, W, L, P, tau)
    qb = [brute.bucket_id(W, q, l, P) for l in range(L)]
    for l in range(L):
        assert p[l, qb[l]] == pytest.approx(1.0, abs=1e-12)
        others = np.delete(p[l], qb[l])
        assert others.max() < 1e-12
    ids, _ = so.hash_keys(K[None, None], W, L, P)
    vn = so.value_norms(V[None, None])
    s = so.scores(p[None, None], ids, vn)[0, 0]
    hard = np.array([math.sqrt(sum(x * x for x in V[i])) *
                     sum(brute.bucket_id(W, K[i], l, P) == qb[l] for l in range(L))
                     for i in range(n)])
    np.testing.assert_allclose(s, hard, rtol=1e-10, atol=1e-12)


def check_tau_to_inf_and_p1(so):
    rng = np.random.default_rng(4)
    W = rng.standard_normal((3 * 5, 8))
    q = rng.standard_normal(8)
    p = so.soft_tables(q, W, 3, 5, 1e9)
    np.testing.assert_allclose(p, 1.0 / 32, rtol=1e-6)
    # P = 1: p(bit 1) = sigmoid(2u/tau), p(bit 0) = sigmoid(-2u/tau)
    W1 = rng.standard_normal((7, 8))
    for tau in (0.3, 1.0):
        p1 = so.soft_tables(q, W1, 7, 1, tau)
        u = W1 @ q
        np.testing.assert_allclose(p1[:, 1], expit(2 * u / tau), rtol=1e-13)
        np.testing.assert_allclose(p1[:, 0], expit(-2 * u / tau), rtol=1e-13)


def check_brute_force(so):
    """Vectorised oracle == pure-Python loops on tiny GQA inputs with ragged lengths."""
    rng = np.random.default_rng(5)
    B, Hq, Hkv, n, d, L, P, tau = 2, 4, 2, 24, 6, 3, 3, 0.5
    W = rng.standard_normal((L * P, d))
    K = rng.standard_normal((B, Hkv, n, d))
    V = rng.standard_normal((B, Hkv, n, d))
    q = rng.standard_normal((B, Hq, d))
    lens = [24, 17]
    ids, _ = so.hash_keys(K, W, L, P)
    vn = so.value_norms(V)
    t = so.soft_tables(q, W, L, P, tau)
    s = so.scores(t, ids, vn, lens)
    group = Hq // Hkv
    for b in range(B):
        for h in range(Hkv):
            for i in range(n):
                assert [brute.bucket_id(W, K[b, h, i], l, P) for l in range(L)] == \
                    ids[b, h, i].tolist()
        for g in range(Hq):
            for l in range(L):
                np.testing.assert_allclose(t[b, g, l],
                                           brute.bucket_distribution(W, q[b, g], l, P, tau),
                                           rtol=1e-12)
            h = g // group
            ref = [brute.score(W, q[b, g], K[b, h, i], V[b, h, i], L, P, tau)
                   for i in range(lens[b])]
            np.testing.assert_allclose(s[b, g, :lens[b]], ref, rtol=1e-12)
            assert np.isnan(s[b, g, lens[b]:]).all()
            for k in (1, 5, lens[b]):
                sel = so.topk(s[b, g], k, lens[b])
                assert sel.tolist() == brute.top_k(ref, k)
                out = so.sparse_attention(q[b, g], K[b, h], V[b, h], sel, 1 / math.sqrt(d))
                bo = brute.attention(q[b, g], [K[b, h, i] for i in sel],
                                     [V[b, h, i] for i in sel], 1 / math.sqrt(d))
                np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-14)


def check_topk_ties_and_sort(so):
    s = np.array([3.0, 5.0, 5.0, 1.0, 5.0, 2.0, 3.0])
    assert so.topk(s, 2).tolist() == [1, 2]          # equal scores: lower index first
    assert so.topk(s, 4).tolist() == [0, 1, 2, 4]
    assert so.topk(s, 3, n=4).tolist() == [0, 1, 2]  # only the first n keys compete
    rng = np.random.default_rng(6)
    x = rng.standard_normal(1000)
    sel = so.topk(x, 100)
    assert len(set(sel.tolist())) == 100
    rest = np.setdiff1d(np.arange(1000), sel)
    assert x[sel].min() >= x[rest].max()


def check_select_sink_window(so):
    """Selection with always-attended sink and local-window keys (Sec. 6 setup)
    against k-fold arg max loops, plus the cases it reduces to."""
    rng = np.random.default_rng(9)
    for trial in range(200):
        n = int(rng.integers(0, 40))
        k = int(rng.integers(0, 12))
        sink, window = int(rng.integers(0, 8)), int(rng.integers(0, 8))
        s = rng.integers(0, 6, size=n).astype(float)     # many equal scores
        sel = so.select(s, k, n, sink, window)
        assert sel.tolist() == brute.select(s.tolist(), k, sink, window), (n, k, sink, window)
        assert len(sel) == min(n, k + sink + window)
        assert len(set(sel.tolist())) == len(sel)
    s = np.array([3.0, 5.0, 5.0, 1.0, 5.0, 2.0, 3.0, 4.0])
    assert so.select(s, 3, None, 0, 0).tolist() == so.topk(s, 3).tolist()
    assert so.select(s, 0, None, 2, 1).tolist() == [0, 1, 7]       # k = 0: forced keys only
    assert so.select(s, 2, None, 2, 1).tolist() == [0, 1, 2, 4, 7]  # 5, 5 of the rest; tie -> 2, 4
    assert so.select(s, 1, 6, 1, 2).tolist() == [0, 1, 4, 5]        # only the first n keys count
    assert so.select(s, 3, None, 5, 5).tolist() == list(range(8))   # sink + window cover all


def check_hard_scores_brute(so):
    """Hard-LSH scores (value norm x number of tables where the key shares the
    query's bucket) against loops over tables, on GQA inputs with ragged lengths."""
    rng = np.random.default_rng(10)
    B, Hq, Hkv, n, d = 2, 4, 2, 30, 6
    for L, P in ((7, 2), (3, 4), (12, 1)):
        W = rng.standard_normal((L * P, d))
        K = rng.standard_normal((B, Hkv, n, d))
        V = rng.standard_normal((B, Hkv, n, d))
        q = rng.standard_normal((B, Hq, d))
        lens = [30, 19]
        ids, _ = so.hash_keys(K, W, L, P)
        s = so.hard_collision_scores(q, W, ids, so.value_norms(V), L, P, lens)
        for b in range(B):
            for g in range(Hq):
                h = g // (Hq // Hkv)
                qb = [brute.bucket_id(W, q[b, g], l, P) for l in range(L)]
                for i in range(lens[b]):
                    hits = sum(brute.bucket_id(W, K[b, h, i], l, P) == qb[l] for l in range(L))
                    vn = math.sqrt(sum(float(x) * float(x) for x in V[b, h, i]))
                    assert s[b, g, i] == pytest.approx(vn * hits, rel=1e-12, abs=1e-300)
                assert np.isnan(s[b, g, lens[b]:]).all()


def _sampling_case(seed=11, n=40, L=5, P=3, d=6):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((L * P, d))
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d)) * rng.lognormal(0, 0.5, size=(n, 1))
    q = rng.standard_normal(d)
    return W, K, V, q, L, P


def check_sampling_law_brute(so):
    """Soft counts, the value-aware law and the inverse-CDF draw against loops."""
    W, K, V, q, L, P = _sampling_case()
    tau = 0.5
    tab = so.soft_tables(q, W, L, P, tau)
    ids, _ = so.hash_keys(K, W, L, P)
    vn = so.value_norms(V)
    sc = so.soft_counts(tab, ids)
    for i in range(len(K)):
        ref = brute.score(W, q, K[i], V[i], L, P, tau) / math.sqrt(sum(x * x for x in V[i]))
        assert sc[i] == pytest.approx(ref, rel=1e-12)
    p, S1, a = so.sampling_distribution(tab, ids, vn)
    total = sum(sc)
    S1_ref = sum(sc[i] / total * vn[i] for i in range(len(K)))
    assert S1 == pytest.approx(S1_ref, rel=1e-12)
    for i in range(len(K)):
        assert a[i] == pytest.approx(sc[i] / total, rel=1e-12)
        assert p[i] == pytest.approx(sc[i] / total * vn[i] / S1_ref, rel=1e-12)
    pz = np.array([0.0, 0.25, 0.0, 0.5, 0.25, 0.0])
    for u, want in [(0.0, 1), (0.2499, 1), (0.25, 3), (0.7499, 3), (0.75, 4), (0.99999, 4)]:
        acc, got = 0.0, None
        for j, pj in enumerate(pz):
            acc += pj
            if acc > u:
                got = j
                break
        assert got == want
        assert int(so.inverse_cdf(pz, np.array([u]))[0]) == want


def check_sampling_unbiased_identity(so):
    """E[X | W] over the law equals the soft-attention output y (Theorem 3, part 1),
    summed exactly over every key instead of sampled."""
    W, K, V, q, L, P = _sampling_case(seed=12)
    tab = so.soft_tables(q, W, L, P, 0.4)
    ids, _ = so.hash_keys(K, W, L, P)
    vn = so.value_norms(V)
    p, S1, a = so.sampling_distribution(tab, ids, vn)
    assert p.sum() == pytest.approx(1.0, rel=1e-12)
    # X(j) as the estimator forms it: run it with all the mass of one draw on key j
    ex = np.zeros(V.shape[1])
    for j in range(len(K)):
        lo = float(np.cumsum(p)[j] - p[j])
        u = (lo + 0.5 * p[j]) if p[j] > 0 else None
        if u is None:
            continue
        T, J = so.sample_estimate(tab, ids, V, np.array([u]))
        assert int(J[0]) == j
        ex += p[j] * T
    y = so.soft_attention(tab, ids, V)
    np.testing.assert_allclose(ex, y, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(y, (a[:, None] * V).sum(0), rtol=1e-12)


def check_sampling_concentration(so):
    """Theorem 3, part 2: with probability >= 1 - delta,
    ||T(q) - y|| <= ||V||_2 sqrt(8 log(2/delta) / M); 20 seeded draws of M = 2000."""
    W, K, V, q, L, P = _sampling_case(seed=13, n=300, L=8, P=4, d=16)
    tab = so.soft_tables(q, W, L, P, 0.5)
    ids, _ = so.hash_keys(K, W, L, P)
    y = so.soft_attention(tab, ids, V)
    M, delta = 2000, 1e-3
    bound = np.linalg.norm(V, 2) * math.sqrt(8 * math.log(2 / delta) / M)
    rng = np.random.default_rng(14)
    errs = []
    for _ in range(20):
        T, _ = so.sample_estimate(tab, ids, V, rng.random(M))
        errs.append(float(np.linalg.norm(T - y)))
    assert max(errs) <= bound, (max(errs), bound)
    # and the error shrinks like M^-1/2: mean error at M is within a factor of the bound
    assert np.mean(errs) < 0.25 * bound


def check_attention_library(so):
    """k = n equals dense softmax attention (torch SDPA, float64 CPU); k = 1 returns v[argmax]."""
    import torch
    rng = np.random.default_rng(7)
    n, d = 50, 16
    q = rng.standard_normal(d)
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    out = so.sparse_attention(q, K, V, np.arange(n), 1 / math.sqrt(d))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None], torch.from_numpy(K)[None, None],
        torch.from_numpy(V)[None, None])[0, 0, 0].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    i = 13
    np.testing.assert_allclose(so.sparse_attention(q, K, V, np.array([i]), 0.125), V[i],
                               rtol=1e-15)


# ----------------------------------------------------------------------------- the pins

ALL_CHECKS = [check_golden_hash, check_golden_soft_table, check_golden_score_topk,
              check_golden_attention, check_tables_sum_to_one, check_product_of_sigmoids,
              check_tau_to_zero, check_tau_to_inf_and_p1, check_brute_force,
              check_topk_ties_and_sort, check_select_sink_window, check_hard_scores_brute,
              check_sampling_law_brute, check_sampling_unbiased_identity,
              check_sampling_concentration, check_attention_library]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(impl())


def test_collision_probability_statistical():
    """Per-table hard collision rate over random planes -> (1 - theta/pi)^P (SOCKET App. B.2)."""
    rng = np.random.default_rng(8)
    d, P, T = 16, 4, 20000
    q = rng.standard_normal(d)
    k = q + 0.8 * rng.standard_normal(d)
    theta = math.acos(q @ k / (np.linalg.norm(q) * np.linalg.norm(k)))
    W = rng.standard_normal((T * P, d))
    both = np.stack([q, k])
    ids, _ = SO.hash_keys(both, W, T, P)
    rate = float((ids[0] == ids[1]).mean())
    expect = (1 - theta / math.pi) ** P
    sigma = math.sqrt(expect * (1 - expect) / T)
    assert abs(rate - expect) < 4 * sigma, (rate, expect, sigma)


def test_memory_arithmetic():
    """~600 bits/token = L*P at P=10, L=60 (SOCKET Sec. 1, App. A.1); ~15% over the KV cache
    (Sec. 7) when ids + one fp32 norm are kept per KV head of d=128 bf16 K and V."""
    L, P, d = 60, 10, 128
    assert L * P == 600
    overhead = (L * P + 32) / (2 * d * 16)
    assert 0.14 < overhead < 0.16


def test_decode_step_matches_parts():
    """decode_step composes the parts on a small shared-input workload (GQA, ragged)."""
    w = make_workload("c4", n=(40, 64), B=3, Hq=4, Hkv=2, L=4, P=3, d=8, k=0.25)
    r = SO.decode_step(w)
    group = w.Hq // w.Hkv
    for b in range(w.B):
        for g in range(w.Hq):
            h = g // group
            ref_s = [brute.score(w.W, w.q[b, g], w.K[b, h, i], w.V[b, h, i], w.L, w.P, w.tau)
                     for i in range(w.lens[b])]
            np.testing.assert_allclose(r["scores"][b, g, :w.lens[b]], ref_s, rtol=1e-11)
            assert r["idx"][(b, g)].tolist() == brute.top_k(ref_s, int(w.ks[b]))


# ----------------------------------------------------------------------------- planted mistakes

def _hash_ge(K, W, L, P):           # z == 0 would give bit 1
    z = (np.asarray(K, float) @ np.asarray(W, float).T).reshape(*np.shape(K)[:-1], L, P)
    return ((z >= 0) * (1 << np.arange(P))).sum(-1), z


def _hash_msb(K, W, L, P):          # plane j -> bit P-1-j
    z = (np.asarray(K, float) @ np.asarray(W, float).T).reshape(*np.shape(K)[:-1], L, P)
    return ((z > 0) * (1 << np.arange(P)[::-1])).sum(-1), z


def _tables_flipped(q, W, L, P, tau):   # corner sign flipped
    return SO.soft_tables(-np.asarray(q, float), W, L, P, tau)


def _tables_no_tau(q, W, L, P, tau):    # temperature dropped
    return SO.soft_tables(q, W, L, P, 1.0)


def _gqa_mod(tables, ids, vnorm, lens=None):
    B, Hq, L, _ = tables.shape
    Hkv, n = ids.shape[1], ids.shape[2]
    out = np.empty((B, Hq, n))
    for b in range(B):
        for g in range(Hq):
            h = g % Hkv
            out[b, g] = np.asarray(vnorm)[b, h] * tables[b, g][np.arange(L)[None], ids[b, h]].sum(-1)
            if lens is not None:
                out[b, g, int(lens[b]):] = np.nan
    return out


def _scores_no_norm(tables, ids, vnorm, lens=None):
    return SO.scores(tables, ids, np.ones_like(np.asarray(vnorm, float)), lens)


def _scores_mean(tables, ids, vnorm, lens=None):
    return SO.scores(tables, ids, vnorm, lens) / tables.shape[2]


def _topk_high_index(s, k, n=None):   # ties -> higher index
    s = np.asarray(s, float)
    n = len(s) if n is None else n
    order = np.argsort(-s[:n][::-1], kind="stable")
    return np.sort((n - 1 - order)[:k])


def _select_budget_shared(s, k, n=None, sink=0, window=0):   # top-k over all keys, then union
    s = np.asarray(s, float)
    n = len(s) if n is None else n
    forced = set(range(min(sink, n))) | set(range(max(n - window, 0), n))
    return np.array(sorted(forced | set(SO.topk(s, k, n).tolist())), dtype=np.int64)


def _select_window_shift(s, k, n=None, sink=0, window=0):    # window one key too early
    s = np.asarray(s, float)
    n = len(s) if n is None else n
    forced = np.zeros(n, bool)
    forced[:min(sink, n)] = True
    forced[max(n - window - 1, 0):max(n - 1, 0)] = True
    rest = np.nonzero(~forced)[0]
    picked = rest[np.argsort(-s[:n][rest], kind="stable")[:k]]
    return np.sort(np.concatenate([np.nonzero(forced)[0], picked]))


def _hard_any_plane(q, W, ids, vnorm, L, P, lens=None):   # counts plane agreements, not tables
    qids, _ = SO.hash_keys(np.asarray(q, float)[..., None, :], W, L, P)
    qids = qids[..., 0, :]
    B, Hq = qids.shape[:2]
    Hkv = ids.shape[1]
    out = np.empty((B, Hq, ids.shape[2]))
    for b in range(B):
        for g in range(Hq):
            h = g // (Hq // Hkv)
            same = ~((ids[b, h] ^ qids[b, g][None, :])[..., None] >> np.arange(P) & 1).astype(bool)
            out[b, g] = np.asarray(vnorm, float)[b, h] * same.sum(axis=(-1, -2))
            if lens is not None:
                out[b, g, int(lens[b]):] = np.nan
    return out


def _law_no_norm(tables_row, ids_rows, vnorm_row):     # draws by a~ only, X unchanged
    p, S1, a = SO.sampling_distribution(tables_row, ids_rows, vnorm_row)
    return a, S1, a


def _estimate_raw_v(tables_row, ids_rows, V_rows, u):    # X = v_J (no S_1 / ||v_J||)
    p, S1, _ = SO.sampling_distribution(tables_row, ids_rows, SO.value_norms(V_rows))
    J = SO.inverse_cdf(p, u)
    return np.asarray(V_rows, float)[J].mean(axis=0), J


def _icdf_left(p, u):                                    # boundary goes to the lower key
    cdf = np.cumsum(np.asarray(p, float))
    return np.minimum(np.searchsorted(cdf, np.asarray(u) * cdf[-1], side="left"), len(cdf) - 1)


def _attn_no_scale(q, K, V, idx, scale):
    return SO.sparse_attention(q, K, V, idx, 1.0)


def _attn_transposed(q, K, V, idx, scale):  # values gathered with the key matrix
    return SO.sparse_attention(q, K, K, idx, scale)


MUTANTS = {
    "hash_ge": dict(hash_keys=_hash_ge),
    "hash_msb": dict(hash_keys=_hash_msb),
    "tables_flipped": dict(soft_tables=_tables_flipped),
    "tables_no_tau": dict(soft_tables=_tables_no_tau),
    "scores_mod_gqa": dict(scores=_gqa_mod),
    "scores_no_norm": dict(scores=_scores_no_norm),
    "scores_mean": dict(scores=_scores_mean),
    "topk_high_index": dict(topk=_topk_high_index),
    "select_budget_shared": dict(select=_select_budget_shared),
    "select_window_shift": dict(select=_select_window_shift),
    "hard_any_plane": dict(hard_collision_scores=_hard_any_plane),
    "law_no_norm": dict(sampling_distribution=_law_no_norm),
    "estimate_raw_v": dict(sample_estimate=_estimate_raw_v),
    "icdf_left": dict(inverse_cdf=_icdf_left),
    "attn_no_scale": dict(sparse_attention=_attn_no_scale),
    "attn_transposed": dict(sparse_attention=_attn_transposed),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    so = impl(**MUTANTS[name])
    failed = []
    for check in ALL_CHECKS:
        try:
            check(so)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
