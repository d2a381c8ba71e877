"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Per-kernel cases at small, ragged sizes; end-to-end
cases at the full workload sizes (32K, 128K, the 16-sequence ragged batch and
the prefill + 256-step decode loop), checked on every output or on sampled
heads where the oracle would take too long."""
from __future__ import annotations

import functools
import math

import numpy as np
import pytest
import torch

import gpu_cases as GC
from gpu_cases import DEV
from oracle import socket_oracle as SO
import soft_lsh_token_amd as S
from soft_lsh_token_amd.inputs import make_workload

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=2)
def workload(name, **kw):
    return make_workload(name, **dict(kw))



def sync():
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------- hashing

@pytest.mark.parametrize("case", [
    dict(name="c1"),                                   # fp32, generic path
    dict(name="c2", n=1000),                           # bf16 MFMA, ragged tail
    dict(name="c2", n=3000, L=32),                     # MFMA with 4 waves
    dict(name="c2", n=40),                             # few keys: generic bf16 path
    dict(name="c2", n=500, L=7, P=5, Hkv=2, Hq=4),     # odd shapes: generic path
    dict(name="c2", n=300, L=3, P=8, Hkv=2, Hq=2),
    dict(name="c4", n=(300, 900), B=3, Hkv=2, Hq=8),   # batch with different lengths
    dict(name="c2", n=1000, L=60, P=10),               # packed IDs, MFMA, 10 consumer waves
    dict(name="c2", n=700, L=64, P=10, Hkv=4, Hq=8),   # packed IDs, MFMA, 11 consumer waves
    dict(name="c2", n=500, L=20, P=10, Hkv=2, Hq=4),   # MFMA, two tables per word
    dict(name="c2", n=300, L=5, P=10, Hkv=2, Hq=2),    # MFMA, one table per word
    dict(name="c2", n=40, L=60, P=10),                 # few keys: generic, packed IDs
    dict(name="c2", n=300, L=5, P=9, Hkv=2, Hq=2),     # generic, one table per word
    dict(name="c2", n=700, L=40, P=9, Hkv=2, Hq=4),    # generic, packed nine-bit IDs
    dict(name="c1", L=60, P=10),                       # fp32: generic
], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_hash_parity(case):
    print("case", case, flush=True)
    w = make_workload(**case)
    d = GC.upload(w)
    ids, vn = GC.gpu_hash(w, d)
    sync()
    ids, vn = GC.ids_np(ids, w.L, P=w.P), vn.cpu().numpy()
    n_cap = w.n_cap
    for b in range(w.B):
        for h in range(w.Hkv):
            GC.check_ids(ids[b, h], w.K[b, h], w.W, w.L, w.P, n_cap)
            ref = SO.value_norms(w.V[b, h])
            np.testing.assert_allclose(vn[b, h], ref, rtol=2e-6)


def test_hash_full_c2_mfma():
    w = workload("c2")
    d = GC.upload(w)
    ids, vn = GC.gpu_hash(w, d)
    sync()
    ids, vn = GC.ids_np(ids, w.L, P=w.P), vn.cpu().numpy()
    band = 0
    for h in range(w.Hkv):
        band += GC.check_ids(ids[0, h], w.K[0, h], w.W, w.L, w.P, w.n_cap)
        np.testing.assert_allclose(vn[0, h], SO.value_norms(w.V[0, h]), rtol=2e-6)
    print("id bits inside the 1e-5 band:", band)


@pytest.mark.parametrize("case", [
    dict(name="c2", n=3000),                          # bf16 MFMA
    dict(name="c2", n=1000, L=60, P=10),              # packed IDs, MFMA
    dict(name="c1", n=700),                           # fp32, generic
    dict(name="c4", n=(30, 50), B=3, Hkv=2, Hq=4),    # few keys, generic bf16
], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_hash_outputs_apart(case):
    """IDs only (V = vnorm = None) and norms only (ids = None) give exactly the
    IDs and norms of the joint call, and leave the other cache untouched."""
    w = make_workload(**case)
    d = GC.upload(w)
    ids1, vn1 = GC.gpu_hash(w, d)
    pos0 = torch.zeros(w.B, dtype=torch.int32, device=DEV)
    count = int(w.lens.max())
    ids2 = S.alloc_ids(w.B, w.Hkv, w.n_cap, w.L, w.P, DEV)
    S.socket_hash_keys(d["K"], None, d["W"], ids2, None, pos0, count, w.L, w.P)
    vn2 = torch.full((w.B, w.Hkv, w.n_cap), -3.0, dtype=torch.float32, device=DEV)
    S.socket_hash_keys(None, d["V"], None, None, vn2, pos0, count, w.L, w.P)
    sync()
    assert torch.equal(ids1, ids2)
    live = torch.zeros_like(vn2, dtype=torch.bool)
    for b in range(w.B):
        live[b, :, :min(count, w.n_cap)] = True
    assert torch.equal(vn1[live], vn2[live])
    assert (vn2[~live] == -3.0).all()


@pytest.mark.parametrize("L,n", [(60, 1000), (20, 333), (5, 200), (37, 64)])
def test_hash_wide_pads_and_range(L, n):
    """P = 10 IDs (two-byte cells for L <= 32, packed ten-bit cells above): the
    hashed keys' cells of tables >= L (up to 16 words) are cleared, and keys
    past the hashed range keep their bytes."""
    w = make_workload("c2", n=n, L=L, P=10, Hkv=2, Hq=4, n_cap=n + 100)
    d = GC.upload(w)
    ids = S.alloc_ids(w.B, w.Hkv, w.n_cap, w.L, w.P, DEV).fill_(0xAB)
    untouched = GC.ids_np(ids, 16 * S.layout.tables_per_word(L), P=10)  # the fill, as cells
    ids, _ = GC.gpu_hash(w, d, ids=ids)
    sync()
    slots = 16 * S.layout.tables_per_word(L)
    full = GC.ids_np(ids, slots, P=10)            # every cell of every word
    for h in range(w.Hkv):
        GC.check_ids(full[0, h, :, :L], w.K[0, h], w.W, w.L, w.P, n)
    assert (full[0, :, :n, L:] == 0).all()
    assert (full[0, :, n:, :] == untouched[0, :, n:, :]).all()
    assert S.layout.packed(L, 10) or (untouched == 0xABAB).all()


@pytest.mark.parametrize("L,P", [(64, 8), (60, 10)])
def test_hash_append_rows_only(L, P):
    """count=1 at pos0=lens hashes exactly one new row per (sequence, head)."""
    w = make_workload("c4", n=(200, 600), B=2, Hkv=2, Hq=8, L=L, P=P)
    d = GC.upload(w)
    ids = S.alloc_ids(w.B, w.Hkv, w.n_cap, w.L, w.P, DEV).fill_(0xAB)
    fill = GC.ids_np(ids, w.L, w.n_cap, w.P)  # the fill byte, as cells of this layout
    vn = torch.full((w.B, w.Hkv, w.n_cap), -1.0, dtype=torch.float32, device=DEV)
    pos0 = d["lens"].clone()
    GC.gpu_hash(w, d, pos0=pos0, count=1, ids=ids, vnorm=vn)
    sync()
    ids, vn = GC.ids_np(ids, w.L, w.n_cap, w.P), vn.cpu().numpy()
    for b in range(w.B):
        p = int(w.lens[b])
        for h in range(w.Hkv):
            if p < w.n_cap:
                GC.check_ids(ids[b, h, p:p + 1], w.K[b, h, p:p + 1], w.W, w.L, w.P, 1)
                np.testing.assert_allclose(vn[b, h, p], SO.value_norms(w.V[b, h, p]), rtol=2e-6)
            mask = np.ones(w.n_cap, bool)
            mask[p:p + 1] = False
            assert (ids[b, h, mask] == fill[b, h, mask]).all()
            assert (vn[b, h, mask] == -1.0).all()


# ----------------------------------------------------------------------------- scoring + top-k

SCORE_CASES = [
    dict(name="c1"),
    dict(name="c2", n=5000),
    dict(name="c2", n=4500, Hq=8, Hkv=8),          # one query head per KV head
    dict(name="c2", n=4500, Hq=16, Hkv=8),         # two
    dict(name="c2", n=3333, L=32),
    dict(name="c2", n=2000, L=3, Hq=8, Hkv=2),     # L not a multiple of 4
    dict(name="c2", n=2000, L=20, P=5, Hq=8, Hkv=2),
    dict(name="c2", n=2000, tau=0.3),
    dict(name="c2", n=2500, L=100, Hq=8, Hkv=2),   # 8 tables a word: 1 full + 7 factored
    dict(name="c2", n=2000, L=128, Hq=8, Hkv=4),   # the same at two query heads per KV head
    dict(name="c4", n=(1000, 9000), B=4, k=0.02),  # ragged batch
    dict(name="c2", n=600, Hq=384, Hkv=96),        # 96 KV rows: more table blocks than fit at once
    # two-byte IDs (P = 9, 10): every table kept as two 32-entry halves
    dict(name="c2", n=5000, L=60, P=10),
    dict(name="c2", n=3000, L=60, P=10, Hq=8, Hkv=8),
    dict(name="c2", n=3000, L=64, P=10, Hq=16, Hkv=8),
    dict(name="c2", n=2000, L=9, P=9, Hq=8, Hkv=2),
    dict(name="c2", n=2000, L=30, P=10, Hq=8, Hkv=2, tau=0.3),
    # more than four query heads per KV head: passes of four (or two, or one)
    dict(name="c2", n=3000, Hq=16, Hkv=2),          # 8 a KV head: two passes of four
    dict(name="c2", n=2000, Hq=6, Hkv=2),           # 3: three passes of one
    dict(name="c2", n=2500, L=60, P=10, Hq=16, Hkv=2),
    dict(name="c4", n=(1000, 5000), B=3, Hq=24, Hkv=2, k=0.02),  # 12, ragged
    dict(name="c2", n=2500, L=45, P=9, Hq=8, Hkv=2),    # packed nine-bit IDs
    # many short and empty rows: ragged shares that start or lie inside a row's fixed cost
    dict(name="c4", n=(10, 20), B=24, Hq=8, Hkv=2, n_cap=3000, k=0.02,
         lens=[0, 1, 64, 65, 127, 128, 129, 300, 1000, 0, 2, 3000, 17, 640, 641, 960, 5, 2047,
               2048, 2049, 1, 64, 700, 2999]),
]


def _oracle_ids(w):
    ids = np.empty((w.B, w.Hkv, w.n_cap, w.L), np.uint16 if w.P > 8 else np.uint8)
    vn = np.empty((w.B, w.Hkv, w.n_cap), np.float32)
    for b in range(w.B):
        for h in range(w.Hkv):
            ids[b, h] = SO.hash_keys(w.K[b, h], w.W, w.L, w.P)[0]
            vn[b, h] = SO.value_norms(w.V[b, h]).astype(np.float32)
    return ids, vn


@pytest.mark.parametrize("case", SCORE_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_score_topk_parity(case):
    """Scorer fed the oracle's IDs and norms, so it is tested on its own."""
    print("case", case, flush=True)
    w = make_workload(**case)
    d = GC.upload(w)
    ids_np, vn_np = _oracle_ids(w)
    ids = GC.ids_dev(ids_np, w.n_cap, w.P)
    vn = torch.from_numpy(vn_np).to(DEV)
    idx, sc = GC.gpu_score_topk(w, d, ids, vn)
    sync()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    tables = SO.soft_tables(w.q, w.W, w.L, w.P, w.tau)
    s_ref = SO.scores(tables, ids_np, vn_np.astype(np.float64), w.lens)
    for b in range(w.B):
        n, k = int(w.lens[b]), int(w.ks[b])
        for g in range(w.Hq):
            GC.check_scores(sc[b, g, :n], s_ref[b, g, :n])
            GC.check_exact_topk(idx[b, g], sc[b, g], k, n)
            GC.check_set(idx[b, g], s_ref[b, g, :n], k)


SINK_WINDOW_CASES = [
    dict(case=dict(name="c2", n=5000), sink=64, window=128),
    dict(case=dict(name="c2", n=4500, Hq=8, Hkv=8, L=60, P=10), sink=128, window=64),
    dict(case=dict(name="c2", n=20000, k=300), sink=64, window=64),    # several scan workgroups
    dict(case=dict(name="c4", n=(1000, 9000), B=4, k=0.02), sink=64, window=128),
    dict(case=dict(name="c4", n=(10, 20), B=5, Hq=8, Hkv=2, lens=[0, 50, 191, 192, 700],
                   n_cap=1000, k=5), sink=64, window=128),        # n <= sink + window, n = 0
    dict(case=dict(name="c2", n=3000, Hq=8, Hkv=2, k=0), sink=7, window=33),  # k = 0: forced only
    dict(case=dict(name="c2", n=3000, Hq=8, Hkv=2), sink=0, window=100),
    dict(case=dict(name="c2", n=3000, Hq=8, Hkv=2), sink=100, window=0),
]


@pytest.mark.parametrize("sw", SINK_WINDOW_CASES,
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c["case"].items())
                         + f"-s{c['sink']}-w{c['window']}")
def test_select_sink_window_parity(sw):
    """Sink and window keys always selected, top-k over the rest, then attention."""
    print("case", sw, flush=True)
    w = make_workload(**sw["case"])
    sink, window = sw["sink"], sw["window"]
    d = GC.upload(w)
    ids_np, vn_np = _oracle_ids(w)
    ids = GC.ids_dev(ids_np, w.n_cap, w.P)
    vn = torch.from_numpy(vn_np).to(DEV)
    idx, sc = GC.gpu_score_topk(w, d, ids, vn, sink=sink, window=window)
    out = GC.gpu_decode(w, d, idx)
    sync()
    idx, sc, out = idx.cpu().numpy(), sc.cpu().numpy(), out.cpu().numpy()
    tables = SO.soft_tables(w.q, w.W, w.L, w.P, w.tau)
    s_ref = SO.scores(tables, ids_np, vn_np.astype(np.float64), w.lens)
    group = w.Hq // w.Hkv
    for b in range(w.B):
        n, k = int(w.lens[b]), int(w.ks[b])
        for g in range(w.Hq):
            GC.check_scores(sc[b, g, :n], s_ref[b, g, :n])
            GC.check_exact_select(idx[b, g], sc[b, g], k, n, sink, window)
            GC.check_select_set(idx[b, g], s_ref[b, g, :n], k, n, sink, window)
            if g % 3 == 0:
                GC.check_out(out[b, g], w.q[b, g], w.K[b, g // group], w.V[b, g // group],
                             idx[b, g], w.scale)


@pytest.mark.parametrize("n", [3000, 8000, 20000, 70000])
def test_topk_ties_lower_index_wins(n):
    """All keys of a head share one bucket pattern and norm -> equal scores.
    3000 and 8000 equal keys fit the streaming top-k's LDS candidate list;
    20000 and 70000 overflow it and take its second pass through the global
    candidate list."""
    w = make_workload("c2", n=n, Hq=8, Hkv=2, k=100)
    d = GC.upload(w)
    ids = S.alloc_ids(w.B, w.Hkv, w.n_cap, w.L, w.P, DEV)
    vn = torch.ones(w.B, w.Hkv, w.n_cap, dtype=torch.float32, device=DEV)
    # KV head 1: second half of the keys gets a larger norm -> they win, ties among them
    half = n // 2
    vn[:, 1, half:] = 2.0
    idx, sc = GC.gpu_score_topk(w, d, ids, vn)
    sync()
    idx = idx.cpu().numpy()
    for g in range(w.Hq):
        h = g // (w.Hq // w.Hkv)
        expect = np.arange(100) if h == 0 else np.arange(half, half + 100)
        assert idx[0, g, :100].tolist() == expect.tolist()
        assert (idx[0, g, 100:] == -1).all()


@pytest.mark.parametrize("tied", [900, 3000, 6000])
def test_topk_resolve_tied_block(tied):
    """Rows of 45000 keys (scan + resolve) where a block of `tied` keys shares
    the top score: all of them are boundary candidates of one bin, up to one
    per resolve thread or past that (the rest loaded in a second round trip),
    and the lower indices win."""
    n, k, start = 45000, 100, 20000
    w = make_workload("c2", n=n, Hq=8, Hkv=2, k=k)
    d = GC.upload(w)
    ids = S.alloc_ids(w.B, w.Hkv, w.n_cap, w.L, w.P, DEV)
    vn = torch.ones(w.B, w.Hkv, w.n_cap, dtype=torch.float32, device=DEV)
    vn[:, 1, start:start + tied] = 2.0
    idx, _ = GC.gpu_score_topk(w, d, ids, vn)
    sync()
    idx = idx.cpu().numpy()
    for g in range(w.Hq):
        h = g // (w.Hq // w.Hkv)
        expect = np.arange(k) if h == 0 else np.arange(start, start + k)
        assert idx[0, g, :k].tolist() == expect.tolist(), g


@pytest.mark.parametrize("B,Hq,Hkv,n", [(4, 32, 8, 40000), (1, 264, 66, 140000)],
                         ids=["4x32-heads-40000", "264-heads-140000"])
def test_topk_ties_large_batches(B, Hq, Hkv, n):
    """Equal scores in large launches: every key is a boundary candidate, so
    the streaming top-k's LDS candidate list overflows into the global list,
    and the lower indices must still win.  264 heads (more than CUs) of
    140000 keys take the 1024-thread form (rows too long for the 512-thread
    one), whose bitmap spans several emit segments."""
    w = make_workload("c4", n=(64, 64), B=B, Hq=Hq, Hkv=Hkv, k=100)  # q and W; keys set below
    w.n_cap = n + 1
    w.lens = np.full(w.B, n, np.int32)
    w.ks = np.full(w.B, 100, np.int32)
    d = GC.upload(w)
    ids = S.alloc_ids(w.B, w.Hkv, w.n_cap, w.L, w.P, DEV)
    vn = torch.ones(w.B, w.Hkv, w.n_cap, dtype=torch.float32, device=DEV)
    half = n // 2
    vn[:, 1, half:] = 2.0  # KV head 1: the second half wins, ties among them
    idx, _ = GC.gpu_score_topk(w, d, ids, vn)
    sync()
    idx = idx.cpu().numpy()
    for b in range(w.B):
        for g in range(w.Hq):
            h = g // (w.Hq // w.Hkv)
            expect = np.arange(half, half + 100) if h == 1 else np.arange(100)
            assert idx[b, g].tolist() == expect.tolist(), (b, g)


@pytest.mark.parametrize("ties", [False, True], ids=["scores", "ties"])
def test_topk_long_rows_scan_resolve(ties):
    """Rows longer than the streaming top-k's LDS bitmap (512K keys) take the
    scan + resolve kernels: 600000 keys for two query heads, on the oracle's
    scores, or with every score equal (all keys boundary candidates, kept in
    the global list; the lower indices win)."""
    w = make_workload("c2", n=600000, Hq=2, Hkv=1, L=16, k=1200)
    d = GC.upload(w)
    if ties:
        ids = S.alloc_ids(w.B, w.Hkv, w.n_cap, w.L, w.P, DEV)
        vn = torch.ones(w.B, w.Hkv, w.n_cap, dtype=torch.float32, device=DEV)
        idx, _ = GC.gpu_score_topk(w, d, ids, vn, sink=5, window=7)
        sync()
        idx = idx.cpu().numpy()
        n = int(w.lens[0])
        expect = list(range(5 + 1200)) + list(range(n - 7, n))
        for g in range(w.Hq):
            assert idx[0, g].tolist() == expect
        return
    ids_np, vn_np = _oracle_ids(w)
    ids = GC.ids_dev(ids_np, w.n_cap, w.P)
    vn = torch.from_numpy(vn_np).to(DEV)
    idx, sc = GC.gpu_score_topk(w, d, ids, vn)
    sync()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    tables = SO.soft_tables(w.q, w.W, w.L, w.P, w.tau)
    s_ref = SO.scores(tables, ids_np, vn_np.astype(np.float64), w.lens)
    n, k = int(w.lens[0]), int(w.ks[0])
    for g in range(w.Hq):
        GC.check_scores(sc[0, g, :n], s_ref[0, g, :n])
        GC.check_exact_topk(idx[0, g], sc[0, g], k, n)
        GC.check_set(idx[0, g], s_ref[0, g, :n], k)


def test_topk_edge_lengths():
    """Empty sequence, one key, k = n, k > n (clamped) in one batch."""
    w = make_workload("c4", n=(10, 20), B=4, Hq=8, Hkv=2, lens=[0, 1, 777, 300], n_cap=1000, k=5)
    d = GC.upload(w)
    ids_np, vn_np = _oracle_ids(w)
    ids = GC.ids_dev(ids_np, w.n_cap, w.P)
    vn = torch.from_numpy(vn_np).to(DEV)
    ks = torch.tensor([5, 5, 777, 999], dtype=torch.int32, device=DEV)
    k_max = 1000
    idx, sc = GC.gpu_score_topk(w, d, ids, vn, ks=ks, k_max=k_max)
    out = GC.gpu_decode(w, d, idx)
    sync()
    idx, sc, out = idx.cpu().numpy(), sc.cpu().numpy(), out.cpu().numpy()
    assert (idx[0] == -1).all()
    assert (out[0] == 0).all()
    assert (idx[1, :, 0] == 0).all() and (idx[1, :, 1:] == -1).all()
    assert (idx[2, :, :777] == np.arange(777)).all() and (idx[2, :, 777:] == -1).all()
    assert (idx[3, :, :300] == np.arange(300)).all() and (idx[3, :, 300:] == -1).all()
    for b in (1, 2, 3):
        for g in range(w.Hq):
            GC.check_out(out[b, g], w.q[b, g], w.K[b, g // 4], w.V[b, g // 4], idx[b, g], w.scale)


# ----------------------------------------------------------------------------- attention

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("k_max,n", [(1, 4096), (63, 4096), (200, 4096), (1024, 4096),
                                     # 47, 188 and 266 splits of 64 entries: the merges for
                                     # up to 128, up to 256 and any number of splits
                                     (3000, 4096), (12000, 16384), (17000, 20480)])
def test_sparse_decode_parity(dtype, k_max, n):
    w = make_workload("c2", n=n, Hq=8, Hkv=2, dtype=dtype)
    d = GC.upload(w)
    rng = np.random.default_rng(k_max)
    idx = np.full((w.B, w.Hq, k_max), -1, np.int32)
    for g in range(w.Hq):
        kk = rng.integers(0, k_max + 1) if g else k_max
        idx[0, g, :kk] = rng.choice(n, size=kk, replace=False)
        rng.shuffle(idx[0, g])
    out = GC.gpu_decode(w, d, torch.from_numpy(idx).to(DEV))
    sync()
    out = out.cpu().numpy()
    for g in range(w.Hq):
        GC.check_out(out[0, g], w.q[0, g], w.K[0, g // 4], w.V[0, g // 4], idx[0, g], w.scale)


# ----------------------------------------------------------------------------- sampling estimator

def _estimate_run(w, M, seed=0):
    from soft_lsh_token_amd.inputs import uniforms
    d = GC.upload(w)
    ids_np, vn_np = _oracle_ids(w)
    ids = GC.ids_dev(ids_np, w.n_cap, w.P)
    vn = torch.from_numpy(vn_np).to(DEV)
    u = uniforms(w.B, w.Hq, M, seed)
    out = torch.full((w.B, w.Hq, w.d), float("nan"), dtype=torch.float32, device=DEV)
    draws = torch.full((w.B, w.Hq, M), -7, dtype=torch.int32, device=DEV)
    sc = torch.zeros(w.B, w.Hq, S.score_stride(w.n_cap), dtype=torch.float32, device=DEV)
    S.socket_sample_estimate(d["q"], d["W"], ids, vn, d["V"], d["lens"], torch.from_numpy(u).to(DEV),
                             w.tau, w.L, w.P, out, draws, sc)
    sync()
    return ids_np, vn_np, u, out.cpu().numpy(), draws.cpu().numpy(), sc.cpu().numpy()


def _check_estimate(w, ids_np, vn_np, u, out, draws, sc, heads=None):
    """Draws against the oracle's inverse-CDF draws (a different key only where
    the uniform lies within 1e-5 of the boundary between the two), and T
    against the oracle run on uniforms that reproduce the GPU's draws."""
    tables = SO.soft_tables(w.q, w.W, w.L, w.P, w.tau)
    group = w.Hq // w.Hkv
    moved = 0
    for b in range(w.B):
        n = int(w.lens[b])
        for g in (heads if heads is not None else range(w.Hq)):
            h = g // group
            if n == 0:
                assert (out[b, g] == 0).all() and (draws[b, g] == -1).all()
                continue
            vref = vn_np[b, h, :n].astype(np.float64)
            s_ref = GC.ref_scores(tables[b, g], ids_np[b, h, :n], vref)
            GC.check_scores(sc[b, g, :n], s_ref)
            p, S1, _ = SO.sampling_distribution(tables[b, g], ids_np[b, h, :n], vref)
            cdf = np.cumsum(p)
            J = draws[b, g].astype(np.int64)
            assert (J >= 0).all() and (J < n).all()
            assert (p[J] > 0).all()
            Jr = SO.inverse_cdf(p, u[b, g])
            for m in np.nonzero(J != Jr)[0]:
                lo, hi = cdf[J[m]] - p[J[m]], cdf[J[m]]
                assert lo - 1e-5 <= u[b, g, m] <= hi + 1e-5, (b, g, m, J[m], Jr[m], u[b, g, m])
            moved += int((J != Jr).sum())
            umid = (cdf[J] - 0.5 * p[J]).astype(np.float64)   # uniforms that draw exactly J
            T, Jm = SO.sample_estimate(tables[b, g], ids_np[b, h, :n], w.V[b, h, :n], umid)
            assert (Jm == J).all()
            err = float(np.linalg.norm(out[b, g] - T))
            assert err <= 1e-4 * S1, (b, g, err, S1)
    return moved


@pytest.mark.parametrize("case,M", [
    (dict(name="c2", n=5000), 1024),
    (dict(name="c2", n=3000, Hq=8, Hkv=8, L=60, P=10), 512),
    (dict(name="c4", n=(10, 20), B=4, Hq=8, Hkv=2, lens=[0, 1, 100, 3000], n_cap=3000), 2048),
    (dict(name="c1"), 8192),
], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()) if isinstance(c, dict) else f"M{c}")
def test_sample_estimate_parity(case, M):
    print("case", case, M, flush=True)
    w = make_workload(**case)
    moved = _check_estimate(w, *_estimate_run(w, M))
    print("draws decided by rounding at a CDF boundary:", moved)


def test_sample_estimate_c2_concentration():
    """At the 32K GQA shape the estimate lies within the pages' concentration
    bound (Theorem 3, part 2) of the oracle's soft-attention output, delta = 1e-3."""
    w = workload("c2")
    M = 4096
    ids_np, vn_np, u, out, draws, sc = _estimate_run(w, M, seed=1)
    _check_estimate(w, ids_np, vn_np, u, out, draws, sc, heads=[0, 11, 30])
    tables = SO.soft_tables(w.q, w.W, w.L, w.P, w.tau)
    n, group = int(w.lens[0]), w.Hq // w.Hkv
    for g in range(w.Hq):
        h = g // group
        y = SO.soft_attention(tables[0, g], ids_np[0, h, :n], w.V[0, h, :n])
        bound = np.linalg.norm(w.V[0, h, :n].astype(np.float64), 2) * math.sqrt(
            8 * math.log(2 / 1e-3) / M)
        assert np.linalg.norm(out[0, g] - y) <= bound


# ----------------------------------------------------------------------------- hard-LSH mode

HARD_CASES = [
    dict(case=dict(name="c2", n=5000, L=300, P=2), sink=0, window=0),
    dict(case=dict(name="c2", n=3000, L=500, P=2, Hq=16, Hkv=8), sink=0, window=0),
    dict(case=dict(name="c2", n=3000, L=64, P=1, Hq=8, Hkv=8), sink=0, window=0),
    dict(case=dict(name="c1", L=100, P=4), sink=0, window=0),              # float32
    dict(case=dict(name="c2", n=2000, L=64, P=8, Hq=8, Hkv=2), sink=0, window=0),
    dict(case=dict(name="c2", n=2000, L=8, P=16, Hq=8, Hkv=2), sink=0, window=0),
    dict(case=dict(name="c4", n=(1000, 9000), B=3, L=300, P=2), sink=64, window=128),
    dict(case=dict(name="c4", n=(10, 20), B=4, Hq=8, Hkv=2, L=300, P=2, lens=[0, 1, 150, 900],
                   n_cap=1000, k=5), sink=16, window=16),
    dict(case=dict(name="c2", n=3000, L=300, P=2, Hq=16, Hkv=2), sink=0, window=0),   # G = 8
    dict(case=dict(name="c2", n=2000, L=64, P=4, Hq=6, Hkv=2), sink=8, window=8),    # G = 3
]


@pytest.mark.parametrize("L,P,n,off", [
    (300, 2, 1000, 0),     # 600 bits: two chunks of five waves
    (500, 2, 777, 0),      # 1000 bits: two chunks of eight waves, ragged tail
    (64, 1, 300, 0),       # 64 bits: one chunk with an idle wave
    (1024, 4, 200, 0),     # 4096 bits, the largest code: eight chunks
    (300, 2, 500, 123),    # a key range that starts past 0
], ids=lambda v: str(v))
def test_hash_codes_mfma(L, P, n, off):
    """bf16 sign codes from the MFMA path: the hashed keys' code bits (within
    the float32 band) and value norms against the oracle, bits past L*P
    cleared, and cells outside [off, off + n) untouched."""
    w = make_workload("c2", n=off + n, L=L, P=P, Hkv=2, Hq=4, n_cap=off + n + 70)
    d = GC.upload(w)
    codes = S.alloc_codes(w.B, w.Hkv, w.n_cap, L, P, DEV).fill_(0x5A5A5A5A)
    vn = torch.full((w.B, w.Hkv, w.n_cap), -1.0, dtype=torch.float32, device=DEV)
    pos0 = torch.full((w.B,), off, dtype=torch.int32, device=DEV)
    S.socket_hash_codes(d["K"], d["V"], d["W"], codes, vn, pos0, n, L, P)
    sync()
    c = codes.cpu().numpy().view(np.uint32)
    vn = vn.cpu().numpy()
    ids = S.layout.codes_to_ids(c[:, :, :, off:off + n], L, P)
    for h in range(w.Hkv):
        GC.check_ids(ids[0, h], w.K[0, h, off:off + n], w.W, L, P, n)
        np.testing.assert_allclose(vn[0, h, off:off + n], SO.value_norms(w.V[0, h, off:off + n]),
                                   rtol=2e-6)
    if (L * P) % 32:
        assert (c[:, :, -1, off:off + n] >> np.uint32((L * P) % 32) == 0).all()
    assert (c[:, :, :, :off] == 0x5A5A5A5A).all() and (c[:, :, :, off + n:] == 0x5A5A5A5A).all()
    assert (vn[:, :, :off] == -1.0).all() and (vn[:, :, off + n:] == -1.0).all()


def _hard_run(w, d, sink, window, heads=None):
    """Hard mode on the GPU (codes, query codes, scores, selection, attention)
    against the oracle; IDs are float-decided integers, so the scores are
    compared on the GPU's key IDs after those are checked against the oracle's."""
    L, P = w.L, w.P
    zeros = torch.zeros(w.B, dtype=torch.int32, device=DEV)
    codes = S.alloc_codes(w.B, w.Hkv, w.n_cap, L, P, DEV)
    vn = torch.zeros(w.B, w.Hkv, w.n_cap, dtype=torch.float32, device=DEV)
    S.socket_hash_codes(d["K"], d["V"], d["W"], codes, vn, zeros, int(w.lens.max()), L, P)
    # the query codes through the same projections: each query head as a one-key row
    q4 = d["q"].reshape(w.B, w.Hq, 1, w.d).contiguous()
    qc = S.alloc_codes(w.B, w.Hq, 1, L, P, DEV)
    qv = torch.zeros(w.B, w.Hq, 1, dtype=torch.float32, device=DEV)
    S.socket_hash_codes(q4, q4, d["W"], qc, qv, zeros, 1, L, P)
    k_max = w.k_max + sink + window
    idx = torch.full((w.B, w.Hq, k_max), -7, dtype=torch.int32, device=DEV)
    sc = torch.zeros(w.B, w.Hq, S.score_stride(w.n_cap), dtype=torch.float32, device=DEV)
    S.socket_hard_score_topk(d["q"], d["W"], codes, vn, d["lens"], d["ks"], k_max, L, P, idx, sc,
                             sink=sink, window=window)
    out = GC.gpu_decode(w, d, idx)
    sync()
    ids = S.layout.codes_to_ids(codes.cpu().numpy(), L, P)
    qids = S.layout.codes_to_ids(qc.cpu().numpy(), L, P)[:, :, 0]
    vn, idx, sc, out = (t.cpu().numpy() for t in (vn, idx, sc, out))
    group = w.Hq // w.Hkv
    for b in range(w.B):
        n = int(w.lens[b])
        for h in range(w.Hkv):
            GC.check_ids(ids[b, h], w.K[b, h], w.W, L, P, n)
            np.testing.assert_allclose(vn[b, h, :n], SO.value_norms(w.V[b, h, :n]), rtol=2e-6)
    qref, _ = SO.hash_keys(w.q[:, :, None, :], w.W, L, P)
    assert (qids == qref[:, :, 0]).all(), "a query plane fell inside the float32 band"
    s_ref = SO.hard_collision_scores(w.q, w.W, ids, vn.astype(np.float64), L, P, w.lens)
    for b in range(w.B):
        n, k = int(w.lens[b]), int(w.ks[b])
        for g in (heads if heads is not None else range(w.Hq)):
            GC.check_scores(sc[b, g, :n], s_ref[b, g, :n])
            GC.check_exact_select(idx[b, g], sc[b, g], k, n, sink, window)
            GC.check_select_set(idx[b, g], s_ref[b, g, :n], k, n, sink, window)
            if g % 5 == 0:
                GC.check_out(out[b, g], w.q[b, g], w.K[b, g // group], w.V[b, g // group],
                             idx[b, g], w.scale)


@pytest.mark.parametrize("hc", HARD_CASES,
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c["case"].items())
                         + f"-s{c['sink']}-w{c['window']}")
def test_hard_mode_parity(hc):
    print("case", hc, flush=True)
    w = make_workload(**hc["case"])
    _hard_run(w, GC.upload(w), hc["sink"], hc["window"])


def test_hard_mode_c2_full_600_bits():
    """The 32K GQA step in hard mode at the pages' 600-bit budget (P = 2, L = 300)."""
    w = workload("c2", L=300, P=2)
    _hard_run(w, GC.upload(w), 0, 0)


# ----------------------------------------------------------------------------- dense reference

DENSE_CASES = [
    dict(name="c2", n=5000),                                    # ragged last split
    dict(name="c2", n=4500, Hq=8, Hkv=8),                       # one query head per KV head
    dict(name="c2", n=4500, Hq=16, Hkv=8),                      # two
    dict(name="c1"),                                            # float32
    dict(name="c4", n=(10, 20), B=5, Hq=8, Hkv=2, lens=[0, 1, 17, 256, 3000], n_cap=3001),
    dict(name="c4", n=(1000, 9000), B=3),
    dict(name="c2", n=20000, Hq=8, Hkv=2),                      # 157 splits: eight-group merge
    dict(name="c2", n=20000, Hq=4, Hkv=1),                      # 313 splits: general merge
    dict(name="c2", n=4500, Hq=16, Hkv=2),                      # 8 query heads a KV head
    dict(name="c2", n=3000, Hq=6, Hkv=2),                       # 3
]


@pytest.mark.parametrize("case", DENSE_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_dense_decode_parity(case):
    """Full attention over every key of the sequence against the oracle."""
    print("case", case, flush=True)
    w = make_workload(**case)
    d = GC.upload(w)
    out = torch.full((w.B, w.Hq, w.d), float("nan"), dtype=torch.float32, device=DEV)
    S.socket_dense_decode(d["q"], d["K"], d["V"], d["lens"], w.scale, out)
    sync()
    out = out.cpu().numpy()
    group = w.Hq // w.Hkv
    for b in range(w.B):
        n = int(w.lens[b])
        for g in range(w.Hq):
            h = g // group
            GC.check_out(out[b, g], w.q[b, g], w.K[b, h], w.V[b, h], np.arange(n, dtype=np.int64),
                         w.scale)


@pytest.mark.parametrize("name,heads", [("c2", range(32)), ("c3", [0, 7, 13, 31])])
def test_dense_decode_full_size(name, heads):
    """The dense reference at the 32K and 128K GQA shapes (sampled heads at 128K)."""
    w = workload(name)
    d = GC.upload(w)
    out = torch.empty(w.B, w.Hq, w.d, dtype=torch.float32, device=DEV)
    S.socket_dense_decode(d["q"], d["K"], d["V"], d["lens"], w.scale, out)
    sync()
    out = out.cpu().numpy()
    n, group = int(w.lens[0]), w.Hq // w.Hkv
    for g in heads:
        h = g // group
        GC.check_out(out[0, g], w.q[0, g], w.K[0, h], w.V[0, h], np.arange(n, dtype=np.int64),
                     w.scale)


# ----------------------------------------------------------------------------- end to end

def _e2e(w, heads=None):
    """Hash -> score + top-k -> attention on the GPU, checked against the oracle."""
    d = GC.upload(w)
    ids, vn = GC.gpu_hash(w, d)
    idx, sc = GC.gpu_score_topk(w, d, ids, vn)
    out = GC.gpu_decode(w, d, idx)
    sync()
    ids = GC.ids_np(ids, w.L, w.n_cap, w.P)
    vn, idx, sc, out = (t.cpu().numpy() for t in (vn, idx, sc, out))
    group = w.Hq // w.Hkv
    tables = SO.soft_tables(w.q, w.W, w.L, w.P, w.tau)
    stats = dict(band_bits=0, id_rows_differ=0, set_diff=0, max_out_err=0.0)
    for b in range(w.B):
        n, k = int(w.lens[b]), int(w.ks[b])
        hs = sorted({g // group for g in (heads if heads is not None else range(w.Hq))})
        for h in hs:
            band, diff_rows, ids_ref = GC.check_ids(ids[b, h], w.K[b, h], w.W, w.L, w.P, n,
                                                    detail=True)
            stats["band_bits"] += band
            stats["id_rows_differ"] += len(diff_rows)
            vref = SO.value_norms(w.V[b, h, :n])
            np.testing.assert_allclose(vn[b, h, :n], vref, rtol=2e-6)
            for g in range(h * group, (h + 1) * group):
                if heads is not None and g not in heads:
                    continue
                s_ref = GC.check_scores_both(sc[b, g, :n], tables[b, g], ids[b, h, :n], ids_ref,
                                             vref, diff_rows)
                GC.check_exact_topk(idx[b, g], sc[b, g], k, n)
                stats["set_diff"] += GC.check_set(idx[b, g], s_ref, k)
                e = GC.check_out(out[b, g], w.q[b, g], w.K[b, h], w.V[b, h], idx[b, g], w.scale)
                stats["max_out_err"] = max(stats["max_out_err"], e)
    print("e2e", w.name, stats, flush=True)
    return stats


def test_e2e_c1_full():
    _e2e(workload("c1"))


def test_e2e_c2_full():
    _e2e(workload("c2"))


def test_e2e_c2_sink_window_full():
    """The 32K GQA step with 64 sink and 128 window keys next to the top-656."""
    w = workload("c2")
    d = GC.upload(w)
    ids, vn = GC.gpu_hash(w, d)
    idx, sc = GC.gpu_score_topk(w, d, ids, vn, sink=64, window=128)
    out = GC.gpu_decode(w, d, idx)
    sync()
    ids = GC.ids_np(ids, w.L, w.n_cap, w.P)
    vn, idx, sc, out = (t.cpu().numpy() for t in (vn, idx, sc, out))
    tables = SO.soft_tables(w.q, w.W, w.L, w.P, w.tau)
    n, k, group = int(w.lens[0]), int(w.ks[0]), w.Hq // w.Hkv
    for g in range(w.Hq):
        h = g // group
        s_ref = GC.ref_scores(tables[0, g], ids[0, h, :n], SO.value_norms(w.V[0, h, :n]))
        GC.check_scores(sc[0, g, :n], s_ref)
        assert GC.check_exact_select(idx[0, g], sc[0, g], k, n, 64, 128) == k + 192
        GC.check_select_set(idx[0, g], s_ref, k, n, 64, 128)
        GC.check_out(out[0, g], w.q[0, g], w.K[0, h], w.V[0, h], idx[0, g], w.scale)


def test_e2e_c2_p10_l60_full():
    """The 32K GQA step at 10 planes x 60 tables (600 bits per key)."""
    _e2e(workload("c2", L=60, P=10))


def test_e2e_c3_full_sampled_heads():
    _e2e(workload("c3"), heads=[0, 5, 14, 22, 31])


def test_e2e_c4_full_sampled_heads():
    _e2e(workload("c4"), heads=[0, 13, 30])


@pytest.mark.parametrize("fused", [False, True], ids=["three-calls", "decode-step"])
def test_decode_loop_c5(fused):
    """Prefill 131072 keys, then 256 steps each appending one key/value per KV head
    (through the three calls, or through socket_decode_step); steps 0, 1, 2, 127
    and 255 are checked against the oracle on sampled heads."""
    w = workload("c5")
    d = GC.upload(w)
    n0 = int(w.lens[0])
    ids, vn = GC.gpu_hash(w, d, count=n0)
    heads = [0, 9, 27]
    check_steps = {0, 1, 2, 127, 255}
    lens = d["lens"].clone()
    ks = d["ks"]
    keep = {}
    for t in range(w.steps):
        # the caller has written row n0+t of K/V (the inputs already hold it); hash it
        q = torch.from_numpy(w.q_steps[t]).to(DEV).to(torch.bfloat16)
        if fused:
            lens += 1
            idx = torch.empty(w.B, w.Hq, w.k_max, dtype=torch.int32, device=DEV)
            sc = torch.zeros(w.B, w.Hq, S.score_stride(w.n_cap), dtype=torch.float32, device=DEV)
            out = torch.empty(w.B, w.Hq, w.d, dtype=torch.float32, device=DEV)
            S.socket_decode_step(q, d["K"], d["V"], d["W"], ids, vn, lens, ks, w.k_max, w.tau,
                                 w.L, w.P, w.scale, idx, out, scores=sc)
        else:
            GC.gpu_hash(w, d, pos0=lens, count=1, ids=ids, vnorm=vn)
            lens += 1
            idx, sc = GC.gpu_score_topk(w, d, ids, vn, lens=lens, q=q)
            out = GC.gpu_decode(w, d, idx, q=q)
        if t in check_steps:
            keep[t] = [x.cpu().numpy() for x in (idx, sc, out)]
    sync()
    ids_np, vn_np = GC.ids_np(ids, w.L, w.n_cap, w.P), vn.cpu().numpy()
    group = w.Hq // w.Hkv
    for h in sorted({g // group for g in heads}):
        n_all = n0 + w.steps
        band, diff_rows, ids_ref = GC.check_ids(ids_np[0, h], w.K[0, h], w.W, w.L, w.P, n_all,
                                                detail=True)
        print("kv head", h, "band bits", band, "rows whose ids differ", diff_rows.tolist(),
              flush=True)
        vref = SO.value_norms(w.V[0, h, :n_all])
        np.testing.assert_allclose(vn_np[0, h, :n_all], vref, rtol=2e-6)
        for t, (idx, sc, out) in keep.items():
            n = n0 + t + 1
            qt = w.q_steps[t]
            tables = SO.soft_tables(qt, w.W, w.L, w.P, w.tau)
            for g in heads:
                if g // group != h:
                    continue
                s_ref = GC.check_scores_both(sc[0, g, :n], tables[0, g], ids_np[0, h, :n],
                                             ids_ref[:n], vref[:n], diff_rows[diff_rows < n])
                k = int(w.ks[0])
                GC.check_exact_topk(idx[0, g], sc[0, g], k, n)
                GC.check_set(idx[0, g], s_ref, k)
                GC.check_out(out[0, g], qt[0, g], w.K[0, h], w.V[0, h], idx[0, g], w.scale)


def test_run_twice_bitwise():
    w = workload("c2")
    d = GC.upload(w)
    ids, vn = GC.gpu_hash(w, d)
    r1 = [GC.gpu_score_topk(w, d, ids, vn)]
    r1.append(GC.gpu_decode(w, d, r1[0][0]))
    ids2, vn2 = GC.gpu_hash(w, d)
    r2 = [GC.gpu_score_topk(w, d, ids2, vn2)]
    r2.append(GC.gpu_decode(w, d, r2[0][0]))
    sync()
    assert torch.equal(ids, ids2) and torch.equal(vn, vn2)
    assert torch.equal(r1[0][0], r2[0][0]) and torch.equal(r1[0][1], r2[0][1])
    assert torch.equal(r1[1], r2[1])


@pytest.mark.parametrize("case,sw", [
    (dict(name="c2", n=5000), (0, 0)),
    (dict(name="c4", n=(1000, 9000), B=3, k=0.02), (64, 128)),
    (dict(name="c4", n=(10, 20), B=4, Hq=8, Hkv=2, lens=[0, 1, 300, 999], n_cap=1000, k=5), (8, 8)),
    (dict(name="c2", n=3000, L=60, P=10, Hq=16, Hkv=8), (0, 0)),
    (dict(name="c2", n=2000, L=40, P=9, Hq=8, Hkv=2), (8, 8)),   # packed, generic append
    (dict(name="c1"), (0, 16)),
    # longer rows: the scan + resolve top-k
    (dict(name="c2", n=20000), (0, 0)),
    (dict(name="c2", n=20000, k=300), (64, 128)),          # k_max 492: 8 splits
    # 300000 keys: the range kernel's widest ranges (24 blocks), 49 ranges a
    # head, merged by the wide combine
    (dict(name="c2", n=300000, Hq=2, Hkv=1, L=16, k=600), (0, 0)),
    (dict(name="c4", n=(9000, 30000), B=3, Hq=8, Hkv=2, lens=[30000, 9000, 12345]), (16, 16)),
    (dict(name="c1", n=10000, k=200), (0, 0)),              # float32
    (dict(name="c1", n=70000, k=300), (0, 16)),             # float32, 256-thread ranges
    # attention inside the selecting workgroups: the resolve form (rows past
    # the streaming top-k's length), the 512-thread streaming form (more heads
    # than CUs), and a selection too long to be kept in LDS (separate attention)
    (dict(name="c2", n=50000, Hq=8, Hkv=2), (0, 0)),
    (dict(name="c4", n=(1000, 3000), B=9, k=0.02), (16, 16)),
    (dict(name="c2", n=30000, Hq=8, Hkv=2, k=17000), (0, 0)),
    # eight and twelve query heads per KV head
    (dict(name="c2", n=6000, Hq=16, Hkv=2), (16, 16)),
    (dict(name="c4", n=(1000, 4000), B=3, Hq=24, Hkv=2, k=0.02), (0, 0)),
], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()) if isinstance(c, dict) else f"sw{c}")
def test_decode_step_matches_three_calls(case, sw):
    """socket_decode_step (append hashed inside the table kernel, attention
    inside the selecting workgroups where it fits) equals socket_hash_keys +
    socket_score_topk + socket_sparse_decode: IDs, norms, scores and indices
    bit for bit; the attention output, summed in another order, to 1e-5, and
    within the oracle's bar on its own."""
    print("case", case, sw, flush=True)
    sink, window = sw
    w = make_workload(**case)
    d = GC.upload(w)
    # every sequence's first lens-1 keys are cached; its key lens-1 is the new one
    n0 = np.maximum(w.lens - 1, 0).astype(np.int32)
    ids1 = S.alloc_ids(w.B, w.Hkv, w.n_cap, w.L, w.P, DEV)
    vn1 = torch.zeros(w.B, w.Hkv, w.n_cap, dtype=torch.float32, device=DEV)
    zero = torch.zeros(1, dtype=torch.int32, device=DEV)
    for b in range(w.B):
        if n0[b]:
            ib = S.alloc_ids(1, w.Hkv, w.n_cap, w.L, w.P, DEV)
            vb = torch.zeros(1, w.Hkv, w.n_cap, dtype=torch.float32, device=DEV)
            S.socket_hash_keys(d["K"][b:b + 1].contiguous(), d["V"][b:b + 1].contiguous(), d["W"],
                               ib, vb, zero, int(n0[b]), w.L, w.P)
            ids1[b:b + 1] = ib
            vn1[b:b + 1] = vb
    ids2, vn2 = ids1.clone(), vn1.clone()
    k_max = w.k_max + sink + window
    # three calls; a sequence with lens = 0 has no new key
    for b in range(w.B):
        if w.lens[b] > 0:
            ib, vb = ids1[b:b + 1].clone(), vn1[b:b + 1].clone()
            S.socket_hash_keys(d["K"][b:b + 1].contiguous(), d["V"][b:b + 1].contiguous(), d["W"],
                               ib, vb, torch.full((1,), int(n0[b]), dtype=torch.int32, device=DEV),
                               1, w.L, w.P)
            ids1[b:b + 1] = ib
            vn1[b:b + 1] = vb
    idx1, sc1 = GC.gpu_score_topk(w, d, ids1, vn1, sink=sink, window=window)
    out1 = GC.gpu_decode(w, d, idx1)
    # one call
    idx2 = torch.full_like(idx1, -7)
    sc2 = torch.zeros_like(sc1)
    out2 = torch.full_like(out1, float("nan"))
    S.socket_decode_step(d["q"], d["K"], d["V"], d["W"], ids2, vn2, d["lens"], d["ks"], k_max, w.tau,
                         w.L, w.P, w.scale, idx2, out2, scores=sc2, sink=sink, window=window)
    sync()
    assert torch.equal(ids1, ids2)
    assert torch.equal(vn1, vn2)
    assert torch.equal(idx1, idx2)
    assert torch.equal(sc1, sc2)
    assert not torch.isnan(out2).any()
    torch.testing.assert_close(out2, out1, rtol=0, atol=1e-5)
    idx_np, out_np = idx2.cpu().numpy(), out2.cpu().numpy()
    group = w.Hq // w.Hkv
    for b in range(w.B):
        for g in range(0, w.Hq, 5):
            GC.check_out(out_np[b, g], w.q[b, g], w.K[b, g // group], w.V[b, g // group],
                         idx_np[b, g], w.scale)


@pytest.mark.parametrize("n,tied", [(20000, 900), (20000, 3000), (45000, 20000)],
                         ids=["20000-tied900", "20000-tied3000", "45000-tied20000"])
def test_decode_step_ties_match_three_calls(n, tied):
    """Equal scores inside socket_decode_step: every cached key has the same
    bucket IDs and a block of `tied` keys the larger norm, so the boundary bin
    holds the whole block (900 candidates fit the range workgroups' LDS list;
    3000 and 20000 are settled in place from the global list).  Indices must
    equal the three calls' (lower indices win the ties) bit for bit, the
    output to 1e-5."""
    print("case", n, tied, flush=True)
    w = make_workload("c2", n=n, Hq=8, Hkv=2, k=100)
    d = GC.upload(w)
    start = 1000
    ids1 = S.alloc_ids(w.B, w.Hkv, w.n_cap, w.L, w.P, DEV)
    vn1 = torch.ones(w.B, w.Hkv, w.n_cap, dtype=torch.float32, device=DEV)
    vn1[:, 1, start:start + tied] = 2.0
    ids2, vn2 = ids1.clone(), vn1.clone()
    # three calls: hash the new key (position n - 1), select, attend
    S.socket_hash_keys(d["K"], d["V"], d["W"], ids1, vn1,
                       torch.full((1,), n - 1, dtype=torch.int32, device=DEV), 1, w.L, w.P)
    idx1, sc1 = GC.gpu_score_topk(w, d, ids1, vn1)
    out1 = GC.gpu_decode(w, d, idx1)
    idx2 = torch.full_like(idx1, -7)
    sc2 = torch.zeros_like(sc1)
    out2 = torch.full_like(out1, float("nan"))
    S.socket_decode_step(d["q"], d["K"], d["V"], d["W"], ids2, vn2, d["lens"], d["ks"], w.k_max,
                         w.tau, w.L, w.P, w.scale, idx2, out2, scores=sc2)
    sync()
    assert torch.equal(ids1, ids2) and torch.equal(vn1, vn2)
    assert torch.equal(sc1, sc2)
    assert torch.equal(idx1, idx2)
    torch.testing.assert_close(out2, out1, rtol=0, atol=1e-5)
    idx = idx2.cpu().numpy()
    for g in range(4, 8):  # KV head 1: the tied block beats the other cached keys
        sel = [i for i in idx[0, g].tolist() if i != n - 1]
        assert sel[:99] == list(range(start, start + 99)), g


def test_decode_step_graph_replays():
    """socket_decode_step_noalloc captured in a HIP graph on a side stream
    (it allocates nothing and records no memset) and replayed three times,
    with eager work on the outputs between replays: every replay equals the
    eager call bit for bit (IDs, norms, scores, indices, output)."""
    w = make_workload("c2", n=20000)
    d = GC.upload(w)
    n0 = int(w.lens[0]) - 1
    ids0, vn0 = GC.gpu_hash(w, d, count=n0)
    shape_sc = (w.B, w.Hq, S.score_stride(w.n_cap))

    def bufs():
        return (ids0.clone(), vn0.clone(),
                torch.full((w.B, w.Hq, w.k_max), -7, dtype=torch.int32, device=DEV),
                torch.zeros(shape_sc, dtype=torch.float32, device=DEV),
                torch.full((w.B, w.Hq, w.d), float("nan"), dtype=torch.float32, device=DEV))

    def call(b):
        ids, vn, idx, sc, out = b
        S.socket_decode_step_noalloc(d["q"], d["K"], d["V"], d["W"], ids, vn, d["lens"], d["ks"],
                                     w.k_max, w.tau, w.L, w.P, w.scale, idx, out, scores=sc)

    ref = bufs()
    call(ref)
    sync()
    gb = bufs()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(gb)  # warm-up on the capture stream
    sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(gb)
    sync()
    for rep in range(3):
        gb[0].copy_(ids0)
        gb[1].copy_(vn0)
        gb[2].fill_(-7)
        gb[3].zero_()
        gb[4].fill_(float("nan"))
        sync()
        g.replay()
        sync()
        for a, b in zip(ref, gb):
            assert torch.equal(a, b), rep
    GC.check_out(gb[4][0, 3].cpu().numpy(), w.q[0, 3], w.K[0, 0], w.V[0, 0],
                 gb[2][0, 3].cpu().numpy(), w.scale)


def test_stage_entry_points_match_fused_call():
    """socket_soft_tables + socket_score + socket_topk == socket_score_topk, bit for bit."""
    w = make_workload("c4", n=(3000, 9000), B=3, k=0.02)
    d = GC.upload(w)
    ids, vn = GC.gpu_hash(w, d)
    idx1, sc1 = GC.gpu_score_topk(w, d, ids, vn)
    ws = S.alloc_workspace(S.socket_score_topk_workspace(w.B, w.Hq, w.Hkv, w.n_cap, w.L, w.P, w.k_max),
                           DEV)
    sc2 = torch.zeros_like(sc1)
    idx2 = torch.full_like(idx1, -7)
    S.socket_soft_tables(d["q"], d["W"], w.Hkv, w.L, w.P, w.tau, w.n_cap, ws)
    S.socket_score(ids, vn, d["lens"], w.Hq, w.L, w.P, sc2, ws)
    S.socket_topk(sc2, d["lens"], d["ks"], w.Hkv, w.L, w.n_cap, idx2, ws)
    sync()
    assert torch.equal(sc1, sc2)
    assert torch.equal(idx1, idx2)
    # and with sink and window keys
    idx3, sc3 = GC.gpu_score_topk(w, d, ids, vn, sink=64, window=128)
    ws = S.alloc_workspace(S.socket_score_topk_workspace(w.B, w.Hq, w.Hkv, w.n_cap, w.L, w.P,
                                                         idx3.shape[-1]), DEV)
    sc4 = torch.zeros_like(sc3)
    idx4 = torch.full_like(idx3, -7)
    S.socket_soft_tables(d["q"], d["W"], w.Hkv, w.L, w.P, w.tau, w.n_cap, ws)
    S.socket_score(ids, vn, d["lens"], w.Hq, w.L, w.P, sc4, ws, sink=64, window=128)
    S.socket_topk(sc4, d["lens"], d["ks"], w.Hkv, w.L, w.n_cap, idx4, ws, sink=64, window=128)
    sync()
    assert torch.equal(sc3, sc4)
    assert torch.equal(idx3, idx4)


def test_side_stream_temporary_workspace():
    """Calls on a side stream with ws=None: the temporary workspace is freed when
    the call returns, while its kernels still wait behind other work on that
    stream.  Blocks that the current stream then allocates and overwrites must
    not be that workspace; results equal the default-stream calls bit for bit."""
    w = make_workload("c2", n=20000, n_cap=20064)
    d = GC.upload(w)
    ids, vn = GC.gpu_hash(w, d)
    idx1, sc1 = GC.gpu_score_topk(w, d, ids, vn)
    out1 = GC.gpu_decode(w, d, idx1)
    k_max = idx1.shape[-1]
    lens1 = d["lens"] + 1   # the step appends key 20000
    idx3 = torch.full_like(idx1, -7)
    out3 = torch.full_like(out1, float("nan"))
    S.socket_decode_step(d["q"], d["K"], d["V"], d["W"], ids.clone(), vn.clone(), lens1, d["ks"],
                         k_max, w.tau, w.L, w.P, w.scale, idx3, out3)
    sync()
    # the exact sizes of the three temporary workspaces (what the binding allocates)
    sizes = [S.socket_score_topk_workspace(w.B, w.Hq, w.Hkv, w.n_cap, w.L, w.P, k_max),
             S.socket_sparse_decode_workspace(w.B, w.Hq, w.d, k_max),
             S.socket_decode_step_workspace(w.B, w.Hq, w.Hkv, w.n_cap, w.L, w.P, k_max)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    a = torch.randn(4096, 4096, device=DEV)
    idx2 = torch.full_like(idx1, -7)
    sc2 = torch.zeros_like(sc1)
    out2 = torch.full_like(out1, float("nan"))
    idx4 = torch.full_like(idx1, -7)
    out4 = torch.full_like(out1, float("nan"))
    ids4, vn4 = ids.clone(), vn.clone()
    sync()
    with torch.cuda.stream(side):
        for _ in range(20):  # keep the side stream busy so the calls below queue up
            a = a @ a
            a = a / a.abs().max()
    junk = []

    def scribble(v):
        junk.extend(torch.full((n + 256,), v, dtype=torch.uint8, device=DEV) for n in sizes)

    S.socket_score_topk(d["q"], d["W"], ids, vn, d["lens"], d["ks"], k_max, w.tau, w.L, w.P, idx2,
                        sc2, stream=side)
    scribble(0xFF)
    S.socket_sparse_decode(d["q"], d["K"], d["V"], idx2, w.scale, out2, stream=side)
    scribble(0x7F)
    S.socket_decode_step(d["q"], d["K"], d["V"], d["W"], ids4, vn4, lens1, d["ks"], k_max, w.tau,
                         w.L, w.P, w.scale, idx4, out4, stream=side)
    scribble(0x3F)
    side.synchronize()
    sync()
    del junk
    assert torch.equal(idx1, idx2) and torch.equal(sc1, sc2) and torch.equal(out1, out2)
    assert torch.equal(idx3, idx4) and torch.equal(out3, out4)
