"""Shared helpers of the GPU parity tests: upload a workload, run the HIP path
through the C ABI, and check results against the CPU oracle with the
tolerances of the method's parity contract:

* bucket IDs bit-exact except bits whose float64 projection |W.k| < 1e-5,
* scores within 1e-5 relative (1e-30 absolute floor for underflowed ones),
* top-k sets equal except keys whose score is within 1e-5 (relative) of the
  k-th score; on the GPU's own float32 scores the set must match exactly,
* attention output within 2e-3 absolute.
"""
from __future__ import annotations

import numpy as np
import torch

import soft_lsh_token_amd as S
from oracle import socket_oracle as SO
from soft_lsh_token_amd import layout

DEV = "cuda:0"
ID_BAND = 1e-5
SCORE_RTOL, SCORE_ATOL = 1e-5, 1e-30
SET_BAND = 1e-5
OUT_ATOL = 2e-3


def tdtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def upload(w):
    dt = tdtype(w)
    dev = dict(
        K=torch.from_numpy(w.K).to(DEV).to(dt).contiguous(),
        V=torch.from_numpy(w.V).to(DEV).to(dt).contiguous(),
        W=torch.from_numpy(w.W).to(DEV).to(dt).contiguous(),
        q=torch.from_numpy(w.q).to(DEV).to(dt).contiguous(),
        lens=torch.from_numpy(w.lens).to(DEV),
        ks=torch.from_numpy(w.ks).to(DEV),
    )
    return dev


def gpu_hash(w, d, pos0=None, count=None, ids=None, vnorm=None):
    B, Hkv, n_cap = w.B, w.Hkv, w.n_cap
    if ids is None:
        ids = S.alloc_ids(B, Hkv, n_cap, w.L, w.P, DEV)
    if vnorm is None:
        vnorm = torch.zeros(B, Hkv, n_cap, dtype=torch.float32, device=DEV)
    if pos0 is None:
        pos0 = torch.zeros(B, dtype=torch.int32, device=DEV)
    if count is None:
        count = int(w.lens.max())
    S.socket_hash_keys(d["K"], d["V"], d["W"], ids, vnorm, pos0, count, w.L, w.P)
    return ids, vnorm


def gpu_score_topk(w, d, ids, vnorm, lens=None, ks=None, k_max=None, q=None, sink=0, window=0):
    lens = d["lens"] if lens is None else lens
    ks = d["ks"] if ks is None else ks
    k_max = w.k_max + sink + window if k_max is None else k_max
    q = d["q"] if q is None else q
    idx = torch.full((w.B, w.Hq, k_max), -7, dtype=torch.int32, device=DEV)
    scores = torch.zeros(w.B, w.Hq, S.score_stride(w.n_cap), dtype=torch.float32, device=DEV)
    S.socket_score_topk(q, d["W"], ids, vnorm, lens, ks, k_max, w.tau, w.L, w.P, idx, scores,
                        sink=sink, window=window)
    return idx, scores


def gpu_decode(w, d, idx, q=None):
    q = d["q"] if q is None else q
    out = torch.full((w.B, w.Hq, w.d), float("nan"), dtype=torch.float32, device=DEV)
    S.socket_sparse_decode(q, d["K"], d["V"], idx, w.scale, out)
    return out


def ids_np(ids_dev, L, n=None, P=8):
    """Tiled device cache -> [B, Hkv, n, L] numpy bucket IDs."""
    return layout.unpack(ids_dev.cpu().numpy(), L, n, P)


def ids_dev(ids_plain, n_cap, P=8):
    """[B, Hkv, n, L] numpy bucket IDs -> tiled device cache."""
    dt = np.uint16 if P > 8 else np.uint8
    return torch.from_numpy(layout.pack(np.ascontiguousarray(ids_plain, dtype=dt),
                                        n_cap, P)).to(DEV)


def check_ids(ids_gpu, K, W, L, P, n, detail=False):
    """ids_gpu: [n, L] uint8 numpy; K: [n, d].  Returns the number of bits inside
    the band (and, with detail, the rows whose IDs differ from the oracle's)."""
    ids_ref, z = SO.hash_keys(K[:n], W, L, P)
    bits_gpu = (ids_gpu[:n, :, None].astype(np.int64) >> np.arange(P)) & 1
    bits_ref = (ids_ref[:, :, None] >> np.arange(P)) & 1
    bad = (bits_gpu != bits_ref)
    in_band = np.abs(z) < ID_BAND
    assert not (bad & ~in_band).any(), f"{int((bad & ~in_band).sum())} id bits differ outside the band"
    if detail:
        return int(in_band.sum()), np.nonzero(bad.any(axis=(1, 2)))[0], ids_ref
    return int(in_band.sum())


def ref_scores(tables_row, ids_rows, vref):
    """Oracle soft-count scores of one query head over the given ID rows."""
    L = ids_rows.shape[1]
    return vref * tables_row[np.arange(L)[None, :], ids_rows.astype(np.int64)].sum(-1)


def check_scores_both(s_gpu, tables_row, ids_gpu, ids_ref, vref, diff_rows):
    """Scores against the oracle fed the GPU's bucket IDs (the bucket is a
    float-decided integer, so both sides score the same decision), and against
    the oracle's own IDs on every key whose IDs agree."""
    s_ref = ref_scores(tables_row, ids_gpu, vref)
    check_scores(s_gpu, s_ref)
    keep = np.ones(len(s_gpu), bool)
    keep[diff_rows] = False
    s_own = ref_scores(tables_row, ids_ref, vref)
    check_scores(s_gpu[keep], s_own[keep])
    return s_ref


def check_scores(s_gpu, s_ref):
    err = np.abs(s_gpu.astype(np.float64) - s_ref)
    lim = SCORE_RTOL * np.abs(s_ref) + SCORE_ATOL
    bad = err > lim
    assert not bad.any(), (f"{int(bad.sum())} scores off at {np.nonzero(bad)[0][:8].tolist()}; "
                           f"worst rel {float((err / np.maximum(np.abs(s_ref), 1e-300)).max()):.3e}")


def check_set(sel_gpu, s_ref, k):
    sel = [int(i) for i in sel_gpu if i >= 0]
    assert len(sel) == k and len(set(sel)) == k
    if k == 0:
        return 0
    ref = SO.topk(s_ref, k)
    kth = float(np.sort(s_ref)[::-1][k - 1])
    diff = set(sel) ^ set(ref.tolist())
    for i in diff:
        assert abs(s_ref[i] - kth) <= SET_BAND * abs(kth) + SCORE_ATOL, (i, s_ref[i], kth)
    return len(diff)


def check_exact_topk(idx_row, s_gpu_row, k, n):
    """On the GPU's own float32 scores the set (and ascending order) is exact."""
    ref = SO.topk(s_gpu_row[:n].astype(np.float64), k)
    got = idx_row[:k]
    assert got.tolist() == ref.tolist()
    assert (idx_row[k:] == -1).all()


def forced_keys(n, sink, window):
    return sorted(set(range(min(sink, n))) | set(range(max(n - window, 0), n)))


def check_exact_select(idx_row, s_gpu_row, k, n, sink, window):
    """Sink + window + top-k of the rest, on the GPU's own float32 scores: exact."""
    ref = SO.select(s_gpu_row[:n].astype(np.float64), k, n, sink, window)
    got = idx_row[:len(ref)]
    assert got.tolist() == ref.tolist()
    assert (idx_row[len(ref):] == -1).all()
    return len(ref)


def check_select_set(sel_gpu, s_ref, k, n, sink, window):
    """Against the oracle's scores: the forced keys exactly, the top-k part up to
    keys whose score is within SET_BAND of the k-th one among the rest."""
    sel = [int(i) for i in sel_gpu if i >= 0]
    forced = forced_keys(n, sink, window)
    ref = SO.select(s_ref, k, n, sink, window)
    assert len(sel) == len(ref) == len(set(sel))
    assert set(forced) <= set(sel)
    rest = np.array([i for i in range(n) if i not in set(forced)], dtype=np.int64)
    kk = min(k, len(rest))
    if kk == 0:
        assert sorted(sel) == forced
        return 0
    kth = float(np.sort(s_ref[rest])[::-1][kk - 1])
    diff = set(sel) ^ set(ref.tolist())
    for i in diff:
        assert abs(s_ref[i] - kth) <= SET_BAND * abs(kth) + SCORE_ATOL, (i, s_ref[i], kth)
    return len(diff)


def check_out(out_gpu, q, K, V, idx, scale):
    sel = idx[idx >= 0]
    if len(sel) == 0:
        assert np.all(out_gpu == 0)
        return 0.0
    ref = SO.sparse_attention(q, K, V, sel, scale)
    err = float(np.abs(out_gpu - ref).max())
    assert err <= OUT_ATOL, err
    return err
