"""Benchmark of the SOCKET decode hot path on one MI355X.

One step = one decode step of the GQA 32/8 workload at n = 32768 cached keys
(d = 128, L = 64 tables x P = 8 planes, tau = 0.5, k = 656 = ceil(2% of n)),
issued as a caller would, through three C calls:

  socket_hash_keys     append: hash the new key of every KV head, store its norm
  socket_score_topk    soft tables, soft-count scores of all n + 1 keys for the
                       32 query heads, top-656 per query head
  socket_sparse_decode exact attention of each query head over its keys

`value` is keys scored+selected per second: 32 query heads x (n + 1) keys per
step, divided by the wall time of K steps bracketed by device syncs.  Inputs
are resident in HBM.  The cache is replicated `--replicas` times (one replica
per step, round robin, like successive layers) so the 256 MiB Infinity Cache
cannot serve a step from the previous one.

Also reported: per-stage GPU time (batches of steps cut after each stage,
timed with one pair of HIP events per batch while the launches queue behind a
long matrix product, so host launch gaps stay out; a stage's time includes
its dispatch), the scorer's average launch time (a batch of scorer launches
alone) for the roofline, the 128K-key step, the prefill hashing rate against
the bf16 MFMA peak, and the CPU oracle's rate on a bounded sample.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import resource
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
SCORER_SRC = os.path.join(ROOT, "soft_lsh_token_amd", "csrc", "score_topk.hip")
COUNTERS = os.path.join(ROOT, "profiles", "scorer_c2_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--replicas", type=int, default=40)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-128k", action="store_true")
    p.add_argument("--no-batched", action="store_true",
                   help="skip the 16-sequence ragged batch (lengths 8K-32K)")
    p.add_argument("--no-hard", action="store_true",
                   help="skip the hard-LSH comparison mode")
    p.add_argument("--no-p10", action="store_true",
                   help="skip the 10-plane, 60-table measurement")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time budget of the oracle baseline")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="also run one device-to-device copy of this many MiB (a known-size "
                        "reference kernel for hardware byte counters)")
    return p.parse_args()


class Case:
    """Device buffers and pre-marshalled C calls of one decode workload."""

    def __init__(self, name, replicas, lib, torch, S, sink=0, window=0, **over):
        from soft_lsh_token_amd.inputs import make_workload
        t0 = time.time()
        self.w = w = make_workload(name, steps=1, **over)   # one extra row: the appended key
        log(f"[bench] {name}: inputs drawn in {time.time() - t0:.1f}s (n={int(w.lens[0])}, "
            f"n_cap={w.n_cap}, replicas={replicas})")
        dev = "cuda:0"
        bf = torch.bfloat16
        self.n = int(w.lens.max())             # prefill count (every sequence's rows)
        self.kv_keys = w.Hkv * int((w.lens.astype(np.int64) + 1).sum())  # keys scored per step
        self.B, self.Hq, self.Hkv, self.L, self.P = w.B, w.Hq, w.Hkv, w.L, w.P
        self.k = int(w.ks.max())
        self.sink, self.window = int(sink), int(window)
        self.k_max = self.k + self.sink + self.window   # index row: top-k + sink + window
        K0 = torch.from_numpy(w.K).to(dev).to(bf)
        V0 = torch.from_numpy(w.V).to(dev).to(bf)
        self.K = [K0] + [K0.clone() for _ in range(replicas - 1)]
        self.V = [V0] + [V0.clone() for _ in range(replicas - 1)]
        del K0, V0
        self.W = torch.from_numpy(w.W).to(dev).to(bf)
        self.q = torch.from_numpy(w.q).to(dev).to(bf)
        self.pos_prefill = torch.zeros(w.B, dtype=torch.int32, device=dev)
        self.pos_append = torch.from_numpy(w.lens.astype(np.int32)).to(dev)
        self.lens = torch.from_numpy(w.lens.astype(np.int32) + 1).to(dev)
        self.ks = torch.from_numpy(w.ks).to(dev)
        self.ids = [S.alloc_ids(w.B, w.Hkv, w.n_cap, w.L, w.P, dev) for _ in range(replicas)]
        self.vn = [torch.empty(w.B, w.Hkv, w.n_cap, dtype=torch.float32, device=dev)
                   for _ in range(replicas)]
        self.idx = torch.empty(w.B, w.Hq, self.k_max, dtype=torch.int32, device=dev)
        self.scores = torch.empty(w.B, w.Hq, S.score_stride(w.n_cap), dtype=torch.float32,
                                  device=dev)
        self.out = torch.empty(w.B, w.Hq, w.d, dtype=torch.float32, device=dev)
        sws = S.socket_score_topk_workspace(w.B, w.Hq, w.Hkv, w.n_cap, w.L, w.P, self.k_max)
        dws = S.socket_sparse_decode_workspace(w.B, w.Hq, w.d, self.k_max)
        self.sws = S.alloc_workspace(sws, dev)
        self.dws = S.alloc_workspace(dws, dev)
        self.sws_p = self.sws.data_ptr() + (-self.sws.data_ptr()) % 256
        self.dws_p = self.dws.data_ptr() + (-self.dws.data_ptr()) % 256
        self.sws_n, self.dws_n = sws, dws
        xsw = S.socket_decode_step_workspace(w.B, w.Hq, w.Hkv, w.n_cap, w.L, w.P, self.k_max)
        self.fws = S.alloc_workspace(xsw, dev)
        self.fws_p = self.fws.data_ptr() + (-self.fws.data_ptr()) % 256
        self.fws_n = xsw
        xws = S.socket_dense_decode_workspace(w.B, w.Hq, w.Hkv, w.d, w.n_cap)
        self.xws = S.alloc_workspace(xws, dev)
        self.xws_p = self.xws.data_ptr() + (-self.xws.data_ptr()) % 256
        self.xws_n = xws
        self.replicas = replicas
        self.lib = lib
        self.stream = torch.cuda.current_stream().cuda_stream
        self._prep()

    def _prep(self):
        w, lib = self.w, self.lib
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        st = vp(self.stream)
        self.c_append, self.c_prefill, self.c_score, self.c_decode, self.c_score_topk = \
            [], [], [], [], []
        self.c_dense = []
        self.c_fused = []
        for r in range(self.replicas):
            K, V, ids, vn = self.K[r].data_ptr(), self.V[r].data_ptr(), self.ids[r].data_ptr(), \
                self.vn[r].data_ptr()
            common = (vp(K), vp(V), 1, w.B, w.Hkv, w.d, i64(w.n_cap))
            self.c_prefill.append(common + (vp(self.pos_prefill.data_ptr()), self.n,
                                             vp(self.W.data_ptr()), w.L, w.P, vp(ids), vp(vn), st))
            self.c_append.append(common + (vp(self.pos_append.data_ptr()), 1,
                                            vp(self.W.data_ptr()), w.L, w.P, vp(ids), vp(vn), st))
            self.c_score.append((w.B, w.Hq, w.Hkv, w.L, w.P, vp(ids), vp(vn),
                                 vp(self.lens.data_ptr()), i64(w.n_cap), self.sink, self.window,
                                 vp(self.scores.data_ptr()), vp(self.sws_p),
                                 ctypes.c_size_t(self.sws_n), st))
            self.c_score_topk.append((vp(self.q.data_ptr()), 1, w.B, w.Hq, w.Hkv, w.d,
                                      vp(self.W.data_ptr()), w.L, w.P, ctypes.c_float(w.tau),
                                      vp(ids), vp(vn), vp(self.lens.data_ptr()), i64(w.n_cap),
                                      vp(self.ks.data_ptr()), self.k_max, self.sink, self.window,
                                      vp(self.idx.data_ptr()),
                                      vp(self.scores.data_ptr()), vp(self.sws_p),
                                      ctypes.c_size_t(self.sws_n), st))
            self.c_decode.append((vp(self.q.data_ptr()), vp(K), vp(V), 1, w.B, w.Hq, w.Hkv, w.d,
                                  i64(w.n_cap), vp(self.idx.data_ptr()), self.k_max,
                                  ctypes.c_float(w.scale), vp(self.out.data_ptr()),
                                  vp(self.dws_p), ctypes.c_size_t(self.dws_n), st))
            self.c_fused.append((vp(self.q.data_ptr()), vp(K), vp(V), 1, w.B, w.Hq, w.Hkv, w.d,
                                 vp(self.W.data_ptr()), w.L, w.P, ctypes.c_float(w.tau), vp(ids),
                                 vp(vn), vp(self.lens.data_ptr()), i64(w.n_cap),
                                 vp(self.ks.data_ptr()), self.k_max, self.sink, self.window,
                                 ctypes.c_float(w.scale), vp(self.idx.data_ptr()),
                                 vp(self.scores.data_ptr()), vp(self.out.data_ptr()),
                                 vp(self.fws_p), ctypes.c_size_t(self.fws_n), st))
            self.c_dense.append((vp(self.q.data_ptr()), vp(K), vp(V), 1, w.B, w.Hq, w.Hkv, w.d,
                                 i64(w.n_cap), vp(self.lens.data_ptr()), ctypes.c_float(w.scale),
                                 vp(self.out.data_ptr()), vp(self.xws_p),
                                 ctypes.c_size_t(self.xws_n), st))
        self.c_tables = (vp(self.q.data_ptr()), 1, w.B, w.Hq, w.Hkv, w.d, vp(self.W.data_ptr()), w.L,
                         w.P, ctypes.c_float(w.tau), i64(w.n_cap), vp(self.sws_p),
                         ctypes.c_size_t(self.sws_n), st)
        self.c_topk = (w.B, w.Hq, w.Hkv, w.L, vp(self.scores.data_ptr()), vp(self.lens.data_ptr()),
                       i64(w.n_cap), vp(self.ks.data_ptr()), self.k_max, self.sink, self.window,
                       vp(self.idx.data_ptr()),
                       vp(self.sws_p), ctypes.c_size_t(self.sws_n), st)

    @staticmethod
    def _ok(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} returned status {rc}")

    def prefill(self, r):
        self._ok(self.lib.socket_hash_keys(*self.c_prefill[r]), "socket_hash_keys")

    def step(self, r):
        """One decode step on replica r through socket_decode_step (the new key
        hashed inside the table kernel, then selection and attention)."""
        self._ok(self.lib.socket_decode_step(*self.c_fused[r]), "socket_decode_step")

    def step3(self, r):
        """The same step through the three separate C calls."""
        lib = self.lib
        rc = lib.socket_hash_keys(*self.c_append[r])
        rc |= lib.socket_score_topk(*self.c_score_topk[r])
        rc |= lib.socket_sparse_decode(*self.c_decode[r])
        if rc:
            raise RuntimeError(f"a decode-step call failed (status bits {rc})")

    STAGES = ["append", "tables", "score", "topk", "attend"]

    def stages(self, r, upto):
        """The first `upto` stages of one step on replica r, through the stage entry points."""
        lib = self.lib
        calls = [(lib.socket_hash_keys, self.c_append[r]), (lib.socket_soft_tables, self.c_tables),
                 (lib.socket_score, self.c_score[r]), (lib.socket_topk, self.c_topk),
                 (lib.socket_sparse_decode, self.c_decode[r])]
        rc = 0
        for fn, a in calls[:upto]:
            rc |= fn(*a)
        if rc:
            raise RuntimeError(f"a decode-stage call failed (status bits {rc})")

    def free(self):
        for a in ("K", "V", "ids", "vn"):
            setattr(self, a, None)


def busy_prologue(torch, ms_target=40.0):
    """Queue ~ms_target of matrix products so the launches that follow pile up
    behind them and then run back to back."""
    a = torch.randn(8192, 8192, device="cuda:0", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda:0", dtype=torch.bfloat16)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(); c = a @ b; e1.record(); torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1), 0.05)
    reps = int(math.ceil(ms_target / one))
    return lambda: [a @ b for _ in range(reps)], reps * one


def timed_steps(case, torch, steps, warmup, step=None):
    step = step or case.step
    for i in range(warmup):
        step(i % case.replicas)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i % case.replicas)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def gpu_batch_us(torch, run, count):
    """GPU microseconds per item of `count` items enqueued by run(i), all queued
    behind a busy prologue so that the events see GPU time only."""
    run_busy, busy_ms = busy_prologue(torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    run_busy()
    t0 = time.perf_counter()
    e0.record()
    for i in range(count):
        run(i)
    e1.record()
    host_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    if host_ms > busy_ms:
        log(f"[bench] warning: host enqueue {host_ms:.1f} ms exceeded the busy prologue "
            f"{busy_ms:.1f} ms; GPU times may include launch gaps")
    return e0.elapsed_time(e1) * 1e3 / count, host_ms * 1e3 / count


def per_stage(case, torch, steps):
    """GPU time of each stage: batches of `steps` steps cut after stage 1..5;
    successive differences are the stages' costs (dispatch included)."""
    cum = []
    for upto in range(1, len(case.STAGES) + 1):
        us, _ = gpu_batch_us(torch, lambda i: case.stages(i % case.replicas, upto), steps)
        cum.append(us)
    full_us, host_us = gpu_batch_us(torch, lambda i: case.step(i % case.replicas), steps)
    st = {n: cum[i] - (cum[i - 1] if i else 0.0) for i, n in enumerate(case.STAGES)}
    return st, full_us, host_us


def scorer_launch_us(case, torch, launches):
    """Average GPU time of one scorer launch (launches back to back on the replicas)."""
    lib = case.lib
    case.stages(0, 2)   # a table image for the scorer to read
    us, _ = gpu_batch_us(torch, lambda i: lib.socket_score(*case.c_score[i % case.replicas]),
                         launches)
    return us


def dense_decode(case, torch, launches):
    """The dense reference: full attention over all n + 1 keys of every query
    head, back to back on the replicas (cold caches), as GPU us per call and
    the HBM rate of its K and V reads."""
    lib = case.lib
    us, _ = gpu_batch_us(torch, lambda i: case._ok(lib.socket_dense_decode(
        *case.c_dense[i % case.replicas]), "socket_dense_decode"), launches)
    w = case.w
    kv_bytes = case.kv_keys * 2 * w.d * 2
    return dict(us=us, kv_gbs=kv_bytes / (us * 1e-6) / 1e9)


def sample_estimate(case, torch, S, M=1024):
    """The value-aware sampling estimator at the case's shape: GPU us per
    socket_sample_estimate call (tables, scores + soft-count sums, M draws per
    head and the mean of the drawn unit value rows)."""
    from soft_lsh_token_amd.inputs import uniforms
    w = case.w
    dev = "cuda:0"
    u = torch.from_numpy(uniforms(w.B, w.Hq, M, 0)).to(dev)
    out = torch.empty(w.B, w.Hq, w.d, dtype=torch.float32, device=dev)
    sc = torch.empty(w.B, w.Hq, S.score_stride(w.n_cap), dtype=torch.float32, device=dev)
    ws = S.alloc_workspace(S.socket_score_topk_workspace(w.B, w.Hq, w.Hkv, w.n_cap, w.L, w.P, 1),
                           dev)

    def run(i):
        r = i % case.replicas
        S.socket_sample_estimate(case.q, case.W, case.ids[r], case.vn[r], case.V[r], case.lens, u,
                                 w.tau, w.L, w.P, out, None, sc, ws)
    run(0)
    torch.cuda.synchronize()
    us, _ = gpu_batch_us(torch, run, 2 * case.replicas)
    return dict(draws_per_head=M, us=us)


def hard_mode(lib, torch, S, L, P, replicas):
    """Hard-LSH comparison mode at the 32K GQA shape: GPU us per
    socket_hard_score_topk call (query codes, collision-count scores, top-k),
    back to back on `replicas` copies of the code cache."""
    from soft_lsh_token_amd.inputs import make_workload
    w = make_workload("c2", steps=1, L=L, P=P)
    dev, bf = "cuda:0", torch.bfloat16
    n = int(w.lens[0])
    K = torch.from_numpy(w.K).to(dev).to(bf)
    V = torch.from_numpy(w.V).to(dev).to(bf)
    Wt = torch.from_numpy(w.W).to(dev).to(bf)
    q = torch.from_numpy(w.q).to(dev).to(bf)
    codes = S.alloc_codes(w.B, w.Hkv, w.n_cap, L, P, dev)
    vn = torch.zeros(w.B, w.Hkv, w.n_cap, dtype=torch.float32, device=dev)
    S.socket_hash_codes(K, V, Wt, codes, vn, torch.zeros(w.B, dtype=torch.int32, device=dev),
                        n + 1, L, P)
    del K, V
    reps = [codes] + [codes.clone() for _ in range(replicas - 1)]
    lens = torch.full((w.B,), n + 1, dtype=torch.int32, device=dev)
    ks = torch.from_numpy(w.ks).to(dev)
    k = int(w.ks[0])
    idx = torch.empty(w.B, w.Hq, k, dtype=torch.int32, device=dev)
    sc = torch.empty(w.B, w.Hq, S.score_stride(w.n_cap), dtype=torch.float32, device=dev)
    ws = S.alloc_workspace(S.socket_hard_score_topk_workspace(w.B, w.Hq, w.Hkv, w.n_cap, L, P, k),
                           dev)
    for r in range(replicas):
        S.socket_hard_score_topk(q, Wt, reps[r], vn, lens, ks, k, L, P, idx, sc, ws)
    torch.cuda.synchronize()
    us, _ = gpu_batch_us(torch, lambda i: S.socket_hard_score_topk(
        q, Wt, reps[i % replicas], vn, lens, ks, k, L, P, idx, sc, ws), 4 * replicas)
    code_bytes = w.B * w.Hkv * (n + 1) * (4 * S.codes_words(L, P) + 4)
    return dict(L=L, P=P, bits_per_key=L * P, score_topk_us=us,
                code_gbs=code_bytes / (us * 1e-6) / 1e9)


def prefill_rate(case, torch):
    """GPU time of one prefill hash launch (all n keys of every KV head): a batch
    of launches on the replicas in turn, queued behind the busy prologue."""
    case.prefill(0)
    torch.cuda.synchronize()
    us, _ = gpu_batch_us(torch, lambda i: case.prefill(i % case.replicas),
                         max(8, 2 * case.replicas))
    t = us * 1e-6
    w = case.w
    keys = w.B * w.Hkv * case.n
    flops = 2.0 * keys * w.d * w.L * w.P
    hbm = keys * (2 * w.d * 2 + w.L + 4)   # K and V rows read, ids and norm written
    return dict(keys=keys, seconds=t, tflops=flops / t / 1e12,
                mfma_frac=flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, hbm_gbs=hbm / t / 1e9)


def scorer_bytes(case):
    """Algorithmic bytes of one scorer launch: per KV key its L P-bit IDs (bit
    packed) and its float32 norm are read and G float32 scores are written."""
    w = case.w
    G = w.Hq // w.Hkv
    kv_keys = case.kv_keys
    return kv_keys * ((w.L * w.P + 7) // 8 + 4 + 4 * G), kv_keys


def scorer_stored_bytes(case):
    """Bytes one scorer launch moves in the cache's own layout (cells of one or
    two bytes, tables padded to 16 words per key)."""
    from soft_lsh_token_amd import layout
    w = case.w
    G = w.Hq // w.Hkv
    return case.kv_keys * (layout.key_bytes(w.L, w.P) + 4 + 4 * G)


def counters_traffic(launch_bytes):
    """HBM traffic of the scorer from committed rocprofv3 counters, if they were
    taken on the current scorer source."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
        with open(SCORER_SRC, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if c.get("source_sha256") != sha:
            return None
        return float(c["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(seconds):
    """The CPU oracle, as it stands, on a bounded sample of the 32K decode step."""
    from oracle import socket_oracle as SO
    from soft_lsh_token_amd.inputs import make_workload
    w = make_workload("c2", steps=1)
    n = int(w.lens[0])
    log("[bench] cpu baseline: oracle prefill hash (untimed)")
    ids = np.empty((w.B, w.Hkv, w.n_cap, w.L), dtype=np.int64)
    for h in range(w.Hkv):
        ids[0, h, :n] = SO.hash_keys(w.K[0, h, :n], w.W, w.L, w.P)[0]
    vn = np.zeros((w.B, w.Hkv, w.n_cap))
    vn[0, :, :n] = SO.value_norms(w.V[0, :, :n])
    lens = np.array([n + 1], dtype=np.int32)
    # one step = append hash of the new key of every KV head + the decode step
    # (tables, scores, top-k, attention); the sample is as many query heads of
    # successive steps as fit in the time budget
    heads_done, t_used, c_used = 0, 0.0, 0.0
    group = w.Hq // w.Hkv
    while t_used < seconds and heads_done < 64 * w.Hq:
        g = heads_done % w.Hq
        h = g // group
        c0, t0 = time.process_time(), time.perf_counter()
        ids[0, h, n] = SO.hash_keys(w.K[0, h, n:n + 1], w.W, w.L, w.P)[0][0]
        vn[0, h, n] = SO.value_norms(w.V[0, h, n])
        tab = SO.soft_tables(w.q[0, g], w.W, w.L, w.P, w.tau)
        s = SO.scores(tab[None, None], ids[:, h:h + 1], vn[:, h:h + 1], lens)[0, 0]
        sel = SO.topk(s, int(w.ks[0]), n + 1)
        SO.sparse_attention(w.q[0, g], w.K[0, h], w.V[0, h], sel, w.scale)
        t_used += time.perf_counter() - t0
        c_used += time.process_time() - c0
        heads_done += 1
    keys = heads_done * (n + 1)
    cores = max(1, int(round(c_used / max(t_used, 1e-9))))
    return dict(value=keys / t_used, unit="keys/s", cores=cores, kind="oracle",
                sample=f"{heads_done} query heads x {n + 1} keys of the 32K decode step "
                       f"(append hash + tables + scores + top-k + attention per head), "
                       f"{t_used:.1f}s wall; host affinity {len(os.sched_getaffinity(0))} cpus")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path has "
              f"no multi-GPU mode: every run uses exactly one GPU).", file=sys.stderr)
        sys.exit(2)
    import torch
    import soft_lsh_token_amd as S
    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible; bench.py needs an MI355X")
    lib = S.lib()
    torch.cuda.set_device(0)
    if args.copy_calibration:
        nb = args.copy_calibration << 20
        src = torch.empty(nb, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.copy_calibration} MiB done")
        del src, dst

    case = Case("c2", args.replicas, lib, torch, S)
    for r in range(case.replicas):
        case.prefill(r)
    torch.cuda.synchronize()
    pre32 = prefill_rate(case, torch)
    log(f"[bench] prefill hash 32K: {pre32}")
    sec = timed_steps(case, torch, args.steps, args.warmup)
    log(f"[bench] 32K step wall {sec * 1e6:.1f} us")
    sec3 = timed_steps(case, torch, args.steps, args.warmup, case.step3)
    log(f"[bench] 32K step wall through the three calls {sec3 * 1e6:.1f} us")
    stages, gpu_step_us, host_step_us = per_stage(case, torch, min(args.steps, 200))
    log(f"[bench] 32K per-stage GPU us {stages}; full step GPU {gpu_step_us:.1f} us; "
        f"host enqueue {host_step_us:.1f} us/step")
    score_us = scorer_launch_us(case, torch, 4 * case.replicas)
    log(f"[bench] 32K scorer launch {score_us:.2f} us")
    dense32 = dense_decode(case, torch, 2 * case.replicas)
    dense32["socket_speedup"] = dense32["us"] / gpu_step_us
    log(f"[bench] 32K dense decode {dense32}")
    est32 = sample_estimate(case, torch, S)
    log(f"[bench] 32K sampling estimator {est32}")
    launch_bytes, kv_keys = scorer_bytes(case)
    achieved = launch_bytes / (score_us * 1e-6) / 1e9
    traffic = counters_traffic(launch_bytes)
    w = case.w
    keys_per_step = case.kv_keys * (w.Hq // w.Hkv)
    extra32 = dict(
        step_us_wall=sec * 1e6, step_us_wall_three_calls=sec3 * 1e6,
        step_us_gpu=gpu_step_us, host_enqueue_us_per_step=host_step_us,
        stage_us=stages, scorer_launch_us=score_us,
        score_topk_us=stages["tables"] + stages["score"] + stages["topk"],
        prefill=pre32, dense_decode=dense32, sampling_estimator=est32)
    case.free()
    del case
    torch.cuda.empty_cache()

    extra128 = None
    if not args.no_128k:
        c3 = Case("c3", max(4, args.replicas // 5), lib, torch, S)
        for r in range(c3.replicas):
            c3.prefill(r)
        torch.cuda.synchronize()
        pre128 = prefill_rate(c3, torch)
        log(f"[bench] prefill hash 128K (the decode-loop prefill): {pre128}")
        sec3 = timed_steps(c3, torch, args.steps, args.warmup)
        st3, gpu3, host3 = per_stage(c3, torch, max(20, args.steps // 4))
        sc3 = scorer_launch_us(c3, torch, 4 * c3.replicas)
        lb3, _ = scorer_bytes(c3)
        dense128 = dense_decode(c3, torch, 4 * c3.replicas)
        dense128["socket_speedup"] = dense128["us"] / gpu3
        extra128 = dict(step_us_wall=sec3 * 1e6, step_us_gpu=gpu3, stage_us=st3,
                        scorer_launch_us=sc3,
                        keys_per_s=c3.kv_keys * (c3.w.Hq // c3.w.Hkv) / sec3,
                        scorer_gbs=lb3 / (sc3 * 1e-6) / 1e9,
                        prefill=pre128, dense_decode=dense128)
        log(f"[bench] 128K: {extra128}")
        c3.free()
        del c3
        torch.cuda.empty_cache()

    hard = None
    if not args.no_hard:
        hard = [hard_mode(lib, torch, S, L, 2, 16) for L in (300, 500)]
        for h in hard:
            h["soft_score_topk_us"] = extra32["score_topk_us"]
        log(f"[bench] 32K hard-LSH mode: {hard}")
        torch.cuda.empty_cache()
    extra32["hard_lsh"] = hard

    extra_p10 = None
    if not args.no_p10:
        c10 = Case("c2", max(8, args.replicas // 2), lib, torch, S, L=60, P=10)
        for r in range(c10.replicas):
            c10.prefill(r)
        torch.cuda.synchronize()
        pre10 = prefill_rate(c10, torch)
        sec10 = timed_steps(c10, torch, args.steps, args.warmup)
        st10, gpu10, _ = per_stage(c10, torch, max(50, args.steps // 2))
        sc10 = scorer_launch_us(c10, torch, 4 * c10.replicas)
        lb10, _ = scorer_bytes(c10)
        extra_p10 = dict(step_us_wall=sec10 * 1e6, step_us_gpu=gpu10, stage_us=st10,
                         scorer_launch_us=sc10,
                         keys_per_s=c10.kv_keys * (c10.w.Hq // c10.w.Hkv) / sec10,
                         scorer_gbs_algorithmic=lb10 / (sc10 * 1e-6) / 1e9,
                         scorer_gbs_stored=scorer_stored_bytes(c10) / (sc10 * 1e-6) / 1e9,
                         prefill=pre10)
        log(f"[bench] 32K at P=10, L=60: {extra_p10}")
        c10.free()
        del c10
        torch.cuda.empty_cache()

    extra_b16 = None
    if not args.no_batched:
        c4 = Case("c4", 2, lib, torch, S)
        for r in range(c4.replicas):
            c4.prefill(r)
        torch.cuda.synchronize()
        sec4 = timed_steps(c4, torch, args.steps, args.warmup)
        st4, gpu4, _ = per_stage(c4, torch, max(20, args.steps // 4))
        sc4 = scorer_launch_us(c4, torch, 8 * c4.replicas)
        lb4, kk4 = scorer_bytes(c4)
        dense4 = dense_decode(c4, torch, 4 * c4.replicas)
        dense4["socket_speedup"] = dense4["us"] / gpu4
        lens4 = c4.w.lens
        extra_b16 = dict(sequences=int(c4.w.B), lens_min=int(lens4.min()),
                         lens_max=int(lens4.max()), kv_keys=kk4,
                         step_us_wall=sec4 * 1e6, step_us_gpu=gpu4, stage_us=st4,
                         keys_per_s=c4.kv_keys * (c4.w.Hq // c4.w.Hkv) / sec4,
                         scorer_launch_us=sc4, scorer_gbs=lb4 / (sc4 * 1e-6) / 1e9,
                         scorer_hbm_frac=lb4 / (sc4 * 1e-6) / 1e9 / HBM_PEAK_GBS,
                         dense_decode=dense4)
        log(f"[bench] 16 ragged sequences: {extra_b16}")
        c4.free()
        del c4
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_seconds)
        log(f"[bench] cpu baseline: {cpu}")

    line = {
        "metric": "keys scored+selected/s per GPU (32K-key GQA decode step)",
        "value": keys_per_step / sec,
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "GQA 32/8 decode step, n=32768 (+1 appended key), d=128, L=64, "
                               "P=8, tau=0.5, k=656, batch 1",
                   "global_batch": 1, "seq_len": 32768, "parallelism": "single GPU",
                   "replicas": args.replicas},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "scorer_kernel (soft-count scores + first-digit histogram)",
                     "bytes_per_launch": launch_bytes, "kv_keys_per_launch": kv_keys},
        "cpu_baseline": cpu,
        "extra": {"ctx32k": extra32, "ctx128k": extra128, "ctx32k_p10_l60": extra_p10,
                  "batch16_ragged": extra_b16},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
