"""Benchmark of the SOCKET decode hot path on one MI355X.

One step = one decode step of the GQA 32/8 workload at n = 32768 cached keys
(d = 128, L = 64 tables x P = 8 planes, tau = 0.5, k = 656 = ceil(2% of n)):
the new key of every KV head is hashed and its value norm stored, then soft
tables, soft-count scores of all n + 1 keys for the 32 query heads, the
top-656 per query head and exact attention over them -- one
socket_decode_step call (the same step through the three calls
socket_hash_keys, socket_score_topk and socket_sparse_decode is reported
beside it).

`value` is keys scored+selected per second: 32 query heads x (n + 1) keys per
step, divided by the wall time of K steps bracketed by device syncs.  Inputs
are resident in HBM.  The cache is replicated `--replicas` times (one replica
per step, round robin, like successive layers) so the 256 MiB Infinity Cache
cannot serve a step from the previous one.

`roofline` is the selection stage (soft tables + scores + top-k, one
socket_score_topk call) at 32K: its algorithmic bytes (per KV-key the L*P-bit
IDs and the float32 norm read and G float32 scores written; per query-key the
score read back by the top-k) over its average GPU time in a batch of calls
timed with HIP events on the library's stream.

Also reported: per-stage GPU time (batches of steps cut after each stage,
timed with one pair of HIP events per batch while the launches queue behind a
long matrix product, so host launch gaps stay out; a stage's time includes
its dispatch), the step replayed from a captured HIP graph (one step per
replica in one graph), the scorer alone, the 128K-key step, the 128K prefill hashing
(fused with the norms; IDs only against the bf16 MFMA peak; norms only against
HBM), the prefill + 256-step decode loop at 128K, the comparison modes, and
the CPU oracle on bounded samples.

`--only NAME` runs a few launches of one kernel group and exits (for
rocprofv3 counter runs): prefill128k (IDs only), prefill128k-fused,
norms128k, stage32k, stage128k, step32k, step128k.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.json")


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
    p.add_argument("--loop-steps", type=int, default=256,
                   help="decode steps of the 128K prefill + decode loop")
    p.add_argument("--only", default=None, metavar="NAME",
                   help="run a few launches of one kernel group and exit (counter runs): "
                        "prefill128k, prefill128k-fused, norms128k, stage32k, stage128k, step32k, step128k")
    p.add_argument("--crossover", action="store_true",
                   help="only time the decode step against the dense decode at 32K-128K keys "
                        "(GQA 32/8, L = 64, P = 8, k = 2%%) and print one JSON line")
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
        self.c_prefill_ids, self.c_prefill_norms = [], []
        for r in range(self.replicas):
            K, V, ids, vn = self.K[r].data_ptr(), self.V[r].data_ptr(), self.ids[r].data_ptr(), \
                self.vn[r].data_ptr()
            common = (vp(K), vp(V), 1, w.B, w.Hkv, w.d, i64(w.n_cap))
            self.c_prefill.append(common + (vp(self.pos_prefill.data_ptr()), self.n,
                                             vp(self.W.data_ptr()), w.L, w.P, vp(ids), vp(vn), st))
            # the same prefill split in two: bucket IDs only, value norms only
            self.c_prefill_ids.append((vp(K), None, 1, w.B, w.Hkv, w.d, i64(w.n_cap),
                                       vp(self.pos_prefill.data_ptr()), self.n,
                                       vp(self.W.data_ptr()), w.L, w.P, vp(ids), None, st))
            self.c_prefill_norms.append((None, vp(V), 1, w.B, w.Hkv, w.d, i64(w.n_cap),
                                         vp(self.pos_prefill.data_ptr()), self.n, None, w.L, w.P,
                                         None, vp(vn), st))
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

    def prefill(self, r, mode="fused"):
        c = {"fused": self.c_prefill, "ids": self.c_prefill_ids, "norms": self.c_prefill_norms}[mode]
        self._ok(self.lib.socket_hash_keys(*c[r]), "socket_hash_keys")

    def score_topk(self, r):
        """The selection stage alone: soft tables, scores, top-k."""
        self._ok(self.lib.socket_score_topk(*self.c_score_topk[r]), "socket_score_topk")

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


def graph_steps(case, torch, replays=50):
    """GPU us per decode step when the steps run from a captured HIP graph: one
    graph holds one socket_decode_step per replica (successive layers of a
    serving loop), captured on a side stream with the case's workspace (the
    step allocates nothing), then replayed behind the busy prologue."""
    s = torch.cuda.Stream()
    vp = ctypes.c_void_p
    args = [tuple(c[:-1]) + (vp(s.cuda_stream),) for c in case.c_fused]
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for a in args:  # warm-up on the capture stream
            case._ok(case.lib.socket_decode_step(*a), "socket_decode_step")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for a in args:
            case._ok(case.lib.socket_decode_step(*a), "socket_decode_step")
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    us, _ = gpu_batch_us(torch, lambda i: g.replay(), replays)
    del g
    return us / len(args)


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
    zeros = torch.zeros(w.B, dtype=torch.int32, device=dev)
    S.socket_hash_codes(K, V, Wt, codes, vn, zeros, n + 1, L, P)
    torch.cuda.synchronize()
    # prefill: codes and norms of all n + 1 keys of every KV head
    hash_us, _ = gpu_batch_us(torch, lambda i: S.socket_hash_codes(
        K, V, Wt, codes, vn, zeros, n + 1, L, P), 8)
    keys = w.B * w.Hkv * (n + 1)
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
    key_bytes = 4 * S.codes_words(L, P) + 4  # code words + value norm
    code_bytes = keys * key_bytes
    flops = 2.0 * keys * w.d * L * P
    return dict(L=L, P=P, bits_per_key=L * P, cache_bytes_per_key=key_bytes,
                score_topk_us=us, code_gbs=code_bytes / (us * 1e-6) / 1e9,
                hash_prefill=dict(keys=keys, us=hash_us, tflops=flops / (hash_us * 1e-6) / 1e12,
                                  mfma_frac=flops / (hash_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS))


def prefill_rate(case, torch, mode="fused"):
    """GPU time of one prefill launch (all n keys of every KV head): a batch of
    launches on the replicas in turn, queued behind the busy prologue.  mode
    'fused' hashes and stores the norms, 'ids' hashes only (the bf16 MFMA
    GEMM, against the MFMA peak), 'norms' stores the norms only (against HBM)."""
    case.prefill(0, mode)
    torch.cuda.synchronize()
    us, _ = gpu_batch_us(torch, lambda i: case.prefill(i % case.replicas, mode),
                         max(8, 2 * case.replicas))
    t = us * 1e-6
    w = case.w
    keys = w.B * w.Hkv * case.n
    flops = 2.0 * keys * w.d * w.L * w.P
    from soft_lsh_token_amd import layout
    id_bytes = layout.key_bytes(w.L, w.P)
    k_bytes = w.d * 2
    hbm = {"fused": keys * (2 * k_bytes + id_bytes + 4), "ids": keys * (k_bytes + id_bytes),
           "norms": keys * (k_bytes + 4)}[mode]
    r = dict(mode=mode, keys=keys, us=us, hbm_gbs=hbm / t / 1e9, hbm_frac=hbm / t / 1e9 / HBM_PEAK_GBS)
    if mode != "norms":
        r.update(tflops=flops / t / 1e12, mfma_frac=flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS)
    return r


def scorer_bytes(case):
    """Algorithmic bytes of one scorer launch: per KV key its L P-bit IDs (bit
    packed) and its float32 norm are read and G float32 scores are written."""
    w = case.w
    G = w.Hq // w.Hkv
    kv_keys = case.kv_keys
    return kv_keys * ((w.L * w.P + 7) // 8 + 4 + 4 * G), kv_keys


def stage_bytes(case):
    """Algorithmic bytes of one selection stage (soft tables + scores + top-k):
    the scorer's, plus every query-key's score read back by the top-k (the
    tables' and indices' few kilobytes are left out)."""
    launch, kv_keys = scorer_bytes(case)
    w = case.w
    return launch + 4 * kv_keys * (w.Hq // w.Hkv), kv_keys


def scorer_stored_bytes(case):
    """Bytes one scorer launch moves in the cache's own layout (cells of one or
    two bytes, tables padded to 16 words per key)."""
    from soft_lsh_token_amd import layout
    w = case.w
    G = w.Hq // w.Hkv
    return case.kv_keys * (layout.key_bytes(w.L, w.P) + 4 + 4 * G)


def stage_launch_us(case, torch, calls):
    """Average GPU time of one socket_score_topk call (its three launches back
    to back on the replicas, after a warm call)."""
    case.score_topk(0)
    torch.cuda.synchronize()
    us, _ = gpu_batch_us(torch, lambda i: case.score_topk(i % case.replicas), calls)
    return us


def _sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def counters_traffic(name):
    """HBM bytes per call of a kernel group from committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE counters, if they were taken on the current sources (else None)."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)[name]
        for rel, sha in c["sources"].items():
            if _sha(os.path.join(ROOT, rel)) != sha:
                return None
        return float(c["hbm_bytes_per_call"])
    except (OSError, KeyError, ValueError, TypeError):
        return None


def roofline_entry(name, bytes_, us, kernel, extra=None):
    gbs = bytes_ / (us * 1e-6) / 1e9
    r = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": gbs / HBM_PEAK_GBS, "traffic": counters_traffic(name), "kernel": kernel,
         "bytes_per_call": bytes_, "us_per_call": us}
    r.update(extra or {})
    return r


def decode_loop_c5(lib, torch, S, steps):
    """Prefill 131072 keys x 8 KV heads, then `steps` decode steps, each
    appending one key and value per KV head (socket_decode_step), with a fresh
    query per step.  Per-step GPU times from HIP events around each step on
    the library's stream (the host enqueues faster than the GPU runs, so the
    events see GPU time)."""
    from soft_lsh_token_amd.inputs import make_workload
    t0 = time.time()
    w = make_workload("c5", steps=steps)
    log(f"[bench] c5: inputs drawn in {time.time() - t0:.1f}s (n={int(w.lens[0])}, "
        f"n_cap={w.n_cap}, steps={steps})")
    dev, bf = "cuda:0", torch.bfloat16
    K = torch.from_numpy(w.K).to(dev).to(bf)
    V = torch.from_numpy(w.V).to(dev).to(bf)
    W = torch.from_numpy(w.W).to(dev).to(bf)
    qs = torch.from_numpy(w.q_steps).to(dev).to(bf)
    n0 = int(w.lens[0])
    ids = S.alloc_ids(w.B, w.Hkv, w.n_cap, w.L, w.P, dev)
    vn = torch.zeros(w.B, w.Hkv, w.n_cap, dtype=torch.float32, device=dev)
    pos0 = torch.zeros(w.B, dtype=torch.int32, device=dev)
    lens_all = torch.arange(n0 + 1, n0 + steps + 1, dtype=torch.int32, device=dev).view(steps, 1)
    ks = torch.from_numpy(w.ks).to(dev)
    k_max = int(w.ks.max())
    idx = torch.empty(w.B, w.Hq, k_max, dtype=torch.int32, device=dev)
    out = torch.empty(w.B, w.Hq, w.d, dtype=torch.float32, device=dev)
    ws = S.alloc_workspace(S.socket_decode_step_workspace(w.B, w.Hq, w.Hkv, w.n_cap, w.L, w.P,
                                                          k_max), dev)
    stream = torch.cuda.current_stream()

    def run_once():
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 2)]
        torch.cuda.synchronize()
        t_host = time.perf_counter()
        ev[0].record(stream)
        S.socket_hash_keys(K, V, W, ids, vn, pos0, n0, w.L, w.P)
        ev[1].record(stream)
        for t in range(steps):
            S.socket_decode_step(qs[t], K, V, W, ids, vn, lens_all[t], ks, k_max, w.tau, w.L, w.P,
                                 w.scale, idx, out, ws=ws)
            ev[t + 2].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_host
        return ev, wall

    run_once()  # warm (the first launches of each kernel)
    ev, wall = run_once()
    pre_us = ev[0].elapsed_time(ev[1]) * 1e3
    st = np.array([ev[t + 1].elapsed_time(ev[t + 2]) * 1e3 for t in range(steps)])
    total_ms = ev[0].elapsed_time(ev[-1])
    keys = sum(w.Hq * (n0 + t + 1) for t in range(steps))
    r = dict(prefill_keys=w.B * w.Hkv * n0, steps=steps, prefill_us=pre_us,
             step_us_median=float(np.median(st)), step_us_p95=float(np.percentile(st, 95)),
             step_us_mean=float(st.mean()), step_us_first=float(st[0]), step_us_last=float(st[-1]),
             total_ms=total_ms, wall_ms=wall * 1e3,
             decode_keys_per_s=keys / (st.sum() * 1e-6))
    del K, V, ids, vn, ws
    torch.cuda.empty_cache()
    return r


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("user_api") == "blas"] or [1])
    except Exception:
        return None


def cpu_baseline(seconds):
    """The CPU oracle, as it stands, on bounded samples: (1) query heads of the
    32K decode step, one after another, each with the append hash of its KV
    head's new key, its soft tables, scores, top-k and attention, timed per
    stage (the rate is `value`); (2) the prefill + decode loop at 128K: the
    oracle hashes all 131072 x 8 keys, then runs decode steps 0, 1, 2, 127 and
    255 for the four query heads of KV head 0 (with every KV head's appended
    key), timed per stage.  numpy runs the prefill's matrix products on its
    BLAS threads and everything else on one thread."""
    from oracle import socket_oracle as SO
    from soft_lsh_token_amd.inputs import make_workload
    blas = _blas_threads()
    aff = len(os.sched_getaffinity(0))
    w = make_workload("c2", steps=1)
    n = int(w.lens[0])
    log("[bench] cpu baseline: oracle prefill hash of the 32K cache (untimed)")
    ids = np.empty((w.B, w.Hkv, w.n_cap, w.L), dtype=np.int64)
    for h in range(w.Hkv):
        ids[0, h, :n] = SO.hash_keys(w.K[0, h, :n], w.W, w.L, w.P)[0]
    vn = np.zeros((w.B, w.Hkv, w.n_cap))
    vn[0, :, :n] = SO.value_norms(w.V[0, :, :n])
    lens = np.array([n + 1], dtype=np.int32)
    stage = dict(append=0.0, tables=0.0, scores=0.0, topk=0.0, attend=0.0)
    heads_done, t_used = 0, 0.0
    group = w.Hq // w.Hkv
    budget = 0.6 * seconds
    while t_used < budget and heads_done < 64 * w.Hq:
        g = heads_done % w.Hq
        h = g // group
        t0 = time.perf_counter()
        ids[0, h, n] = SO.hash_keys(w.K[0, h, n:n + 1], w.W, w.L, w.P)[0][0]
        vn[0, h, n] = SO.value_norms(w.V[0, h, n])
        t1 = time.perf_counter()
        tab = SO.soft_tables(w.q[0, g], w.W, w.L, w.P, w.tau)
        t2 = time.perf_counter()
        s = SO.scores(tab[None, None], ids[:, h:h + 1], vn[:, h:h + 1], lens)[0, 0]
        t3 = time.perf_counter()
        sel = SO.topk(s, int(w.ks[0]), n + 1)
        t4 = time.perf_counter()
        SO.sparse_attention(w.q[0, g], w.K[0, h], w.V[0, h], sel, w.scale)
        t5 = time.perf_counter()
        for key, a, b in (("append", t0, t1), ("tables", t1, t2), ("scores", t2, t3),
                          ("topk", t3, t4), ("attend", t4, t5)):
            stage[key] += b - a
        t_used += t5 - t0
        heads_done += 1
    keys = heads_done * (n + 1)
    per_head_ms = {k: v / heads_done * 1e3 for k, v in stage.items()}

    # the 128K prefill + decode loop, steps {0, 1, 2, 127, 255} of KV head 0's query heads
    w5 = make_workload("c5")
    n0 = int(w5.lens[0])
    t0 = time.perf_counter()
    ids5 = np.empty((w5.Hkv, w5.n_cap, w5.L), dtype=np.int64)
    vn5 = np.zeros((w5.Hkv, w5.n_cap))
    for h in range(w5.Hkv):
        ids5[h, :n0] = SO.hash_keys(w5.K[0, h, :n0], w5.W, w5.L, w5.P)[0]
    t1 = time.perf_counter()
    vn5[:, :n0] = SO.value_norms(w5.V[0, :, :n0])
    t2 = time.perf_counter()
    loop = dict(append=0.0, tables=0.0, scores=0.0, topk=0.0, attend=0.0)
    check = [0, 1, 2, 127, 255]
    # keys appended at steps the sample skips are hashed untimed
    for t in range(w5.steps):
        if t in check:
            continue
        for h in range(w5.Hkv):
            ids5[h, n0 + t] = SO.hash_keys(w5.K[0, h, n0 + t:n0 + t + 1], w5.W, w5.L, w5.P)[0][0]
            vn5[h, n0 + t] = SO.value_norms(w5.V[0, h, n0 + t])
    for t in check:
        nt = n0 + t + 1
        a0 = time.perf_counter()
        for h in range(w5.Hkv):
            ids5[h, n0 + t] = SO.hash_keys(w5.K[0, h, n0 + t:n0 + t + 1], w5.W, w5.L, w5.P)[0][0]
            vn5[h, n0 + t] = SO.value_norms(w5.V[0, h, n0 + t])
        a1 = time.perf_counter()
        tab = SO.soft_tables(w5.q_steps[t][0, :group], w5.W, w5.L, w5.P, w5.tau)
        a2 = time.perf_counter()
        s5 = SO.scores(tab[None], ids5[None, :1], vn5[None, :1], np.array([nt]))[0]
        a3 = time.perf_counter()
        sels = [SO.topk(s5[g], int(w5.ks[0]), nt) for g in range(group)]
        a4 = time.perf_counter()
        for g in range(group):
            SO.sparse_attention(w5.q_steps[t][0, g], w5.K[0, 0], w5.V[0, 0], sels[g], w5.scale)
        a5 = time.perf_counter()
        for key, a, b in (("append", a0, a1), ("tables", a1, a2), ("scores", a2, a3),
                          ("topk", a3, a4), ("attend", a4, a5)):
            loop[key] += b - a
    loop_s = sum(loop.values())
    c5 = dict(prefill_hash_s=t1 - t0, prefill_norms_s=t2 - t1, prefill_keys=w5.Hkv * n0,
              steps=check, heads_per_step=group,
              step_stage_ms={k: v / len(check) * 1e3 for k, v in loop.items()},
              step_ms_4_heads=loop_s / len(check) * 1e3,
              step_ms_all_heads_scaled=loop_s / len(check) * 1e3 * w5.Hq / group)
    return dict(value=keys / t_used, unit="keys/s", cores=blas or 1, kind="oracle",
                sample=f"{heads_done} query heads x {n + 1} keys of the 32K decode step, one "
                       f"after another (append hash + tables + scores + top-k + attention per "
                       f"head; numpy, one thread), {t_used:.1f}s; then the 128K prefill "
                       f"(matrix products on {blas} BLAS threads) and decode steps "
                       f"0/1/2/127/255 for 4 query heads; host affinity {aff} cpus",
                blas_threads=blas, affinity_cpus=aff, per_head_stage_ms_32k=per_head_ms,
                decode_loop_128k=c5)


def crossover(args, lib, torch, S):
    """Decode step (socket_decode_step) against the dense decode of the same
    32/8 GQA shape as n grows: GPU us per call over batches of calls on 8
    replicas (cold caches), and the speedup of the sparse step."""
    rows = []
    for n in (32768, 49152, 65536, 98304, 131072):
        case = Case("c2", 8, lib, torch, S, n=n, k=0.02)
        for r in range(case.replicas):
            case.prefill(r)
        torch.cuda.synchronize()
        timed_steps(case, torch, 40, 40)  # warm-up: the first steps after a prefill run slow
        step_us, _ = gpu_batch_us(torch, lambda i: case.step(i % case.replicas), 100)
        dense_decode(case, torch, case.replicas)
        dense = dense_decode(case, torch, 2 * case.replicas)
        row = dict(n=n, k=case.k, step_us=step_us, dense_us=dense["us"],
                   speedup=dense["us"] / step_us)
        log(f"[bench] crossover {row}")
        rows.append(row)
        case.free()
        del case
        torch.cuda.empty_cache()
    print(json.dumps({"crossover": rows}), flush=True)


def only(args, lib, torch, S):
    """A few launches of one kernel group, for counter runs; prints what ran."""
    name = args.only
    reps = 4
    if name in ("prefill128k", "prefill128k-fused", "norms128k"):
        case = Case("c3", reps, lib, torch, S)
        mode = {"prefill128k": "ids", "prefill128k-fused": "fused", "norms128k": "norms"}[name]
        for i in range(2 * reps):
            case.prefill(i % reps, mode)
    elif name in ("stage32k", "stage128k", "step32k", "step128k"):
        case = Case("c3" if name.endswith("128k") else "c2", reps, lib, torch, S)
        for r in range(reps):
            case.prefill(r)
        torch.cuda.synchronize()
        for i in range(4 * reps):
            if name.startswith("step"):
                case.step(i % reps)
            else:
                case.score_topk(i % reps)
    else:
        raise SystemExit(f"unknown --only {name}")
    torch.cuda.synchronize()
    print(json.dumps({"only": name, "calls": 4 * reps if name.startswith(("stage", "step"))
                      else 2 * reps}), flush=True)


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
    if args.only:
        only(args, lib, torch, S)
        return
    if args.crossover:
        crossover(args, lib, torch, S)
        return

    # ---- 32K: the timed step, its stages, the selection stage's roofline
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
    stages, gpu_step_us, host_step_us = per_stage(case, torch, min(max(args.steps, 50), 200))
    log(f"[bench] 32K per-stage GPU us {stages}; full step GPU {gpu_step_us:.1f} us; "
        f"host enqueue {host_step_us:.1f} us/step")
    graph_us = graph_steps(case, torch)
    log(f"[bench] 32K step from a captured HIP graph {graph_us:.1f} us (GPU)")
    stage_us = stage_launch_us(case, torch, 4 * case.replicas)
    score_us = scorer_launch_us(case, torch, 4 * case.replicas)
    log(f"[bench] 32K selection stage {stage_us:.2f} us, scorer launch {score_us:.2f} us")
    dense32 = dense_decode(case, torch, 2 * case.replicas)
    dense32["socket_speedup"] = dense32["us"] / gpu_step_us
    log(f"[bench] 32K dense decode {dense32}")
    est32 = sample_estimate(case, torch, S)
    log(f"[bench] 32K sampling estimator {est32}")
    sbytes, kv_keys = stage_bytes(case)
    lbytes, _ = scorer_bytes(case)
    w = case.w
    keys_per_step = case.kv_keys * (w.Hq // w.Hkv)
    roof = roofline_entry(
        "stage_c2", sbytes, stage_us,
        "selection stage at 32K: soft_tables_kernel + scorer_kernel + topk_stream_kernel "
        "(one socket_score_topk call)", {"kv_keys_per_call": kv_keys})
    extra32 = dict(
        step_us_wall=sec * 1e6, step_us_wall_three_calls=sec3 * 1e6,
        step_us_gpu=gpu_step_us, step_us_graph=graph_us, host_enqueue_us_per_step=host_step_us,
        stage_us=stages, selection_stage_us=stage_us, scorer_launch_us=score_us,
        scorer_roofline=roofline_entry("scorer_c2", lbytes, score_us, "scorer_kernel at 32K"),
        prefill=pre32, dense_decode=dense32, sampling_estimator=est32,
        id_bytes_per_key=S.layout.key_bytes(w.L, w.P))
    case.free()
    del case
    torch.cuda.empty_cache()

    # ---- 128K: the step, its stages, the prefill split into IDs and norms
    extra128 = None
    if not args.no_128k:
        c3 = Case("c3", max(4, args.replicas // 5), lib, torch, S)
        for r in range(c3.replicas):
            c3.prefill(r)
        torch.cuda.synchronize()
        prefill = {m: prefill_rate(c3, torch, m) for m in ("fused", "ids", "norms")}
        log(f"[bench] prefill 128K (the decode loop's): {prefill}")
        sec3 = timed_steps(c3, torch, args.steps, args.warmup)
        st3, gpu3, _ = per_stage(c3, torch, max(20, args.steps // 4))
        graph3 = graph_steps(c3, torch, 20)
        stage3 = stage_launch_us(c3, torch, 4 * c3.replicas)
        sc3 = scorer_launch_us(c3, torch, 4 * c3.replicas)
        sb3, _ = stage_bytes(c3)
        lb3, _ = scorer_bytes(c3)
        dense128 = dense_decode(c3, torch, 4 * c3.replicas)
        dense128["socket_speedup"] = dense128["us"] / gpu3
        extra128 = dict(step_us_wall=sec3 * 1e6, step_us_gpu=gpu3, step_us_graph=graph3,
                        stage_us=st3,
                        selection_stage_us=stage3, scorer_launch_us=sc3,
                        keys_per_s=c3.kv_keys * (c3.w.Hq // c3.w.Hkv) / sec3,
                        selection_roofline=roofline_entry(
                            "stage_c3", sb3, stage3, "selection stage at 128K (soft_tables_kernel"
                            " + scorer_kernel + topk_scan_kernel + topk_resolve_kernel)"),
                        scorer_roofline=roofline_entry("scorer_c3", lb3, sc3,
                                                       "scorer_kernel at 128K"),
                        prefill=prefill, dense_decode=dense128)
        log(f"[bench] 128K: {extra128}")
        c3.free()
        del c3
        torch.cuda.empty_cache()

    # ---- the prefill + 256-step decode loop at 128K
    loop5 = None
    if not args.no_128k:
        loop5 = decode_loop_c5(lib, torch, S, args.loop_steps)
        log(f"[bench] 128K prefill + decode loop: {loop5}")

    hard = None
    if not args.no_hard:
        hard = [hard_mode(lib, torch, S, L, 2, 16) for L in (300, 500)]
        for h in hard:  # the soft path beside it, as SOCKET Table 3 sets them side by side
            h["soft_score_topk_us"] = extra32["selection_stage_us"]
            h["soft_cache_bytes_per_key"] = extra32["id_bytes_per_key"] + 4
            h["soft_hash_prefill_us"] = extra32["prefill"]["us"]
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
        from soft_lsh_token_amd import layout
        extra_p10 = dict(step_us_wall=sec10 * 1e6, step_us_gpu=gpu10, stage_us=st10,
                         scorer_launch_us=sc10,
                         keys_per_s=c10.kv_keys * (c10.w.Hq // c10.w.Hkv) / sec10,
                         id_bytes_per_key=layout.key_bytes(60, 10),
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
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": {"hash_mfma_frac_128k": None if extra128 is None
                  else extra128["prefill"]["ids"]["mfma_frac"],
                  "ctx32k": extra32, "ctx128k": extra128, "decode_loop_128k": loop5,
                  "ctx32k_p10_l60": extra_p10, "batch16_ragged": extra_b16},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
