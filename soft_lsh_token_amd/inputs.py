"""Seeded synthetic inputs for the SOCKET decode path.

This module only draws random numbers and rounds them to their storage
dtype.  It holds none of the method's arithmetic (no hashing, no tables, no
scores, no attention), so both the CPU oracle and the HIP path can consume
exactly the same arrays.

Workloads (SOCKET, "SOft Collision Kernel EsTimator for Sparse Attention",
Section 6 evaluates 32K-128K contexts at 5x-50x sparsity; the datasets and
model weights are not available, so these synthetic tensors stand in for
them at the same shapes):

* ``c1`` single head, n=4096, d=128, fp32 K/V/q ~ N(0,1); L=32, P=8,
  tau=0.5, k=128.
* ``c2`` GQA 32 query / 8 KV heads, d=128, n=32768, bf16.  Keys are
  N(0,1) plus a per-KV-head mean offset of norm 3 (anisotropic keys);
  values are N(0,1) rows scaled per token by lognormal(0, 0.5); queries
  N(0,1); L=64, P=8, tau=0.5, k=656 (= ceil(2% of n)).
* ``c3`` as ``c2`` with n=131072 and k=1024.
* ``c4`` 16 sequences with lengths uniform in [8192, 32768], k_b =
  ceil(2% of n_b), otherwise as ``c2``.
* ``c5`` prefill of 131072 keys per KV head, then ``steps`` decode steps,
  each appending one key/value per KV head and drawing a fresh query;
  k=1024.

All host arrays are float32 numpy arrays whose values are exactly
representable in the storage dtype (bf16 values are rounded once, round to
nearest even, by torch's CPU conversion).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "CONFIGS", "make_workload", "to_bf16_exact", "uniforms"]


@dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    n_cap: int
    lens: np.ndarray          # int32 [B] valid keys per sequence
    ks: np.ndarray            # int32 [B] top-k per sequence
    L: int
    P: int
    tau: float
    dtype: str                # "f32" or "bf16" (storage dtype of K, V, q, W)
    W: np.ndarray             # [L*P, d]
    K: np.ndarray             # [B, Hkv, n_cap, d]
    V: np.ndarray             # [B, Hkv, n_cap, d]
    q: np.ndarray             # [B, Hq, d]
    # decode-loop stream (only for the append workload)
    steps: int = 0
    K_new: np.ndarray | None = None   # [steps, B, Hkv, d]
    V_new: np.ndarray | None = None   # [steps, B, Hkv, d]
    q_steps: np.ndarray | None = None  # [steps, B, Hq, d]
    meta: dict = field(default_factory=dict)

    @property
    def k_max(self) -> int:
        return int(self.ks.max())

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


def to_bf16_exact(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE) and return them as float32."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


# name -> (B, Hq, Hkv, n, L, P, tau, k or k-fraction, dtype, anisotropic)
CONFIGS = {
    "c1": dict(B=1, Hq=1, Hkv=1, n=4096, L=32, P=8, tau=0.5, k=128, dtype="f32", aniso=False),
    "c2": dict(B=1, Hq=32, Hkv=8, n=32768, L=64, P=8, tau=0.5, k=656, dtype="bf16", aniso=True),
    "c3": dict(B=1, Hq=32, Hkv=8, n=131072, L=64, P=8, tau=0.5, k=1024, dtype="bf16", aniso=True),
    "c4": dict(B=16, Hq=32, Hkv=8, n=(8192, 32768), L=64, P=8, tau=0.5, k=0.02, dtype="bf16",
               aniso=True),
    "c5": dict(B=1, Hq=32, Hkv=8, n=131072, L=64, P=8, tau=0.5, k=1024, dtype="bf16", aniso=True,
               steps=256),
}
_CFG_INDEX = {"c1": 1, "c2": 2, "c3": 3, "c4": 4, "c5": 5}


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return to_bf16_exact(x) if dtype == "bf16" else x


def make_workload(name: str = "c2", *, seed: int | None = None, n: int | None = None,
                  B: int | None = None, Hq: int | None = None, Hkv: int | None = None,
                  L: int | None = None, P: int | None = None, tau: float | None = None,
                  k: int | float | None = None, d: int = 128, steps: int | None = None,
                  dtype: str | None = None, lens: list[int] | None = None,
                  n_cap: int | None = None) -> Workload:
    """Draw one workload.  Overrides shrink a config for fast parity cases.

    Stream order from ``SeedSequence(1000 + config index + seed)``:
    W, K, key means, V, value scales, q, lengths, decode-append stream.
    """
    base = dict(CONFIGS[name])
    if B is not None:
        base["B"] = B
    if Hq is not None:
        base["Hq"] = Hq
    if Hkv is not None:
        base["Hkv"] = Hkv
    if L is not None:
        base["L"] = L
    if P is not None:
        base["P"] = P
    if tau is not None:
        base["tau"] = tau
    if k is not None:
        base["k"] = k
    if dtype is not None:
        base["dtype"] = dtype
    if steps is not None:
        base["steps"] = steps
    if n is not None:
        base["n"] = n
    Bn, Hq_, Hkv_ = base["B"], base["Hq"], base["Hkv"]
    Ln, Pn = base["L"], base["P"]
    steps_ = int(base.get("steps", 0))
    ss = np.random.SeedSequence(1000 + _CFG_INDEX[name] + (0 if seed is None else 7919 * seed))
    r_w, r_k, r_mu, r_v, r_vs, r_q, r_len, r_app = [np.random.default_rng(s) for s in ss.spawn(8)]

    # lengths
    nspec = base["n"]
    if lens is not None:
        lens_arr = np.asarray(lens, dtype=np.int32)
        assert lens_arr.shape == (Bn,)
    elif isinstance(nspec, tuple):
        lo, hi = nspec
        lens_arr = r_len.integers(lo, hi + 1, size=Bn).astype(np.int32)
    else:
        lens_arr = np.full(Bn, int(nspec), dtype=np.int32)
    cap = int(lens_arr.max()) + steps_ if n_cap is None else int(n_cap)
    assert cap >= int(lens_arr.max()) + steps_

    kspec = base["k"]
    if isinstance(kspec, float):
        ks = np.array([int(math.ceil(kspec * int(x))) for x in lens_arr], dtype=np.int32)
    else:
        ks = np.minimum(np.full(Bn, int(kspec), dtype=np.int32), lens_arr)

    dt = base["dtype"]
    W = _round(r_w.standard_normal((Ln * Pn, d), dtype=np.float32), dt)
    K = r_k.standard_normal((Bn, Hkv_, cap, d), dtype=np.float32)
    if base["aniso"]:
        u = r_mu.standard_normal((Hkv_, d))
        mu = 3.0 * u / np.linalg.norm(u, axis=1, keepdims=True)
        K += mu[None, :, None, :].astype(np.float32)
    else:
        mu = None
    K = _round(K, dt)
    V = r_v.standard_normal((Bn, Hkv_, cap, d), dtype=np.float32)
    if base["aniso"]:
        g = r_vs.standard_normal((Bn, Hkv_, cap, 1), dtype=np.float32)
        V *= np.exp(0.5 * g).astype(np.float32)
    V = _round(V, dt)
    q = _round(r_q.standard_normal((Bn, Hq_, d), dtype=np.float32), dt)

    K_new = V_new = q_steps = None
    if steps_:
        # the appended rows live at positions lens .. lens+steps-1 of K/V;
        # they are drawn from the same distributions as the prefill rows
        K_new = np.stack([K[b, :, lens_arr[b]:lens_arr[b] + steps_, :] for b in range(Bn)], axis=0)
        K_new = np.ascontiguousarray(K_new.transpose(2, 0, 1, 3))
        V_new = np.stack([V[b, :, lens_arr[b]:lens_arr[b] + steps_, :] for b in range(Bn)], axis=0)
        V_new = np.ascontiguousarray(V_new.transpose(2, 0, 1, 3))
        q_steps = _round(r_app.standard_normal((steps_, Bn, Hq_, d), dtype=np.float32), dt)
    return Workload(name=name, B=Bn, Hq=Hq_, Hkv=Hkv_, d=d, n_cap=cap, lens=lens_arr, ks=ks,
                    L=Ln, P=Pn, tau=float(base["tau"]), dtype=dt, W=W, K=K, V=V, q=q,
                    steps=steps_, K_new=K_new, V_new=V_new, q_steps=q_steps,
                    meta={"mu": mu})


def uniforms(B: int, Hq: int, M: int, seed: int = 0) -> np.ndarray:
    """Seeded float32 uniforms in [0, 1), [B, Hq, M]: the random draws of the
    sampling estimator, passed to both the oracle and the HIP path."""
    rng = np.random.default_rng(np.random.SeedSequence(4242 + seed))
    u = rng.random((B, Hq, M)).astype(np.float32)
    return np.minimum(u, np.nextafter(np.float32(1.0), np.float32(0.0)))
