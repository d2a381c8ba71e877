"""socket_decode_step_noalloc (the library's static scratch array, no
allocation) against socket_decode_step with a caller-owned workspace, through
the C ABI.  Two calls in a row share the one scratch array, the second on a
smaller input (fewer sequences, heads and keys), so stale contents of the
first call would show up in the second; every output must equal the
workspace call's bit for bit (same kernels, same inputs)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_cases as GC
from gpu_cases import DEV
import soft_lsh_token_amd as S
from soft_lsh_token_amd.inputs import make_workload

pytestmark = pytest.mark.gpu

# (workload, (sink, window)); the second is smaller in every dimension
CALLS = [
    (dict(name="c2", n=20000), (64, 128)),
    (dict(name="c4", n=(2000, 6000), B=2, Hq=8, Hkv=2, k=0.02), (0, 0)),
]


def _one(case, sw):
    print("noalloc case", case, sw, flush=True)
    sink, window = sw
    w = make_workload(**case)
    d = GC.upload(w)
    # keys [0, lens-1) are cached; key lens-1 is the one the step appends
    ids0, vn0 = GC.gpu_hash(w, d, count=int(w.lens.max()) - 1)
    k_max = w.k_max + sink + window
    outs = []
    for noalloc in (False, True):
        ids, vn = ids0.clone(), vn0.clone()
        idx = torch.full((w.B, w.Hq, k_max), -7, dtype=torch.int32, device=DEV)
        sc = torch.zeros(w.B, w.Hq, S.score_stride(w.n_cap), dtype=torch.float32, device=DEV)
        out = torch.full((w.B, w.Hq, w.d), float("nan"), dtype=torch.float32, device=DEV)
        fn = S.socket_decode_step_noalloc if noalloc else S.socket_decode_step
        fn(d["q"], d["K"], d["V"], d["W"], ids, vn, d["lens"], d["ks"], k_max, w.tau, w.L, w.P,
           w.scale, idx, out, scores=sc, sink=sink, window=window)
        outs.append((ids, vn, idx, sc, out))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    # and the selection itself is the exact one on the GPU's own scores
    idx, sc = outs[1][2].cpu().numpy(), outs[1][3].cpu().numpy()
    for b in range(w.B):
        n = int(w.lens[b])
        for g in range(w.Hq):
            GC.check_exact_select(idx[b, g], sc[b, g], int(w.ks[b]), n, sink, window)


def test_noalloc_matches_workspace_call_twice():
    for case, sw in CALLS:
        _one(case, sw)


def test_noalloc_rejects_oversized_steps():
    """Sizes whose workspace exceeds the static scratch are refused before
    anything is enqueued (the 16-sequence 32K batch needs about 217 MiB)."""
    need = S.socket_decode_step_workspace(16, 32, 8, 32769, 64, 8, 656)
    assert need > S.NOALLOC_SCRATCH_BYTES
    fake = 0x10000
    rc = S.lib().socket_decode_step_noalloc(fake, fake, fake, 1, 16, 32, 8, 128, fake, 64, 8, 0.5,
                                            fake, fake, fake, 32769, fake, 656, 0, 0, 0.088,
                                            fake, None, fake, None)
    assert rc == -3  # SOCKET_ENOSPC
