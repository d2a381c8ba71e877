"""Build the HIP library ``libsocket_lsh.so`` for gfx950 with hipcc.

The library is built in-tree next to this file.  ``python -m
soft_lsh_token_amd.build`` rebuilds it; it always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsocket_lsh.so")
SOURCES = ["api.hip", "hash.hip", "score_topk.hip", "sparse_decode.hip", "dense_decode.hip",
           "hard_lsh.hip", "sample_estimate.hip", "noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libsocket_lsh.so")


FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    # keep the compiler away from packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def command(out: str = LIB, extra: list[str] | None = None) -> list[str]:
    """One hipcc line that compiles and links every source (for reference and
    for tools that want a single command)."""
    return [
        hipcc(), *FLAGS, "-shared", "-I", os.path.join(ROOT, "include"),
        "-o", out,
        *[os.path.join(CSRC, s) for s in SOURCES],
        *(extra or []),
    ]


def _filter(text: str) -> list[str]:
    return [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile each source to an object in parallel, then link the library."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    jobs = jobs or min(len(SOURCES), max(1, os.cpu_count() or 1), 16)
    objs, procs, msgs = [], [], []
    pending = list(SOURCES)
    running = []

    def reap(block: bool):
        for item in list(running):
            src, proc = item
            if block or proc.poll() is not None:
                out, err = proc.communicate()
                running.remove(item)
                msgs.extend(_filter(out + err))
                if proc.returncode != 0:
                    raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(_filter(out + err)))

    while pending or running:
        while pending and len(running) < jobs:
            src = pending.pop(0)
            obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
            objs.append(obj)
            cmd = [cc, *FLAGS, "-I", os.path.join(ROOT, "include"), "-c", "-o", obj,
                   os.path.join(CSRC, src)]
            if verbose:
                print(" ".join(cmd), flush=True)
            running.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                  stderr=subprocess.PIPE, text=True)))
        if running:
            running[0][1].wait()
            reap(False)
    tmp = LIB + ".tmp"
    link = [cc, *FLAGS, "-shared", "-o", tmp, *objs]
    if verbose:
        print(" ".join(link), flush=True)
    res = subprocess.run(link, capture_output=True, text=True)
    msgs.extend(_filter(res.stdout + res.stderr))
    if res.returncode != 0:
        raise RuntimeError("hipcc link failed:\n" + "\n".join(_filter(res.stdout + res.stderr)))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
