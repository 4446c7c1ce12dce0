"""Build libmoe.so (HIP, gfx950) in-tree: mixture_experts_layer_32_amd/libmoe.so.

    python -m mixture_experts_layer_32_amd.build [-v]

Every .hip file under csrc/ is compiled to an object in parallel (hipcc cross-compiles without
a GPU), then linked into one shared library. The object files go under _build/.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Wno-unused-command-line-argument",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(os.path.dirname(PKG), "include"),
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found (ROCm is required to build libmoe.so)")
    return p


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=1200)
    except subprocess.TimeoutExpired:
        raise RuntimeError(f"command timed out after 1200 s: {' '.join(cmd)}")
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cc = hipcc()
    objs = []
    cmds = []
    for s in srcs:
        o = os.path.join(BUILD, s[:-4] + ".o")
        objs.append(o)
        cmds.append([cc, *CFLAGS, "-c", os.path.join(CSRC, s), "-o", o])
    with cf.ThreadPoolExecutor(max(1, min(jobs, len(cmds)))) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
