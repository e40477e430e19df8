"""Build libgqa_attn.so in-tree with hipcc for gfx950.

Usage: python -m gqa_causal_attention_attn_amd.build  (or call build()).
Every call compiles from source; nothing is cached.

Besides the library, build() compiles the achievable-peak probes of the benchmark
(libgqa_probes.so, include/gqa_probes.h) and the planted-mistake libraries
(libgqa_attn_control{1,2,3}.so, the sources with -DGQA_CONTROL=n: a row that sees one key
past its own, a merge that drops its last chunk, an append one row late).  Only the tests that
must see them miss the oracle load them.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgqa_attn.so")
SOURCES = ["attn_fwd_d256.hip", "attn_fwd_d128.hip", "attn_fwd_d64.hip", "attn_aux.hip", "attn_composed.hip",
           "attn_noalloc.hip", "attn_api.cpp"]
ARCH = "gfx950"
CONTROLS = (1, 2, 3)

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def control_lib(n: int) -> str:
    return os.path.join(PKG, f"libgqa_attn_control{n}.so")


def _jobs(verbose, extra):
    """(library path, [(compile command, object)]) for the library and each control build."""
    out = []
    for n in (0,) + CONTROLS:
        tmp_dir = os.path.join(PKG, "_build" if n == 0 else f"_build_control{n}")
        os.makedirs(tmp_dir, exist_ok=True)
        defs = [] if n == 0 else [f"-DGQA_CONTROL={n}"]
        cmds = []
        for src in SOURCES:
            obj = os.path.join(tmp_dir, src + ".o")
            cmds.append(([hipcc(), *FLAGS, *defs, *extra, "-c", os.path.join(CSRC, src), "-o", obj], obj))
        out.append((LIB if n == 0 else control_lib(n), cmds))
    return out


PROBES_LIB = os.path.join(PKG, "libgqa_probes.so")


def build(verbose: bool = False, extra=(), controls: bool = True) -> str:
    """Compile every source and link the shared libraries; returns the library's path."""
    jobs = _jobs(verbose, extra)
    if not controls:
        jobs = jobs[:1]
    # the achievable-peak probes of the benchmark (libgqa_probes.so)
    pdir = os.path.join(PKG, "_build_probes")
    os.makedirs(pdir, exist_ok=True)
    pobj = os.path.join(pdir, "probes.hip.o")
    jobs.append((PROBES_LIB, [([hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, "probes.hip"), "-o", pobj], pobj)]))
    compiles = [c for _, cmds in jobs for c in cmds]
    # the main passes of the library are by far the longest compiles: start them first
    compiles.sort(key=lambda c: ("attn_fwd_d" not in c[1], "_control" in c[1]))

    def run(cmd):
        if verbose:
            print(" ".join(cmd[0]), flush=True)
        subprocess.run(cmd[0], check=True)

    workers = max(1, min(6, (os.cpu_count() or 2) - 1))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(run, compiles))
    for lib, cmds in jobs:
        tmp_lib = lib + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for _, o in cmds], "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
