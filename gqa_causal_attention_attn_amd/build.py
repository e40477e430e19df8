"""Build libgqa_attn.so in-tree with hipcc for gfx950.

Usage: python -m gqa_causal_attention_attn_amd.build  (or call build()).
Every call compiles from source; nothing is cached.
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgqa_attn.so")
SOURCES = ["attn_fwd.hip", "attn_aux.hip", "attn_composed.hip", "attn_small_d.hip", "attn_api.cpp"]
ARCH = "gfx950"

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


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source and link the shared library; returns its path."""
    objs = []
    tmp_dir = os.path.join(PKG, "_build")
    os.makedirs(tmp_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(tmp_dir, src + ".o")
        cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp_lib = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
