"""Build libattn.so (the HIP kernels + C ABI) in-tree for gfx950.

    python exact_attention_57_amd/build.py      (or __graft_entry__.build())

The library is compiled ahead of time with hipcc for ``--offload-arch=gfx950``
only.  Packed-fp32 VALU instructions are disabled for all HIP code
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass warns
that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libattn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["attn_fwd_kernel.hip", "attn_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libattn.so)")


def compile_flags(extra=()) -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, *extra,
    ]


def build(verbose: bool = False, extra=()) -> str:
    """Compile every HIP/C++ source into ``exact_attention_57_amd/libattn.so``.

    Always recompiles (it is the "does it build" check).  Objects go to a
    private build folder; the library is written atomically.
    """
    cc = hipcc()
    bdir = os.path.join(PKG_DIR, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *compile_flags(extra), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
