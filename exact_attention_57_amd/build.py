"""Build libattn.so (the HIP kernels + C ABI) in-tree for gfx950.

    python exact_attention_57_amd/build.py      (or __graft_entry__.build())

The library is compiled ahead of time with hipcc for ``--offload-arch=gfx950``
only.  Packed-fp32 VALU instructions are disabled for all HIP code
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass warns
that it does not know the feature, which is harmless.

The kernels' LDS DMAs are inline assembly preceded by ``s_nop ATTN_DMA_NOP``.
The build first compiles the kernels to assembly with one wait state
(``ATTN_DMA_NOP=0``) and scans it (``hazards.py``); it keeps that setting only
if no LDS DMA reads an SGPR a VALU instruction wrote fewer than five wait
states earlier, and otherwise builds with five (``ATTN_DMA_NOP=4``).

Two checking builds of the same sources are written next to the library,
both with the always-safe five wait states:

  libattn_racecheck.so  ATTN_RACE_CHECK=1: every barrier drains all memory
                        traffic and is passed twice (outputs must equal the
                        default build's bit for bit)
  libattn_stamps.so     ATTN_STAMPS=1: the forward kernels write per-workgroup
                        timing records after the statistics counters

Object files are compiled in parallel.
"""
from __future__ import annotations

import importlib.util
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libattn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["attn_fwd_kernel.hip", "attn_fwd_fp8_kernel.hip", "attn_bwd_kernel.hip", "attn_scratch.hip", "attn_api.cpp"]
DMA_SOURCES = ["attn_fwd_kernel.hip", "attn_fwd_fp8_kernel.hip", "attn_bwd_kernel.hip"]   # kernels with LDS DMAs
ARCH = "gfx950"
VARIANTS = {                       # checking builds: name -> extra defines
    "racecheck": ["-DATTN_RACE_CHECK=1"],
    "stamps": ["-DATTN_STAMPS=1"],
}


def variant_path(name: str) -> str:
    return os.path.join(PKG_DIR, f"libattn_{name}.so")


def _jobs() -> int:
    return max(1, min(8, os.cpu_count() or 1))


def _run_all(cmds, verbose=False):
    """Run compiler commands in parallel; raise on the first failure."""
    def one(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stderr[-4000:]}")
        return r
    with ThreadPoolExecutor(_jobs()) as ex:
        list(ex.map(one, cmds))


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


def _hazards():
    spec = importlib.util.spec_from_file_location("_attn_hazards", os.path.join(PKG_DIR, "hazards.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def kernel_asm(dma_nop: int, extra=(), cc: str = None) -> str:
    """gfx950 assembly of the kernel sources with LDS DMAs, as build() compiles them."""
    cc = cc or hipcc()
    bdir = os.path.join(PKG_DIR, "_build")
    os.makedirs(bdir, exist_ok=True)
    outs, cmds = [], []
    for src in DMA_SOURCES:
        out = os.path.join(bdir, f"{os.path.splitext(src)[0]}_nop{dma_nop}.s")
        cmds.append([cc, *compile_flags(extra), f"-DATTN_DMA_NOP={dma_nop}", "-x", "hip", "--cuda-device-only",
                     "-S", os.path.join(CSRC, src), "-o", out])
        outs.append(out)
    _run_all(cmds)
    text = []
    for out in outs:
        with open(out) as f:
            text.append(f.read())
    return "\n".join(text)


def choose_dma_nop(extra=(), cc: str = None, verbose: bool = False) -> int:
    """Smallest s_nop operand (0 or 4) whose compiled kernels have no LDS DMA
    wait-state hazard; raises if even 4 leaves one."""
    hz = _hazards()
    problems = []
    for nop in (0, 4):
        n, problems = hz.scan(kernel_asm(nop, extra, cc))
        if n == 0:
            raise RuntimeError("no kernel with LDS DMAs found in the assembly")
        if verbose:
            print(f"ATTN_DMA_NOP={nop}: {n} kernels, {len(problems)} wait-state hazards", flush=True)
        if not problems:
            return nop
    raise RuntimeError("LDS DMA wait-state hazard with s_nop 4: " + problems[0])


def build(verbose: bool = False, extra=()) -> str:
    """Compile every HIP/C++ source into ``exact_attention_57_amd/libattn.so``
    and the checking builds ``libattn_<variant>.so``.

    Always recompiles (it is the "does it build" check).  Objects go to a
    private build folder; each library is written atomically.
    """
    cc = hipcc()
    nop = choose_dma_nop(extra, cc, verbose)
    libs = [(LIB_PATH, "main", [f"-DATTN_DMA_NOP={nop}"])]
    libs += [(variant_path(name), name, ["-DATTN_DMA_NOP=4", *defs]) for name, defs in VARIANTS.items()]
    cmds, objs = [], {}
    for path, tag, defs in libs:
        bdir = os.path.join(PKG_DIR, "_build", tag)
        os.makedirs(bdir, exist_ok=True)
        objs[path] = []
        for src in SOURCES:
            obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
            lang = ["-x", "hip", *defs] if src.endswith(".hip") else []
            cmds.append([cc, *compile_flags(extra), *lang, "-c", os.path.join(CSRC, src), "-o", obj])
            objs[path].append(obj)
    _run_all(cmds, verbose)
    links = []
    for path, _, _ in libs:
        links.append([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", path + ".tmp", *objs[path]])
    _run_all(links, verbose)
    for path, _, _ in libs:
        os.replace(path + ".tmp", path)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
