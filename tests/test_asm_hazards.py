"""Wait states in front of the kernels' LDS DMAs (CPU-only: compiles the kernel
source to gfx950 assembly and reads it with exact_attention_57_amd/hazards.py).

The tile DMAs are inline assembly, which the compiler's hazard checks do not
look into: a VMEM instruction may read an SGPR only five wait states after a
VALU instruction wrote it, and an LDS DMA needs one after M0 is written.  A
build that reloaded a spilled buffer resource with v_readlane right before a
DMA, one wait state ahead of it, faulted the GPU.  build() keeps one wait
state only for assembly this check passes; these tests cover the checker and
the always-safe setting.
"""
import importlib.util
import os
import shutil

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "exact_attention_57_amd")


def _load(name, path):
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


hz = _load("_attn_hazards_t", os.path.join(PKG, "hazards.py"))


def _have_hipcc():
    return any(c and os.path.exists(c) for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"))


def test_checker_flags_short_gaps():
    bad = ["v_readlane_b32 s2, v249, 36", "s_mov_b32 m0, s9", "s_nop 0",
           "buffer_load_dwordx4 v1, s[0:3], s5 offen lds"]
    assert hz.check_function("synthetic", bad)
    soff = ["v_readfirstlane_b32 s5, v3", "s_mov_b32 m0, s9", "s_nop 1",
            "buffer_load_dwordx4 v1, s[0:3], s5 offen lds"]
    assert hz.check_function("synthetic", soff)
    m0 = ["s_mov_b32 m0, s9", "buffer_load_dword v1, s[0:3], 0 offen lds"]
    assert hz.check_function("synthetic", m0)
    ok = ["v_readlane_b32 s2, v249, 36", "s_mov_b32 m0, s9", "s_nop 4",
          "buffer_load_dwordx4 v1, s[0:3], s5 offen lds"]
    assert not hz.check_function("synthetic", ok)
    unrelated = ["v_readlane_b32 s20, v249, 36", "s_mov_b32 m0, s9", "s_nop 0",
                 "buffer_load_dwordx4 v1, s[0:3], s5 offen lds"]
    assert not hz.check_function("synthetic", unrelated)


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc not available")
def test_safe_setting_has_no_hazards():
    build = _load("_attn_build_t", os.path.join(PKG, "build.py"))
    n, problems = hz.scan(build.kernel_asm(4))
    # 24 dense + 6 block-sparse bf16 forward, 6 FP8 forward, 4 backward dQ instances
    assert n >= 40, f"expected every DMA kernel instance, found {n}"
    assert not problems, "\n".join(problems[:20])


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc not available")
def test_build_choice_is_hazard_free():
    build = _load("_attn_build_t2", os.path.join(PKG, "build.py"))
    nop = build.choose_dma_nop()
    assert nop in (0, 4)
    n, problems = hz.scan(build.kernel_asm(nop))
    assert n >= 40 and not problems
