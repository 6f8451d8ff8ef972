"""Wait states in front of the kernels' LDS DMAs (CPU-only: compiles the kernel
source to gfx950 assembly and reads it).

The tile DMAs are inline assembly, which the compiler's hazard checks do not
look into.  On gfx9 a VMEM instruction may read an SGPR only five wait states
after a VALU instruction wrote it, and an LDS DMA needs one wait state after
M0 is written.  The compiler does write such SGPRs right before a DMA when it
reloads spilled SGPRs with v_readlane; a DMA that reads a stale buffer
resource then addresses arbitrary memory.  This test counts the wait states
(one per instruction, N+1 per s_nop N) between each LDS DMA and the last
write of every SGPR it reads, in every kernel instance.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "exact_attention_57_amd", "csrc", "attn_fwd_kernel.hip")
VMEM_AFTER_VALU_SGPR = 5
LDS_DMA_AFTER_M0 = 1


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "k.s"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", os.path.dirname(SRC),
           "-x", "hip", "-c", SRC, "--cuda-device-only", "-S", "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    return out.read_text()


def _instructions(fn_text):
    out = []
    for raw in fn_text.splitlines():
        line = raw.split(";")[0].strip()
        if not line or line.endswith(":") or line.startswith("."):
            continue
        out.append(line)
    return out


def _sgprs(operand_text):
    regs = set()
    for m in re.finditer(r"\bs\[(\d+):(\d+)\]", operand_text):
        regs |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"(?<![\w\[:])s(\d+)\b", operand_text):
        regs.add(int(m.group(1)))
    return regs


def _wait_states(instrs):
    """Wait states contributed by a run of instructions."""
    n = 0
    for ins in instrs:
        m = re.match(r"s_nop\s+(\d+)", ins)
        n += int(m.group(1)) + 1 if m else 1
    return n


def _check_function(name, instrs):
    problems = []
    for i, ins in enumerate(instrs):
        if not (ins.startswith("buffer_load") and ins.endswith(" lds")):
            continue
        read = _sgprs(ins.split(None, 1)[1])
        m0_seen = False
        for k in range(i - 1, -1, -1):
            between = instrs[k + 1:i]
            gap = _wait_states(between)
            if gap >= VMEM_AFTER_VALU_SGPR:
                break              # nothing earlier can be too close
            prev = instrs[k]
            mnem, _, ops = prev.partition(" ")
            dst = ops.split(",")[0].strip()
            if mnem.startswith("v_") and dst.startswith("s") and _sgprs(dst) & read:
                problems.append(f"{name}: {prev!r} -> {ins!r}: {gap} wait states")
            if not m0_seen and dst == "m0":
                m0_seen = True
                if gap < LDS_DMA_AFTER_M0:
                    problems.append(f"{name}: {prev!r} -> {ins!r}: M0 written {gap} wait states before")
    return problems


def test_lds_dma_wait_states(kernel_asm):
    functions = re.split(r"\n(?=_Z\w+:)", kernel_asm)
    checked = 0
    problems = []
    for fn in functions:
        head = fn.split(":", 1)[0]
        if "attn_fwd_kernel" not in head:
            continue
        body = fn.split("s_endpgm", 1)[0]
        instrs = _instructions(body)
        if not any(i.startswith("buffer_load") and i.endswith(" lds") for i in instrs):
            continue
        checked += 1
        problems += _check_function(head, instrs)
    assert checked >= 24, f"expected every kernel instance to contain LDS DMAs, found {checked}"
    assert not problems, "\n".join(problems[:20])


def test_checker_flags_a_short_gap():
    """The checker itself: a v_readlane two instructions before a DMA fails."""
    instrs = ["v_readlane_b32 s2, v249, 36", "s_mov_b32 m0, s9", "s_nop 0",
              "buffer_load_dwordx4 v1, s[0:3], s5 offen lds"]
    assert _check_function("synthetic", instrs)
    ok = ["v_readlane_b32 s2, v249, 36", "s_mov_b32 m0, s9", "s_nop 4",
          "buffer_load_dwordx4 v1, s[0:3], s5 offen lds"]
    assert not _check_function("synthetic", ok)
