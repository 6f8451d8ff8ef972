"""Wait-state check for the kernels' LDS DMAs, on compiler-generated gfx950
assembly (a build-time tool; no GPU needed).

The tile DMAs are inline assembly, which the compiler's hazard checks do not
look into.  On gfx9 a VMEM instruction may read an SGPR only five wait states
after a VALU instruction wrote it, and an LDS DMA needs one wait state after
M0 is written.  The compiler does write such SGPRs right before a DMA when it
reloads spilled SGPRs with v_readlane; a DMA that reads a stale buffer
resource then addresses arbitrary memory.  ``scan`` counts the wait states
(one per instruction, N+1 per s_nop N) between each LDS DMA and the last
writes of every SGPR it reads and of M0.
"""
from __future__ import annotations

import re

VMEM_AFTER_VALU_SGPR = 5
LDS_DMA_AFTER_M0 = 1


def instructions(fn_text: str) -> list:
    out = []
    for raw in fn_text.splitlines():
        line = raw.split(";")[0].strip()
        if not line or line.endswith(":") or line.startswith("."):
            continue
        out.append(line)
    return out


def sgprs(operand_text: str) -> set:
    regs = set()
    for m in re.finditer(r"\bs\[(\d+):(\d+)\]", operand_text):
        regs |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"(?<![\w\[:])s(\d+)\b", operand_text):
        regs.add(int(m.group(1)))
    return regs


def wait_states(instrs) -> int:
    n = 0
    for ins in instrs:
        m = re.match(r"s_nop\s+(\d+)", ins)
        n += int(m.group(1)) + 1 if m else 1
    return n


def is_lds_dma(ins: str) -> bool:
    return ins.startswith("buffer_load") and ins.endswith(" lds")


def check_function(name: str, instrs: list) -> list:
    problems = []
    for i, ins in enumerate(instrs):
        if not is_lds_dma(ins):
            continue
        read = sgprs(ins.split(None, 1)[1])
        m0_seen = False
        for k in range(i - 1, -1, -1):
            gap = wait_states(instrs[k + 1:i])
            if gap >= VMEM_AFTER_VALU_SGPR:
                break              # nothing earlier can be too close
            prev = instrs[k]
            mnem, _, ops = prev.partition(" ")
            dst = ops.split(",")[0].strip()
            if mnem.startswith("v_") and dst.startswith("s") and sgprs(dst) & read:
                problems.append(f"{name}: {prev!r} -> {ins!r}: {gap} wait states")
            if not m0_seen and dst == "m0":
                m0_seen = True
                if gap < LDS_DMA_AFTER_M0:
                    problems.append(f"{name}: {prev!r} -> {ins!r}: M0 written {gap} wait states before")
    return problems


def scan(asm_text: str, kernel_substr: str = ""):
    """Return (number of kernel functions with LDS DMAs, list of violations).

    Every function whose name contains ``kernel_substr`` (default: every
    function) and that issues an LDS DMA is checked."""
    n, problems = 0, []
    for fn in re.split(r"\n(?=_Z\w+:)", asm_text):
        head = fn.split(":", 1)[0]
        if kernel_substr not in head:
            continue
        instrs = instructions(fn.split("s_endpgm", 1)[0])
        if not any(is_lds_dma(i) for i in instrs):
            continue
        n += 1
        problems += check_function(head, instrs)
    return n, problems
