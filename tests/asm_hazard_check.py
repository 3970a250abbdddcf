"""Scan AMDGPU assembly for the VALU-writes-SGPR -> VMEM-reads-SGPR hazard at
LDS-DMA instructions.

On gfx9-family GPUs a vector memory instruction that reads an SGPR written
by a VALU instruction (v_readlane, v_cmp into an SGPR pair, ...) needs 5 wait
states in between.  The compiler inserts them for its own instructions but
not for inline assembly, which is how the library issues its global->LDS
DMAs; with fewer, the DMA may use a stale buffer descriptor.
"""
import re
from typing import List, Set, Tuple

WAIT_STATES = 5


def _sregs(tok: str) -> Set[int]:
    m = re.match(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _wait_states(inst: str) -> int:
    parts = inst.split()
    if parts[0] == "s_nop":
        return int(parts[1], 0) + 1
    return 1


def check_file(path: str) -> List[Tuple[str, int, str]]:
    """Return (function, line index, instruction) for every LDS DMA whose
    descriptor or scalar-offset SGPRs were written by a VALU instruction
    fewer than 5 wait states before it, in program layout order."""
    text = open(path).read()
    bad = []
    for m in re.finditer(r"^(_Z[^:\s]+):", text, re.M):
        name = m.group(1)
        end = text.find(".Lfunc_end", m.end())
        lines = [l.strip() for l in text[m.end():end].split("\n")]
        body = [l for l in lines if l and not l.startswith((";", "."))]
        for k, inst in enumerate(body):
            if not (inst.startswith("buffer_load") and inst.endswith(" lds")):
                continue
            ops = [o.strip() for o in inst.split(",")]
            desc = _sregs(ops[1]) | _sregs(ops[2].split()[0])  # descriptor and scalar offset
            waited = 0
            for q in range(k - 1, -1, -1):
                prev = body[q]
                # layout order, through branches and block starts: the
                # fall-through predecessor is checked; extra paths only add
                # conservative matches
                if waited >= WAIT_STATES:
                    break
                op = prev.split()[0]
                if op.startswith("v_") and len(prev.split()) > 1:
                    if _sregs(prev.split()[1].rstrip(",")) & desc:
                        bad.append((name, k, inst))
                        break
                waited += _wait_states(prev)
    return bad
