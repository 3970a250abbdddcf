"""Scan compiled gfx950 assembly for spill traffic inside the MFMA loops.

A kernel's K loop is its innermost loop that issues MFMA instructions.  A
scratch access in its hot blocks (a spilled vector register) costs a memory
round trip per iteration, and the compiler's wait for it also waits for
every DMA in flight; a v_readlane / v_writelane there moves a spilled scalar
register (and a descriptor restored that way right before an inline-asm DMA
is the hazard asm_hazard_check looks for).  Loops are found from the
assembly's backward branches; the hot blocks are the loop's basic blocks
that issue MFMAs or 16-byte LDS DMAs (the operand refills).  The error paths
of its bounded waits and the once-per-slab flag fetch (a 4-byte DMA) are
cold.
"""
import re
from typing import Dict, List, Tuple

SPILL_OPS = ("scratch_", "buffer_store_dword", "v_readlane_b32", "v_writelane_b32")


def _functions(text: str):
    for m in re.finditer(r"^(_Z[^:\s]+):", text, re.M):
        end = text.find(".Lfunc_end", m.end())
        lines = [l.strip().split(";")[0].strip() for l in text[m.end():end].split("\n")]
        yield m.group(1), [l for l in lines if l and (not l.startswith(".") or re.match(r"^\.L\w+:$", l))]


def mfma_loops(path: str) -> List[Tuple[str, int, List[str]]]:
    """(function, loop length, spill instructions) of every innermost loop
    that issues MFMAs."""
    out = []
    for name, lines in _functions(open(path).read()):
        labels: Dict[str, int] = {l[:-1]: i for i, l in enumerate(lines) if re.match(r"^\.L\w+:$", l)}
        loops = []
        for i, l in enumerate(lines):
            if l.startswith(("s_cbranch", "s_branch")):
                tgt = l.split()[-1]
                if tgt in labels and labels[tgt] < i:
                    loops.append((labels[tgt], i))
        for a, b in loops:
            body = lines[a:b + 1]
            if not any(x.startswith("v_mfma") for x in body):
                continue
            # innermost: no other MFMA loop nested inside
            if any(a < a2 and b2 <= b and (a2, b2) != (a, b) and
                   any(x.startswith("v_mfma") for x in lines[a2:b2 + 1]) for a2, b2 in loops):
                continue
            spills = []
            block: List[str] = []
            for x in body + [".Lend:"]:
                if re.match(r"^\.L\w+:$", x) or x.startswith(("s_branch", "s_cbranch")):
                    if not x.startswith(".L"):
                        block.append(x)
                    if any(y.startswith("v_mfma") or (y.startswith("buffer_load_dwordx4") and y.endswith(" lds"))
                           for y in block):
                        spills += [y for y in block if y.startswith(SPILL_OPS) and not y.endswith(" lds")]
                    block = []
                else:
                    block.append(x)
            out.append((name, b - a + 1, spills))
    return out


def spill_counts(path: str) -> Dict[str, Tuple[int, int]]:
    """Kernel name -> (VGPR spills, SGPR spills) from the code object metadata."""
    t = open(path).read()
    names = re.findall(r"\.name:\s+(\S+)", t)
    vs = re.findall(r"\.vgpr_spill_count:\s+(\d+)", t)
    ss = re.findall(r"\.sgpr_spill_count:\s+(\d+)", t)
    return {n: (int(a), int(b)) for n, a, b in zip(names, vs, ss)}
