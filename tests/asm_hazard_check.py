"""Scan AMDGPU assembly for the VALU-writes-SGPR -> VMEM-reads-SGPR hazard at
LDS-DMA instructions.

On gfx9-family GPUs a vector memory instruction that reads an SGPR written
by a VALU instruction (v_readlane, v_readfirstlane, v_cmp into an SGPR pair,
a carry-out of v_add_co, ...) needs 5 wait states in between.  The compiler
inserts them for its own instructions but not for inline assembly, which is
how the library issues its global->LDS DMAs; with fewer, the DMA may use a
stale buffer descriptor, scalar offset or M0 (the LDS address of the DMA).

Every path into the DMA is followed backwards: the fall-through predecessor
and every branch that targets a label on the way, until 5 wait states have
passed on that path.
"""
import re
from typing import Dict, List, Set, Tuple

WAIT_STATES = 5


def _sregs(tok: str) -> Set[str]:
    tok = tok.strip().rstrip(",")
    m = re.match(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return {f"s{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    m = re.match(r"s(\d+)$", tok)
    if m:
        return {tok}
    if tok in ("m0", "vcc", "vcc_lo", "vcc_hi", "exec", "exec_lo", "exec_hi"):
        return {tok}
    return set()


def _wait_states(inst: str) -> int:
    parts = inst.split()
    if parts[0] == "s_nop":
        return int(parts[1], 0) + 1
    return 1


def _valu_sgpr_dests(inst: str) -> Set[str]:
    """SGPRs (and M0 / VCC) a VALU instruction writes."""
    parts = inst.split(None, 1)
    op = parts[0]
    if not op.startswith("v_") or len(parts) < 2:
        return set()
    ops = [o.strip() for o in parts[1].split(",")]
    dests = set(_sregs(ops[0]))
    # VOP3 forms with a scalar carry-out / condition destination second
    if len(ops) > 1 and ("_co_" in op or op.startswith(("v_div_scale", "v_mad_u64_u32", "v_mad_i64_i32"))):
        dests |= _sregs(ops[1])
    if op.startswith("v_cmp") and op.endswith("_e32"):
        dests.add("vcc")
    return dests


def _body(text: str, start: int) -> List[str]:
    end = text.find(".Lfunc_end", start)
    out = []
    for raw in text[start:end].split("\n"):
        l = raw.strip()
        if not l or l.startswith(";"):
            continue
        if re.match(r"^\.L[\w$]+:", l):
            out.append("LABEL " + l.split(":")[0])
            continue
        if l.startswith("."):
            continue
        out.append(l.split(";")[0].strip())
    return out


def check_file(path: str) -> List[Tuple[str, int, str]]:
    """Return (function, line index, instruction) for every LDS DMA whose
    descriptor, scalar offset or M0 was written by a VALU instruction fewer
    than 5 wait states before it on some path into it."""
    text = open(path).read()
    bad = []
    for m in re.finditer(r"^(_Z[^:\s]+):", text, re.M):
        name = m.group(1)
        body = _body(text, m.end())
        labels: Dict[str, int] = {}
        sources: Dict[str, List[int]] = {}
        for i, inst in enumerate(body):
            if inst.startswith("LABEL "):
                labels[inst[6:]] = i
            elif inst.startswith(("s_branch", "s_cbranch")):
                tgt = inst.split()[-1]
                sources.setdefault(tgt, []).append(i)
        for k, inst in enumerate(body):
            if not (inst.startswith("buffer_load") and inst.endswith(" lds")):
                continue
            ops = [o.strip() for o in inst.split(",")]
            regs = _sregs(ops[1]) | _sregs(ops[2].split()[0]) | {"m0"}
            if _flagged(body, sources, k, regs):
                bad.append((name, k, inst))
    return bad


def _flagged(body: List[str], sources: Dict[str, List[int]], k: int, regs: Set[str]) -> bool:
    stack = [(k - 1, 0)]
    seen = set()
    while stack:
        i, waited = stack.pop()
        while i >= 0 and waited < WAIT_STATES:
            if (i, waited) in seen:
                break
            seen.add((i, waited))
            prev = body[i]
            if prev.startswith("LABEL "):
                for b in sources.get(prev[6:], []):
                    stack.append((b, waited))
                # the fall-through into the label, unless an unconditional
                # branch ends the block before it
                if i > 0 and body[i - 1].startswith("s_branch"):
                    break
                i -= 1
                continue
            if _valu_sgpr_dests(prev) & regs:
                return True
            waited += _wait_states(prev)
            i -= 1
    return False
