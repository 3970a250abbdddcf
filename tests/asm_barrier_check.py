"""Static check of compiled gfx950 assembly: no s_barrier may sit inside a loop
whose exit the compiler implemented with an exec mask (a divergent loop).

Such a loop lets some lanes of a wave leave while the others keep meeting the
loop's barriers, which deadlocks the workgroup.  LLVM annotates every block of
the assembly with its loop ("Loop Header", "Parent Loop", "Header=BB..."), so
the loop nest can be rebuilt from the text.
"""
import re, sys

def analyze(lines):
    out = []
    func = None
    def finish(func, blocks, loopof, parent):
        members = {}
        for b, h in loopof.items():
            members.setdefault(h, set()).add(b)
        def all_blocks(h, seen=()):
            s = set(members.get(h, set())) | {h}
            for c, p in parent.items():
                if p == h and c not in seen:
                    s |= all_blocks(c, seen + (c,))
            return s
        res = []
        for h in set(loopof.values()):
            bl = all_blocks(h)
            own = members.get(h, set()) | {h}
            div = any("s_andn2_b64 exec, exec" in "\n".join(blocks.get(b, [])) for b in own)
            bar = any("s_barrier" in "\n".join(blocks.get(b, [])) for b in bl)
            if div and bar:
                res.append(h)
        return res
    blocks = {}; loopof = {}; parent = {}; cur = None
    for line in lines + ["_Zend:"]:
        m = re.match(r"^(_Z\w+):", line)
        if m:
            if func:
                r = finish(func, blocks, loopof, parent)
                out.append((func, r))
            func = m.group(1); blocks = {}; loopof = {}; parent = {}; cur = "entry"; continue
        m = re.match(r"^(\.LBB\d+_\d+|; %bb\.\d+):(.*)", line)
        if m:
            cur = m.group(1).replace("; %bb.", "bb").replace(".LBB", "BB")
            rest = m.group(2)
            mm = re.search(r"Header=(BB\d+_\d+)", rest)
            if mm: loopof[cur] = mm.group(1)
            mm = re.search(r"Parent Loop (BB\d+_\d+)", rest)
            if mm: parent[cur] = mm.group(1)
            continue
        if cur and re.search(r"=>\s*This (Inner )?Loop Header", line):
            loopof[cur] = cur
        if cur: blocks.setdefault(cur, []).append(line)
    return out


def check_file(path):
    """Return [(function, [loop headers])] of offending loops in one .s file."""
    return [(f, r) for f, r in analyze(open(path).read().split("\n")) if r]


if __name__ == "__main__":
    bad = False
    for path in sys.argv[1:]:
        for func, res in check_file(path):
            bad = True
            print(f"{path}: {func}: divergent loop(s) with barriers: {res}")
    print("FAIL" if bad else "OK: no barrier inside a divergent loop")
    sys.exit(1 if bad else 0)
