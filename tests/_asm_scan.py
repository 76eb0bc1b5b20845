"""Scan of gfx950 assembly (hipcc -S output) for workgroup barriers inside
loops that the compiler made divergent.

A loop whose own blocks remove lanes from the exec mask (the structurizer's
`s_andn2_b64 exec, exec, ...` latch) runs once per lane subset: a wave can
go round it with some lanes while its other lanes wait, so an `s_barrier`
inside such a loop is met a different number of times by different waves.
That is a hang or a lost synchronisation even where the source's loop
condition is uniform in fact (the compiler could not prove it).

The assembly's own loop annotations give the structure: a header block says
"Loop Header" (with "Parent Loop" lines for its enclosing loops) and every
other block of a loop says "in Loop: Header=BB...".
"""
import re


def _blocks(text):
    kern, cur, out = None, None, []
    for line in text.split("\n"):
        m = re.match(r"^(_Z\w+):", line)
        if m:
            kern, cur = m.group(1), None
            continue
        m = re.match(r"^(\.LBB\w+|; %bb\.\d+):\s*(.*)", line)
        if m and kern:
            lab = m.group(1)
            name = lab[2:] if lab.startswith(".L") else lab.replace("; %bb.", "bb")
            cur = dict(kern=kern, name=name, ann=m.group(2), lines=[],
                       parents=re.findall(r"Parent Loop (BB\w+)", m.group(2)))
            out.append(cur)
            continue
        if cur is not None:
            if line.strip().startswith(";"):
                cur["parents"] += re.findall(r"Parent Loop (BB\w+)", line)
                cur["ann"] += " " + line
            else:
                cur["lines"].append(line)
    return out


def divergent_barrier_loops(text):
    """[(kernel, loop header)] for every loop with an exec-mask latch in its
    own blocks and an s_barrier anywhere inside it (nested loops included)."""
    bykern = {}
    for b in _blocks(text):
        bykern.setdefault(b["kern"], []).append(b)
    found = []
    for kern, bl in bykern.items():
        parents = {b["name"]: b["parents"] for b in bl if "Loop Header" in b["ann"]}

        def chain(b):
            if "Loop Header" in b["ann"]:
                h = b["name"]
            else:
                m = re.search(r"in Loop: Header=(BB\w+)", b["ann"])
                if not m:
                    return []
                h = m.group(1)
            return [h] + parents.get(h, [])

        for h in parents:
            members = [b for b in bl if h in chain(b)]
            own = [b for b in members if chain(b)[0] == h]
            divergent = any(re.match(r"\s+s_andn2_b64 exec, exec,", ln)
                            for b in own for ln in b["lines"])
            barrier = any("s_barrier" in ln for b in members for ln in b["lines"])
            if divergent and barrier:
                found.append((kern, h))
    return found
