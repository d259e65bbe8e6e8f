"""Static check of hand-waited loads in compiled gfx950 assembly.

The pipelined chunk kernel issues some global loads as inline asm and waits
for them with explicit `s_waitcnt vmcnt`.  The compiler takes an asm output as
written when the asm issues, so it could reuse or copy a destination register
before the data arrives; the late return would then corrupt the register
(a corrupted address faults the GPU).  This check walks every path of the
compiled kernel (each inline-asm block is one step) from each such load and
reports any instruction that reads or writes the load's destination registers
before a wait that covers the load, and any path that ends the program first.

A wait covers the load only if the count it allows cannot include it.
`vmcnt(N)` lets the wave go on once at most N vector-memory operations are
outstanding.  Loads return in issue order, but a store (or atomic) issued
later may retire before an earlier load, so only later loads can be relied on
to still be outstanding: `vmcnt(N)` covers the load when at least N loads were
issued after it on the path that reaches the wait.  Stores issued after the
load count for nothing.  A wait that does not cover the load (it waits for
older loads) leaves it in flight, and the walk goes on past it.  Waits the
compiler inserted count like the inline-asm ones.

One form is taken on trust: an inline-asm block that branches between
`vmcnt(N)` and `vmcnt(0)` on a flag (the kernel's `vm_wait_or_all`) takes the
`vmcnt(0)` branch exactly when the N later loads were not issued, so it
covers the load on every path.  That relation between the flag and the
issued loads is the kernel's own, stated where it is used.
"""
from __future__ import annotations

import re
from typing import List, Tuple


def _regs(op: str) -> set:
    out = set()
    for m in re.finditer(r"v\[(\d+):(\d+)\]|v(\d+)\b", op):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def function_body(asm_text: str, symbol: str) -> List[str]:
    lines = asm_text.splitlines()
    start = next(i for i, l in enumerate(lines) if l.startswith(symbol + ":"))
    end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
    return lines[start:end]


_VM_LOADS = ("global_load", "buffer_load", "flat_load", "scratch_load")


def _vmcnts(body: List[str]) -> List[int]:
    return [int(m.group(1)) for x in body for m in [re.search(r"vmcnt\((\d+)\)", x)] if m]


def hazards(lines: List[str]) -> Tuple[int, List[str]]:
    """Returns (number of asm loads, list of hazard descriptions)."""
    steps = []          # ("label", name) | ("inst", idx, text) | ("asm", idx, [texts])
    i = 0
    while i < len(lines):
        t = lines[i].strip()
        if t.startswith(";;#ASMSTART"):
            body = []
            i += 1
            while not lines[i].strip().startswith(";;#ASMEND"):
                u = lines[i].strip()
                if u and not u.startswith(";"):
                    body.append(u)
                i += 1
            steps.append(("asm", i, body))
            i += 1
            continue
        m = re.match(r"^(\.LBB\d+_\d+):", t)
        if m:
            steps.append(("label", m.group(1)))
        elif t and not t.startswith(";") and not t.startswith("."):
            steps.append(("inst", i, t))
        i += 1
    labels = {st[1]: k for k, st in enumerate(steps) if st[0] == "label"}
    found, nloads = [], 0
    cap = 64
    for k, st in enumerate(steps):
        if st[0] != "asm":
            continue
        for ia, a in enumerate(st[2]):
            if not a.startswith("global_load"):
                continue
            nloads += 1
            dregs = _regs(a.split()[1].rstrip(","))
            # loads issued after this one inside the same asm block
            later0 = sum(1 for x in st[2][ia + 1:] if x.startswith(_VM_LOADS))
            stack, visited, bad = [(k + 1, later0)], set(), None
            while stack and bad is None:
                j, later = stack.pop()
                while j < len(steps):
                    key = (j, min(later, cap))
                    if key in visited:
                        break
                    visited.add(key)
                    sj = steps[j]
                    if sj[0] == "label":
                        j += 1
                        continue
                    if sj[0] == "asm":
                        waits = _vmcnts(sj[2])
                        if waits and (max(waits) <= later or (len(waits) > 1 and min(waits) == 0)):
                            break                   # covered on every branch of the block
                        later += sum(1 for x in sj[2] if x.startswith(_VM_LOADS))
                        j += 1
                        continue
                    text = sj[2]
                    if text.startswith("s_waitcnt"):
                        waits = _vmcnts([text])
                        if waits and waits[0] <= later:
                            break
                        j += 1
                        continue
                    parts = text.split(None, 1)
                    if len(parts) > 1 and _regs(parts[1]) & dregs:
                        bad = text
                        break
                    if text.startswith(_VM_LOADS):
                        later += 1
                    if text.startswith("s_endpgm"):
                        bad = text
                        break
                    if text.startswith("s_branch"):
                        stack.append((labels[text.split()[1]], later))
                        break
                    if text.startswith("s_cbranch"):
                        stack.append((labels[text.split()[1]], later))
                    j += 1
            if bad is not None:
                found.append(f"{a}  ->  {bad}")
    return nloads, found


_SEXT_OPS = ("s_bfe_i64", "s_bfe_i32", "s_ashr_i64", "s_ashr_i32", "s_sext_i32_i8", "s_sext_i32_i16")


def _sregs(op: str) -> set:
    out = set()
    for m in re.finditer(r"s\[(\d+):(\d+)\]|\bs(\d+)\b", op):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def sign_extended_bases(lines: List[str]) -> Tuple[int, List[str]]:
    """Loads whose scalar 64-bit base was last written by a sign extension.

    A global load with a scalar base adds a zero-extended 32-bit lane offset
    to the full 64-bit base, so the base must carry the pointer's own upper
    half; a base built by sign-extending a 32-bit value is a truncated
    pointer.  For each such load the nearest earlier instruction in program
    text that writes any of the base registers is inspected.  Returns
    (number of scalar-base loads, list of offending loads).
    """
    insts = []
    for l in lines:
        t = l.split(";")[0].strip()
        if t and not t.startswith(".") and not t.endswith(":"):
            insts.append(t)
    n, found = 0, []
    for i, t in enumerate(insts):
        m = re.match(r"global_load_\w+\s+[^,]+,\s*v\d+,\s*(s\[\d+:\d+\])", t)
        if not m:
            continue
        n += 1
        base = _sregs(m.group(1))
        for j in range(i - 1, -1, -1):
            w = insts[j]
            op = w.split()[0]
            if not op.startswith("s_") or len(w.split()) < 2:
                continue
            dst = _sregs(w.split(None, 1)[1].split(",")[0])
            if dst & base:
                if op in _SEXT_OPS:
                    found.append(f"{t}  <-  {w}")
                break
    return n, found
