"""Build-time check of the LDS-DMA copies in the compiled kernels.

The kernels copy tiles from global memory into LDS with inline assembly
(``buffer_load_dwordx4 ... lds``), which the compiler's hazard recognizer
does not look into.  Two hardware rules apply to such a copy:

* a vector-memory instruction that reads an SGPR written by a vector ALU
  instruction (``v_readfirstlane``, ``v_readlane``, a compare into an SGPR
  pair, ...) needs five wait states after that write; the copy reads its
  buffer descriptor from four SGPRs;
* an LDS-DMA load needs one wait state after a scalar write of M0.

Each copy's asm statement starts with ``s_nop 4`` (five wait states) or,
for later copies of a batch that share a descriptor, ``s_nop 0`` (one).
This module walks back from every copy in the device assembly over
straight-line code, counting an instruction as one wait state and
``s_nop N`` as N + 1, and reports any vector-ALU write of a descriptor SGPR
inside the five-wait-state window, any scalar write of M0 directly before
the copy, and any block label inside the window (the copy could then be
reached from code the walk does not see).

The same listings also tell whether a kernel spills: a kernel whose private
segment is not empty keeps registers (or a stack) in scratch memory.  The
attention kernels are sized to fit their register budgets, and one that no
longer does slows down several-fold in the loops that spill, so a build
whose kernels use scratch fails as well.
"""

from __future__ import annotations

import re

_DMA = re.compile(r"^buffer_load_dword\w*\s.*\blds\b")
_SGPR_RANGE = re.compile(r"^s\[(\d+):(\d+)\]$")
_SGPR = re.compile(r"^s(\d+)$")
_WINDOW = 5


def _sgprs(tok: str) -> set:
    m = _SGPR_RANGE.match(tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = _SGPR.match(tok)
    return {int(m.group(1))} if m else set()


def _statements(text: str):
    """(line number, kind, text) for instructions and labels; comments and
    directives dropped.  kind is 'label' or 'inst'."""
    out = []
    for n, raw in enumerate(text.splitlines(), 1):
        line = raw.split(";", 1)[0].strip()
        if not line or line.startswith("."):
            if line.endswith(":"):
                out.append((n, "label", line))
            continue
        if line.endswith(":"):
            out.append((n, "label", line))
        else:
            out.append((n, "inst", line))
    return out


def _dest(inst: str) -> str:
    parts = inst.split(None, 1)
    return parts[1].split(",")[0].strip() if len(parts) > 1 else ""


def check_text(text: str) -> list:
    """Problems found in one assembly listing (empty when every copy is
    covered)."""
    st = _statements(text)
    problems = []
    for i, (n, kind, inst) in enumerate(st):
        if kind != "inst" or not _DMA.match(inst):
            continue
        ops = [t.strip() for t in inst.split(None, 1)[1].split(",")]
        desc = _sgprs(ops[1]) if len(ops) > 1 else set()
        prev = st[i - 1] if i > 0 else None
        if prev and prev[1] == "inst" and prev[2].startswith("s_") and _dest(prev[2]) == "m0":
            problems.append(f"line {n}: M0 written directly before the copy (line {prev[0]})")
        waits, covered = 0, set()
        j = i - 1
        while j >= 0 and waits < _WINDOW:
            pn, pkind, p = st[j]
            if pkind == "label":
                problems.append(f"line {n}: block start {p} within {waits} wait states of the copy")
                break
            op = p.split()[0]
            written = _sgprs(_dest(p))
            hit = written & (desc - covered)
            if hit and op.startswith("v_"):
                problems.append(f"line {n}: s{sorted(hit)} written by a vector ALU instruction "
                                f"{waits} wait states before the copy (line {pn}: {p})")
            covered |= written
            if op == "s_nop":
                waits += int(p.split()[1], 0) + 1
            else:
                waits += 1
            j -= 1
    return problems


def copies(text: str) -> int:
    return sum(1 for _, kind, inst in _statements(text) if kind == "inst" and _DMA.match(inst))


_KNAME = re.compile(r"^\s*\.name:\s+(\S+)")
_PRIVATE = re.compile(r"^\s*\.private_segment_fixed_size:\s+(\d+)")


def scratch_kernels(text: str) -> list:
    """(kernel symbol, bytes) for every kernel of the listing's code-object
    metadata whose private segment (scratch) is not empty."""
    out, name = [], None
    for line in text.splitlines():
        m = _KNAME.match(line)
        if m:
            name = m.group(1)
            continue
        m = _PRIVATE.match(line)
        if m and name is not None and int(m.group(1)) > 0:
            out.append((name, int(m.group(1))))
    return out
