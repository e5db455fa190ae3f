"""Scan gfx950 device assembly for uses of in-flight inline-asm LDS reads.

The LDS rings issue their reads with inline asm that does not wait
(``ds_read_b128`` with an ``=v`` output) and wait later with an
``s_waitcnt lgkmcnt(N)``: LDS reads complete in issue order, so such a wait
completes every asm read but the N most recent (other LGKM operations issued
in between only make the hardware wait longer, so the scan's count is
conservative).  The compiler takes an asm output as written when
the asm statement ends, so it may copy, move or reuse such a register before
the wait, and the late-arriving data then lands in a register that holds
something else.  This scan walks each function's instructions in text order
and reports any instruction other than a wait that reads or writes a register
between an asm LDS read writing it and the wait that completes that read.

The scan is linear (no control-flow graph), so it is a guard against the
common forms of the mistake, not a proof of their absence.
"""
from __future__ import annotations

import re

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")
_FN = re.compile(r"^(_Z\w+):")
_LGKM = re.compile(r"lgkmcnt\((\d+)\)")


def _regs(text: str) -> set:
    out = set()
    for m in _REG.finditer(text):
        if m.group(4) is not None:
            out.add((m.group(1), int(m.group(4))))
        else:
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def scan(asm: str):
    """Return (hazards, n_asm_reads, n_functions) for assembly text.

    Each hazard is (function, line number, instruction, register).
    """
    hazards = []
    fn = None
    in_asm = False
    pending: dict = {}      # register -> sequence number of the asm read writing it
    seq = 0
    n_reads = n_fn = 0
    for ln, raw in enumerate(asm.splitlines(), 1):
        line = raw.strip()
        m = _FN.match(raw)
        if m:
            fn, pending = m.group(1), {}
            n_fn += 1
            continue
        if line.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if line.startswith(";;#ASMEND"):
            in_asm = False
            continue
        text = line.split(";")[0].strip()
        if not text or text.startswith(".") or text.endswith(":"):
            continue
        op, _, rest = text.partition(" ")
        if op == "s_waitcnt":
            w = _LGKM.search(rest)
            if w:
                keep = int(w.group(1))          # the N most recent reads may still be in flight
                pending = {r: q for r, q in pending.items() if q > seq - keep}
            continue
        if op == "s_endpgm":
            pending = {}
            continue
        used = _regs(rest)
        if in_asm and op.startswith("ds_read"):
            dst = _regs(rest.split(",")[0])
            for r in sorted((used - dst) & pending.keys()):
                hazards.append((fn, ln, text, r))
            seq += 1
            for r in dst:
                pending[r] = seq
            n_reads += 1
            continue
        for r in sorted(used & pending.keys()):
            hazards.append((fn, ln, text, r))
    return hazards, n_reads, n_fn
