"""Scan gfx950 device assembly for inline-asm LDS reads left in flight.

The kernels read LDS with ordinary loads (the compiler places the waits)
except where a handful of reads must go out together: there an inline-asm
statement issues them and ends with ``s_waitcnt lgkmcnt(0)``, so no result
register is still being written when the statement ends.  (The compiler
takes an asm output as written when the statement ends; a read still in
flight could land in a register that by then holds something else.)

``asm_blocks`` splits a function's assembly into its inline-asm statements
(the ``;;#ASMSTART`` / ``;;#ASMEND`` markers); ``unwaited_reads`` returns the
statements with a ``ds_read`` that no later ``s_waitcnt lgkmcnt(0)`` in the
same statement completes.  ``scan`` is the older, stricter check of the
whole text: any instruction touching a register between an asm read writing
it and the wait that completes the read.
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


def _instructions(raw_lines):
    for raw in raw_lines:
        text = raw.split(";")[0].strip()
        if text and not text.startswith(".") and not text.endswith(":"):
            yield text


def asm_blocks(asm: str):
    """Yield (function, first line number, [instructions]) per inline-asm statement."""
    fn, block, start = None, None, 0
    for ln, raw in enumerate(asm.splitlines(), 1):
        m = _FN.match(raw)
        if m:
            fn = m.group(1)
            continue
        line = raw.strip()
        if line.startswith(";;#ASMSTART"):
            block, start = [], ln
            continue
        if line.startswith(";;#ASMEND"):
            if block is not None:
                yield fn, start, block
            block = None
            continue
        if block is not None:
            block.extend(_instructions([raw]))


def unwaited_reads(asm: str):
    """Return (bad statements, statements with LDS reads): a statement is bad
    if a ds_read in it is not followed, inside it, by s_waitcnt lgkmcnt(0)."""
    bad, n = [], 0
    for fn, ln, ins in asm_blocks(asm):
        reads = [i for i, t in enumerate(ins) if t.startswith("ds_read")]
        if not reads:
            continue
        n += 1
        waits = [i for i, t in enumerate(ins)
                 if t.startswith("s_waitcnt") and _LGKM.search(t) and _LGKM.search(t).group(1) == "0"]
        if not waits or max(waits) < max(reads):
            bad.append((fn, ln, ins))
    return bad, n


def scan(asm: str):
    """Return (hazards, n_asm_reads, n_functions) for assembly text.

    Each hazard is (function, line number, instruction, register): an
    instruction other than a wait that reads or writes a register between an
    asm LDS read writing it and the wait that completes that read (reads
    complete in issue order, so lgkmcnt(N) completes all but the N most
    recent).  The scan is linear (no control-flow graph).
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
