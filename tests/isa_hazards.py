"""MFMA wait-state scan of gfx950 assembly.

The d = 128 attention kernel issues its MFMAs as inline asm, which the
compiler's hazard recognizer does not look inside, so the wait states the
hardware needs around them are kept by the kernel's own construction.  This
scan checks them on the compiled assembly (a straight-line walk over the
listing, conservative at branches; a wait state is one issued instruction,
s_nop N counts N + 1):

  A. an MFMA (32x32x16, 8 passes) writes R; a later non-MFMA instruction
     reads or writes R                                      -> at least 12
  B. a VALU instruction (v_accvgpr_write included) writes R; a later MFMA
     reads R as an operand                                  -> at least 2
  C. an MFMA reads R as its accumulator; a later VALU instruction writes R
                                                            -> at least 12

The counts are the ones the compiler itself inserts around builtin MFMAs of
this shape on gfx950.
"""
from __future__ import annotations

import re

NEED_MFMA_TO_OTHER = 12
NEED_VALU_TO_MFMA = 2


def _regs(tok: str) -> set:
    m = re.match(r"^([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    if re.match(r"^[va]\d+$", tok):
        return {tok}
    return set()


def _split(line: str):
    parts = line.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    toks = [t.strip() for t in re.split(r",(?![^\[]*\])", parts[1].split(";")[0])]
    return parts[0], [t.split()[0] for t in toks if t]


def scan(lines) -> list:
    """Return one message per violation found in an assembly listing."""
    mfma_w, mfma_c, valu_w = {}, {}, {}
    clock = 0
    found = []
    for n, raw in enumerate(lines):
        line = raw.strip()
        if not line or line.startswith((";", ".", "_")) or line.endswith(":"):
            continue
        op, toks = _split(line)
        if op == "s_nop":
            clock += int(toks[0], 0) + 1
            continue
        if op.startswith("v_mfma"):
            d, a, b, c = (_regs(t) for t in toks[:4])
            for r in sorted(a | b | c):
                if r in valu_w and clock - valu_w[r] < NEED_VALU_TO_MFMA:
                    found.append(f"B {n}: {line} (VALU write of {r} {clock - valu_w[r]} before)")
                    break
            for r in d:
                mfma_w[r] = clock
            for r in c:
                mfma_c[r] = clock
        elif op.startswith(("v_", "ds_", "global_", "buffer_", "scratch_", "flat_")):
            used = set().union(*(_regs(t) for t in toks)) if toks else set()
            for r in sorted(used):
                if r in mfma_w and clock - mfma_w[r] < NEED_MFMA_TO_OTHER:
                    found.append(f"A {n}: {line} (MFMA write of {r} {clock - mfma_w[r]} before)")
                    break
            if op.startswith("v_") and toks:
                dst = _regs(toks[0])
                for r in sorted(dst):
                    if r in mfma_c and clock - mfma_c[r] < NEED_MFMA_TO_OTHER:
                        found.append(f"C {n}: {line} (MFMA accumulator read of {r} {clock - mfma_c[r]} before)")
                        break
                if not op.startswith(("v_readlane", "v_readfirstlane", "v_cmp")):
                    for r in dst:
                        valu_w[r] = clock
        clock += 1
    return found


def functions(asm_text: str, name_part: str) -> dict:
    """Split an assembly file into {symbol: lines} for the functions whose name contains name_part."""
    out, cur = {}, None
    for line in asm_text.splitlines():
        m = re.match(r"^([A-Za-z_][\w.$]*):", line)
        if m and not m.group(1).startswith(".") and "$" not in m.group(1):
            cur = m.group(1) if name_part in m.group(1) else None
            if cur:
                out[cur] = []
            continue
        if cur is not None:
            out[cur].append(line)
            if "s_endpgm" in line:
                cur = None
    return out
