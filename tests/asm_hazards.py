"""Static check of the MFMA data hazards that the compiler cannot see in the attention kernel.

The kernel issues its MFMAs as inline asm, so the compiler neither inserts the wait states an
MFMA result needs before a VALU instruction may read it, nor knows when an MFMA has finished
reading its accumulator.  This walks the generated gfx950 assembly of each kernel in program
order (straight-line, conservatively ignoring that a taken branch adds distance) and reports:

  RAW  an MFMA writes registers that a later VALU instruction (including v_accvgpr_read/mov)
       reads before the result is ready;
  WAR  a later VALU instruction overwrites an MFMA's accumulator input (SrcC) while the MFMA
       may still be reading it;
  OPND an MFMA reads as an operand a register that a VALU instruction wrote fewer than 2 wait
       states before.

Wait states: every instruction counts one, s_nop N counts N + 1.  Requirements for gfx950, the
ones the compiler itself inserts after the builtin forms: 12 after a 32x32x16 bf16 MFMA (8
passes) and 20 after a 32x32x64 e4m3 MFMA (16 passes) for RAW; 8 and 16 for SrcC WAR.
"""
from __future__ import annotations

import re

# A VALU write (v_accvgpr_write/mov included) of a register an MFMA then reads as SrcA/B/C needs 2
# wait states in between (what the compiler inserts, as s_nop 1, before its own MFMA builtins).
OPND_NEED = 2
RAW_NEED = {"v_mfma_f32_32x32x16_bf16": 12, "v_mfma_f32_32x32x64_f8f6f4": 20}
WAR_NEED = {"v_mfma_f32_32x32x16_bf16": 8, "v_mfma_f32_32x32x64_f8f6f4": 16}


def _regs(op: str):
    m = re.match(r"^([va])\[(\d+):(\d+)\]$", op)
    if m:
        return {(m.group(1), k) for k in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"^([va])(\d+)$", op)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def kernel_body(asm: str, name: str):
    i = asm.index(name + ":")
    j = asm.index("s_endpgm", i)
    return [l.split(";")[0].strip() for l in asm[i:j].split("\n")]


def check(lines):
    """Returns a list of (kind, mfma line, offending line, missing wait states)."""
    raw, war, found = [], [], []
    opnd = []  # recent VALU writes: an MFMA may read them as an operand only OPND_NEED wait states later
    for ln, l in enumerate(lines):
        if not l or l.endswith(":") or l.startswith("."):
            continue
        parts = l.replace(",", " ").split()
        op, args = parts[0], parts[1:]
        ws = int(args[0], 0) + 1 if op == "s_nop" else 1
        reads, writes = set(), set()
        if op.startswith("v_") and not op.startswith("v_mfma"):
            if args:
                writes = _regs(args[0])
            for a in args[1:]:
                reads |= _regs(a)
            if op.startswith(("v_dot2c", "v_mac", "v_fmac")):
                reads |= writes
        elif op.startswith(("ds_read", "global_load", "buffer_load", "scratch_load")) and args:
            writes = _regs(args[0])
        elif op.startswith(("ds_write", "global_store", "buffer_store", "scratch_store")):
            for a in args:
                reads |= _regs(a)
        if op in RAW_NEED:
            srcs = set()
            for x in args[1:4]:
                srcs |= _regs(x)
            for rem, rs, src in opnd:
                if rem > 0 and rs & srcs:
                    found.append(("OPND", l, lines[src], rem))
        for rem, rs, src in raw:
            if rem > 0 and rs & reads:
                found.append(("RAW", lines[src], l, rem))
        for rem, rs, src in war:
            if rem > 0 and rs & writes and op.startswith("v_"):
                found.append(("WAR", lines[src], l, rem))
        raw = [(r - ws, rs, s) for r, rs, s in raw if r - ws > 0]
        war = [(r - ws, rs, s) for r, rs, s in war if r - ws > 0]
        opnd = [(r - ws, rs, s) for r, rs, s in opnd if r - ws > 0]
        if op.startswith("v_") and not op.startswith("v_mfma") and writes:
            opnd.append((OPND_NEED, writes, ln))
        if op in RAW_NEED:
            raw.append((RAW_NEED[op], _regs(args[0]), ln))
            if len(args) >= 4:
                war.append((WAR_NEED[op], _regs(args[3]), ln))
    return found
