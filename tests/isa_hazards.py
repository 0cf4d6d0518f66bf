"""Static check of matrix-core data hazards in gfx950 assembly.

The bf16 BoB passes issue their MFMAs as inline assembly so that the register
class of every operand is fixed; the compiler then no longer inserts the wait
states around those instructions, and the kernels place them explicitly.  This
module re-checks the final assembly (hipcc -S of the library) instruction by
instruction, in program order, against the wait-state counts the compiler
itself uses for v_mfma_f32_32x32x16_bf16 on gfx950 (measured from the s_nop it
emits around the builtin):

  R1  VALU writes a register  -> an MFMA reads it (A, B or C):            2
  R2  MFMA writes a register  -> any other instruction reads or writes it: 12
  R3  MFMA reads a VGPR as C  -> another instruction writes it:            7
  R4  MFMA writes a register  -> an MFMA reads it as A or B, or as C with
      a different register range:                                         12
      (accumulating into exactly the same range back to back needs none)

A wait state is one issued instruction; s_nop N counts N + 1.  The check
follows the text order, which is exact inside a basic block and conservative
enough across the loop back edges here because every chain ends in an
explicit fence before its consumers.
"""
from __future__ import annotations

import re

R1, R2, R3, R4 = 2, 12, 7, 12


def _regs(tok):
    m = re.match(r"^([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"^([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _parse(line):
    line = line.split(";")[0].strip()
    if not line or line.endswith(":") or line.startswith("."):
        return None
    parts = line.split(None, 1)
    ops = [o.strip() for o in re.split(r",\s*(?![^\[]*\])", parts[1])] if len(parts) > 1 else []
    return parts[0], ops


def check_kernel(lines, name=""):
    """Findings (strings) for one kernel's assembly lines."""
    insts = [p for p in (_parse(ln) for ln in lines) if p]
    errs = []
    valu_w, mfma_w, mfma_c = {}, {}, {}
    pos = 0
    for k, (op, ops) in enumerate(insts):
        if op == "s_nop":
            pos += int(ops[0], 0) + 1
            continue
        is_mfma = op.startswith("v_mfma")
        is_valu = op.startswith("v_") and not is_mfma
        dst, srcs = set(), []
        if is_mfma:
            dst = _regs(ops[0])
            srcs = [("A", _regs(ops[1])), ("B", _regs(ops[2])), ("C", _regs(ops[3]) if len(ops) > 3 else set())]
        elif op.startswith("global_load_lds"):
            srcs = [("x", _regs(o)) for o in ops]
        elif is_valu or op.startswith(("ds_read", "global_load", "buffer_load", "scratch_load", "flat_load")):
            writes_vreg = not (is_valu and op.startswith(("v_cmp", "v_readfirstlane", "v_readlane")))
            dst = _regs(ops[0]) if ops and writes_vreg else set()
            srcs = [("x", _regs(o)) for o in ops[1:]]
        else:
            srcs = [("x", _regs(o)) for o in ops]
        for kind, rs in srcs:
            for r in rs:
                if is_mfma:
                    if r in valu_w and pos - valu_w[r] < R1:
                        errs.append(f"R1 {name} #{k} {op} reads {r} {pos - valu_w[r]} after a VALU write")
                    if r in mfma_w:
                        p0, rng = mfma_w[r]
                        if kind == "C" and rng == tuple(sorted(rs)):
                            continue
                        if pos - p0 < R4:
                            errs.append(f"R4 {name} #{k} {op} reads {r} as {kind} {pos - p0} after an MFMA write")
                elif r in mfma_w and pos - mfma_w[r][0] < R2:
                    errs.append(f"R2 {name} #{k} {op} reads {r} {pos - mfma_w[r][0]} after an MFMA write")
        if not is_mfma:
            for r in dst:
                if r in mfma_w and pos - mfma_w[r][0] < R2:
                    errs.append(f"R2 {name} #{k} {op} writes {r} {pos - mfma_w[r][0]} after an MFMA write")
                if r in mfma_c and pos - mfma_c[r] < R3:
                    errs.append(f"R3 {name} #{k} {op} writes {r} {pos - mfma_c[r]} after an MFMA read it as C")
        if is_mfma:
            rng = tuple(sorted(dst))
            for r in dst:
                mfma_w[r] = (pos, rng)
                valu_w.pop(r, None)
            for r in srcs[2][1]:
                mfma_c[r] = pos
        else:
            for r in dst:
                mfma_w.pop(r, None)
                if is_valu:
                    valu_w[r] = pos
                else:
                    valu_w.pop(r, None)
        pos += 1
    return errs


def check_asm(text, name_filter=""):
    """{kernel symbol: findings} for every kernel in an assembly listing."""
    lines = text.split("\n")
    out = {}
    i = 0
    while i < len(lines):
        m = re.match(r"^(_Z\S+):", lines[i])
        if m and name_filter in m.group(1):
            j = i
            while j < len(lines) and not lines[j].startswith(".Lfunc_end"):
                j += 1
            out[m.group(1)] = check_kernel(lines[i:j], m.group(1))
            i = j
        i += 1
    return out
