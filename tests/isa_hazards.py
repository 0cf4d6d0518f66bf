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

and two rules of the LDS-DMA copies, which are inline assembly as well (the
compiler inserts these waits for its own memory instructions only):

  R5  VALU writes an SGPR (v_readlane / v_readfirstlane, e.g. a spilled SGPR
      coming back)  -> a VMEM instruction reads it (address base):         5
  R6  SALU writes M0  -> an LDS-DMA load (global_load_lds_*) uses it:      1

A wait state is one issued instruction between the two (s_nop N counts
N + 1); a hazard is fewer wait states than the rule asks.  check_kernel
follows the text order, which is exact inside a basic block; check_loops
re-runs it over each loop body followed by itself, so that the instructions
before a back edge are checked against those after it.
"""
from __future__ import annotations

import re

R1, R2, R3, R4, R5, R6 = 2, 12, 7, 12, 5, 1


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


def _sregs(tok):
    m = re.match(r"^s\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"^s(\d+)$", tok)
    if m:
        return {int(m.group(1))}
    return {"m0"} if tok == "m0" else set()


def check_kernel(lines, name=""):
    """Findings (strings) for one kernel's assembly lines."""
    insts = [p for p in (_parse(ln) for ln in lines) if p]
    errs = []
    valu_w, mfma_w, mfma_c = {}, {}, {}
    valu_sw, salu_m0 = {}, None  # SGPR -> position of a VALU write; position of an M0 write
    pos = 0
    for k, (op, ops) in enumerate(insts):
        if op == "s_nop":
            pos += int(ops[0], 0) + 1
            continue
        if op.startswith(("global_", "buffer_", "flat_", "scratch_")):
            for o in ops[1:]:
                for r in _sregs(o):
                    if r in valu_sw and pos - valu_sw[r] - 1 < R5:
                        errs.append(f"R5 {name} #{k} {op} reads s{r} {pos - valu_sw[r] - 1} wait states after a VALU write")
            if "_lds" in op and salu_m0 is not None and pos - salu_m0 - 1 < R6:
                errs.append(f"R6 {name} #{k} {op} uses M0 {pos - salu_m0 - 1} wait states after it was written")
        sdst = _sregs(ops[0]) if ops else set()
        if op.startswith("v_") and sdst:
            for r in sdst:
                valu_sw[r] = pos
        elif op.startswith("s_") and sdst:
            for r in sdst:
                valu_sw.pop(r, None)
            if "m0" in sdst:
                salu_m0 = pos
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
                    if r in valu_w and pos - valu_w[r] - 1 < R1:
                        errs.append(f"R1 {name} #{k} {op} reads {r} {pos - valu_w[r] - 1} wait states after a VALU write")
                    if r in mfma_w:
                        p0, rng = mfma_w[r]
                        if kind == "C" and rng == tuple(sorted(rs)):
                            continue
                        if pos - p0 - 1 < R4:
                            errs.append(f"R4 {name} #{k} {op} reads {r} as {kind} {pos - p0 - 1} wait states after an MFMA write")
                elif r in mfma_w and pos - mfma_w[r][0] - 1 < R2:
                    errs.append(f"R2 {name} #{k} {op} reads {r} {pos - mfma_w[r][0] - 1} wait states after an MFMA write")
        if not is_mfma:
            for r in dst:
                if r in mfma_w and pos - mfma_w[r][0] - 1 < R2:
                    errs.append(f"R2 {name} #{k} {op} writes {r} {pos - mfma_w[r][0] - 1} wait states after an MFMA write")
                if r in mfma_c and pos - mfma_c[r] - 1 < R3:
                    errs.append(f"R3 {name} #{k} {op} writes {r} {pos - mfma_c[r] - 1} wait states after an MFMA read it as C")
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


def check_loops(lines, name=""):
    """Findings across loop back edges: every loop body (from a label to a
    later branch back to it) checked as two consecutive iterations."""
    labels, errs = {}, []
    for idx, ln in enumerate(lines):
        m = re.match(r"^(\.LBB\w+):", ln)
        if m:
            labels[m.group(1)] = idx
        m = re.match(r"^\s*s_(?:cbranch_\w+|branch)\s+(\.LBB\w+)", ln)
        if m and m.group(1) in labels and labels[m.group(1)] < idx:
            body = lines[labels[m.group(1)]:idx + 1]
            errs += [f"{e} (loop {m.group(1)})" for e in check_kernel(body + body, name)]
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
            out[m.group(1)] = check_kernel(lines[i:j], m.group(1)) + check_loops(lines[i:j], m.group(1))
            i = j
        i += 1
    return out
