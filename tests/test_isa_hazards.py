"""The gfx950 assembly of the library has no unresolved matrix-core data
hazards (see tests/isa_hazards.py for the rules).  Host-only: hipcc
cross-compiles the device code to assembly; no GPU is used."""
import os
import shutil
import subprocess

import pytest

from exact_second_order_fa_amd import build
from tests.isa_hazards import check_asm, check_kernel, check_loops


def test_checker_flags_planted_hazards():
    """The checker itself: a VALU read 3 instructions after an MFMA write, a
    VALU-written operand read by the next MFMA, and a clean sequence."""
    bad = ["v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
           "s_nop 1",
           "v_add_f32_e32 v24, v0, v1"]
    assert any(e.startswith("R2") for e in check_kernel(bad))
    bad2 = ["v_mov_b32_e32 v16, 0", "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0"]
    assert any(e.startswith("R1") for e in check_kernel(bad2))
    # One wait state is one too few: an operand reloaded from an AGPR with a
    # single instruction before the MFMA (the two-waves-per-SIMD dK/dV
    # dropout kernel's wrong dK), and a zero-filled C copied in the same way.
    bad3 = ["v_accvgpr_read_b32 v23, a95", "s_waitcnt lgkmcnt(0)",
            "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]"]
    assert any(e.startswith("R1") for e in check_kernel(bad3))
    bad4 = ["v_mov_b64_e32 v[0:1], v[32:33]", "s_waitcnt lgkmcnt(0)",
            "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]"]
    assert any(e.startswith("R1") for e in check_kernel(bad4))
    assert check_kernel(["v_accvgpr_read_b32 v23, a95", "s_nop 1",
                         "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]"]) == []
    good = ["v_mov_b32_e32 v16, 0", "s_nop 1",
            "v_mfma_f32_32x32x16_bf16 a[0:15], v[16:19], v[20:23], a[0:15]",
            "v_mfma_f32_32x32x16_bf16 a[0:15], v[16:19], v[20:23], a[0:15]",
            "s_nop 7", "s_nop 3", "v_accvgpr_read_b32 v30, a3"]
    assert check_kernel(good) == []


def test_checker_flags_planted_dma_and_back_edge_hazards():
    """R5: a spilled SGPR read back by v_readlane and used at once as the base
    of an LDS-DMA load; R6: M0 written right before the load; a hazard that
    only exists from the end of a loop body to its start."""
    bad5 = ["v_readlane_b32 s4, v127, 2", "s_mov_b32 m0, s8", "s_nop 0",
            "global_load_lds_dwordx4 v4, s[4:5]"]
    assert any(e.startswith("R5") for e in check_kernel(bad5))
    good5 = ["v_readlane_b32 s4, v127, 2", "s_nop 3", "s_mov_b32 m0, s8", "s_nop 0",
             "global_load_lds_dwordx4 v4, s[4:5]"]
    assert check_kernel(good5) == []
    bad6 = ["s_mov_b32 m0, s8", "global_load_lds_dwordx4 v4, s[4:5]"]
    assert any(e.startswith("R6") for e in check_kernel(bad6))
    loop = [".LBB0_1:", "v_add_f32_e32 v0, v1, v2",
            "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0",
            "s_cbranch_scc1 .LBB0_1"]
    assert check_kernel(loop) == []           # straight-line: no reader after the MFMA
    assert any(e.startswith("R2") for e in check_loops(loop))  # next iteration's VALU writes v0


def test_tile_loop_scratch_rule():
    """The spill rule of the library test: scratch stores, or more than four
    reloads, inside a loop nested in another one fail; outside they pass."""
    def kernel(inner):
        return [".LBB0_1:", "scratch_store_dword off, v1, off", ".LBB0_2:",
                "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], 0", *inner,
                "s_cbranch_scc1 .LBB0_2", "scratch_load_dword v1, off, off", "s_cbranch_scc1 .LBB0_1"]
    assert tile_loops_light(kernel([]))
    assert tile_loops_light(kernel(["scratch_load_dwordx2 v[6:7], off, off"] * 4))
    assert not tile_loops_light(kernel(["scratch_load_dwordx2 v[6:7], off, off"] * 5))
    assert not tile_loops_light(kernel(["scratch_store_dword off, v1, off"]))
    assert not tile_loops_light(kernel([])[2:-2])  # no nested loop at all


@pytest.mark.skipif(not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")), reason="hipcc missing")
def test_library_assembly_has_no_mfma_hazards(tmp_path):
    out = tmp_path / "fa.s"
    cmd = [build.hipcc_path(), *[f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")],
           "--cuda-device-only", "-S", "-I", build.INCLUDE, "-I", os.path.dirname(build.SRC), "-o", str(out), build.SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = out.read_text()
    found = check_asm(text)
    for name in ("bob_pass1_ws", "bob_pass1_dma", "bob_pass2_dma"):
        assert any(name in k for k in found), name
    bad = {k: v for k, v in found.items() if v}
    assert not bad, {k: v[:5] for k, v in bad.items()}
    # The bf16 kernels keep everything in registers: a spill to scratch in
    # their key-tile loops would be a silent slowdown.  Three instances are a
    # few dwords short and spill at most 64 bytes: the d = 128 dropout BoB row
    # pass (five bf16 operand chains and the mask words beside 256 accumulator
    # AGPRs, with the U_Q rows already parked in LDS), the d = 128 dropout dQ
    # kernel, and the causal and the dropout two-wave column passes (two waves
    # per SIMD, 256 registers each).  Their spills are stored outside the
    # key-tile loops (the loops nested in another one); inside, at most four
    # reloads per tile are allowed (the causal row pass reloads three 8-byte
    # values before each tile's copy), six for the dropout two-wave column
    # pass (five 8-byte values around the copy of its next 64-row tile).
    def allowed(k, n):
        drop_row_pass = "bob_pass1_dma_kernelILi128ELi64E" in k and k.endswith("ELi0ELb1ELb0EEEvNS_4ArgsE")
        drop_dq = "bwd_dq_dma_kernelILi128ELi64E" in k and k.endswith("ELb1EEEvNS_4ArgsE")
        two_causal = "bob_pass2_dma_kernelILi64ELi64E" in k and k.endswith("ELb1ELb0ELb1EEEvNS_4ArgsE")
        two_drop = "bob_pass2_dma_kernelILi64ELi64E" in k and k.endswith("ELb0ELb1ELb1EEEvNS_4ArgsE")
        return ((drop_row_pass or drop_dq or two_causal or two_drop) and n <= 64
                and tile_loops_light(kernel_lines(text, k), 6 if two_drop else 4))

    spills = {k: n for k, n in scratch_sizes(text).items()
              if ("bob_pass1_ws" in k or "_dma_" in k) and n and not allowed(k, n)}
    assert not spills, spills


def kernel_lines(text, sym):
    lines = text.splitlines()
    start = next(i for i, ln in enumerate(lines) if ln.startswith(sym + ":"))
    end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
    return lines[start:end]


def tile_loops_light(body, max_loads=4):
    """True if the kernel has loops with MFMAs nested inside another loop,
    none of them stores to scratch and each loads from it at most
    max_loads times."""
    import re

    labels, loops = {}, []
    for i, ln in enumerate(body):
        m = re.match(r"^(\.LBB\w+):", ln)
        if m:
            labels[m.group(1)] = i
        m = re.match(r"^\s*s_(?:cbranch_\w+|branch)\s+(\.LBB\w+)", ln)
        if m and m.group(1) in labels and labels[m.group(1)] < i:
            loops.append((labels[m.group(1)], i))
    inner = [body[a:b + 1] for a, b in loops
             if any(c <= a and b <= d and (c, d) != (a, b) for c, d in loops)
             and any("v_mfma" in ln for ln in body[a:b + 1])]
    return bool(inner) and all(
        not any("scratch_store" in ln for ln in lp) and sum("scratch_load" in ln for ln in lp) <= max_loads
        for lp in inner)


def scratch_sizes(text):
    """Kernel symbol -> ScratchSize from the assembler's resource comments."""
    import re

    out, cur = {}, None
    for line in text.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur = m.group(1)
        m = re.match(r"^; ScratchSize: (\d+)", line)
        if m and cur:
            out[cur] = int(m.group(1))
            cur = None
    return out
