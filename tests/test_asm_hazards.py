"""The pair prefill kernel's inline-asm DPP multiply-adds, checked in the
compiled gfx950 assembly (CPU only: hipcc cross-compiles).

The diagonal inverse issues `v_fmac_f32_dpp ... row_newbcast:K` from inline
asm.  A DPP read of a VGPR needs 2 wait states after a VALU instruction
writes that VGPR; the compiler inserts them for its own DPP instructions but
cannot see inside an asm block, and the blocks carry no `s_nop` because their
DPP sources (rows of A read from LDS) are never written by VALU code.  This
test compiles the kernel file with the library's flags and checks every such
instruction of every instantiation: no VALU write of its DPP source within the
2 preceding wait states, and no MFMA result among its operands within the 24
preceding instructions (an MFMA write also needs wait states before a VALU
read).  A register copy placed by the compiler just before a block would fail
it.
"""
import os
import re
import shutil
import subprocess

import pytest

from gated_deltanet_state_delta_amd import build as gdn_build


def _regs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"^([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    m = re.match(r"^([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return set()


def _parse(line):
    s = line.split(";")[0].strip()
    if not s or s.startswith(".") or s.endswith(":"):
        return None
    parts = s.split(None, 1)
    ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
    return parts[0], ops


def dpp_asm_hazards(lines):
    """(number of asm DPP instructions checked, list of hazards found)."""
    hist, inasm, bad, n = [], False, [], 0
    for ln, line in enumerate(lines, 1):
        if ";;#ASMSTART" in line:
            inasm = True
            continue
        if ";;#ASMEND" in line:
            inasm = False
            continue
        if line.startswith(".Lfunc_end") or (line.startswith("_Z") and line.rstrip().endswith(":")):
            hist = []
        p = _parse(line)
        if p is None:
            continue
        op, ops = p
        if inasm and "_dpp" in op and "row_newbcast" in line:
            n += 1
            src0 = _regs(ops[1].split()[0])
            used = src0 | _regs(ops[0]) | _regs(ops[2].split()[0])
            ws = 0
            for pop, pops, pln in reversed(hist):
                if ws >= 2:
                    break
                if pop.startswith("v_") and not pop.startswith("v_mfma") and pops and _regs(pops[0]) & src0:
                    bad.append("line %d: DPP source written by line %d (%s)" % (ln, pln, pop))
                ws += int(pops[0], 0) + 1 if pop == "s_nop" and pops else 1
            for pop, pops, pln in list(reversed(hist))[:24]:
                if pop.startswith("v_mfma") and _regs(pops[0]) & used:
                    bad.append("line %d: operand written by MFMA at line %d" % (ln, pln))
        hist.append((op, ops, ln))
        if len(hist) > 64:
            hist.pop(0)
    return n, bad


def test_checker_finds_a_planted_hazard():
    asm = ["_Zk:", "\tv_mov_b32 v5, v6", "\t;;#ASMSTART",
           "\tv_fmac_f32_dpp v1, v5, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf", "\t;;#ASMEND",
           "\tv_mov_b32 v7, v6", "\ts_nop 1", "\t;;#ASMSTART",
           "\tv_fmac_f32_dpp v1, v7, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf", "\t;;#ASMEND",
           "\tv_mfma_f32_16x16x32_bf16 v[8:11], v[12:15], v[16:19], v[8:11]", "\t;;#ASMSTART",
           "\tv_fmac_f32_dpp v9, v20, v2 row_newbcast:3 row_mask:0xf bank_mask:0xf", "\t;;#ASMEND"]
    n, bad = dpp_asm_hazards(asm)
    assert n == 3 and len(bad) == 2, bad


def test_pair_kernel_dpp_blocks_need_no_wait_states(tmp_path):
    hipcc = gdn_build.hipcc()
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    src = os.path.join(gdn_build.CSRC, "gdn_prefill_pair.hip")
    out = str(tmp_path / "pair.s")
    cmd = ([hipcc] + gdn_build.COMMON + gdn_build.DEVICE_FLAGS + gdn_build.FILE_FLAGS.get("gdn_prefill_pair.hip", [])
           + ["--cuda-device-only", "-S", src, "-o", out])
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    n, bad = dpp_asm_hazards(open(out).read().split("\n"))
    # 24 instantiations (dk 64/128 x fused gate x L2 norm x {one request,
    # segments, multi-request walk}) x 120 fused multiply-adds of the
    # four-block inverse
    assert n == 24 * 120, n
    assert not bad, bad[:10]
