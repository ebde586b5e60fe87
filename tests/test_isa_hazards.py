"""The compiled kernels hold no matrix-core operand read too soon after a vector-ALU write.

On gfx950 a VALU instruction that writes a register read by a following MFMA as its A or B
operand needs two wait states between them; with one, the MFMA reads the register's previous
contents.  The compiler inserts the wait states for the instructions it schedules, but not for
inline assembly, whose results it cannot see.  This test compiles every HIP source of the
library to gfx950 assembly (the build's own flags) and checks each MFMA against the last
writer of its A and B registers inside the basic block.  (The batched W4 kernel once took its
nibble unpack from an inline-assembly v_and_or_b32; two MFMAs of its first chunk then read a B
register one instruction after it was written, and the values of four activation positions per
32 were wrong.)"""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "hybrid_mamba2_decode_amd"))
import build  # noqa: E402

REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")
SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]
NEED = 2  # wait states between a VALU write and an MFMA read of the same register as A or B


def _regs(tok):
    out = set()
    for m in REG.finditer(tok):
        if m.group(4) is not None:
            out.add((m.group(1), int(m.group(4))))
        else:
            out |= {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    return out


def violations(asm_lines):
    """(function, writer, mfma, wait states) for every MFMA whose A or B register was last
    written by a VALU instruction fewer than NEED wait states before it (same basic block)."""
    bad, fn, window = [], None, []
    for raw in asm_lines:
        t = raw.split(";")[0].strip()
        if not t:
            continue
        if t.endswith(":"):  # a function or basic-block label
            if not t.startswith("."):
                fn = t[:-1]
            window = []
            continue
        if t.startswith("."):
            continue
        op = t.split()[0]
        rest = t[len(op):]
        ops = [o.strip() for o in rest.split(",")] if rest.strip() else []
        if op.startswith("v_mfma") and len(ops) >= 3:
            src = _regs(ops[1]) | _regs(ops[2])
            ws = 0
            for ptxt, pdst, pws, pop in reversed(window):
                if pdst & src:
                    if pop.startswith("v_") and not pop.startswith("v_mfma") and ws < NEED:
                        bad.append((fn, ptxt, t, ws))
                    break
                ws += pws
                if ws >= NEED:
                    break
        w = int(ops[0], 0) + 1 if op == "s_nop" and ops else 1
        stores = ("buffer_store", "global_store", "ds_write", "flat_store", "scratch_store", "s_")
        dst = _regs(ops[0]) if ops and not op.startswith(stores) else set()
        window.append((t, dst, w, op))
        del window[:-16]
    return bad


def test_checker_flags_a_one_instruction_gap():
    asm = ["k:", "\tv_and_or_b32 v161, v0, v125, v124", "\tv_lshrrev_b32_e32 v0, 8, v40",
           "\tv_mfma_f32_4x4x4_16b_f16 a[62:65], v[174:175], v[160:161], a[62:65]",
           "\tv_and_or_b32 v38, v1, v2, v3", "\ts_nop 0", "\tv_mov_b32_e32 v5, v6",
           "\tv_mfma_f32_4x4x4_16b_f16 a[0:3], v[38:39], v[8:9], 0"]
    bad = violations(asm)
    assert len(bad) == 1 and bad[0][3] == 1


@pytest.mark.parametrize("src", SOURCES)
def test_no_mfma_operand_hazard(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [build.HIPCC, *build.FLAGS, "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    bad = violations(open(out).read().splitlines())
    assert not bad, bad[:5]
