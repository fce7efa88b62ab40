"""Static check of the inline-asm DPP products in the tree kernels (CPU; needs hipcc).

The power-step products (reblock.hip, fmac_row_bcast) issue v_fmac_f32_dpp through inline asm,
so the compiler's own hazard handling may not cover them.  A DPP operand must not be written by
a VALU instruction in the two issue slots before it (CDNA3/CDNA4 ISA, DPP hazards).  This test
compiles reblock.hip to gfx950 assembly and checks every v_fmac_f32_dpp against the
instructions before it on its fall-through path.  Its broadcast source should come from an LDS
read, never from a VALU write that close."""
import os
import re
import subprocess

import pytest

from block_sparse_video_reblock_amd import build as B


def _vregs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def dpp_hazards(asm_text):
    """(count of v_fmac_f32_dpp, list of (writer, dpp) pairs closer than two wait states)."""
    ins = []
    for line in asm_text.split("\n"):
        t = line.strip()
        if not t or t.startswith((";", ".")) or t.endswith(":"):
            continue
        ins.append(t)
    n, bad = 0, []
    for k, t in enumerate(ins):
        if not t.startswith("v_fmac_f32_dpp"):
            continue
        n += 1
        src = _vregs(t.split(None, 1)[1].split(",")[1])
        waits, j = 0, k - 1
        while j >= 0 and waits < 2:
            op = ins[j].split()[0]
            if op == "s_nop":
                waits += int(ins[j].split()[1]) + 1
            else:
                if op.startswith("v_") and " " in ins[j]:
                    dst = _vregs(ins[j].split(None, 1)[1].split(",")[0])
                    if dst & src:
                        bad.append((ins[j], t))
                waits += 1
            j -= 1
    return n, bad


def test_dpp_checker_flags_a_close_valu_write():
    # the checker itself: a VALU write of the broadcast source one slot before is flagged, a
    # write covered by s_nop 1 (two wait states) is not
    close = "v_mov_b32_e32 v7, v3\n v_fmac_f32_dpp v1, v7, v2 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
    covered = "v_mov_b32_e32 v7, v3\n s_nop 1\n v_fmac_f32_dpp v1, v7, v2 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
    assert dpp_hazards(close) == (1, [(close.split("\n")[0].strip(),
                                       close.split("\n")[1].strip())])
    assert dpp_hazards(covered)[1] == []


def test_tree_kernel_dpp_products_have_no_valu_hazard(tmp_path):
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc is not installed")
    out = tmp_path / "reblock.s"
    cmd = [B.HIPCC, *B.FLAGS, "--cuda-device-only", "-S",
           os.path.join(B.CSRC, "reblock.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    n, bad = dpp_hazards(out.read_text())
    assert n > 0
    assert bad == [], bad[:5]
