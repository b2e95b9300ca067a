"""Static check of the kernels' gfx950 code (CPU; needs hipcc, not a GPU).

A VALU compare that writes a lane mask (an SGPR pair or vcc) must be two
wait states (issued instructions, an s_nop n counting n + 1) ahead of a VALU
instruction that reads that mask: the compiler keeps that distance in every
such pair it schedules for this target, and code in inline assembly is
outside its hazard checks, so the whole compiled file is checked here.
"""
import os
import re
import shutil

import pytest

from lossless_kv_cache_amd import build as b


def _pairs(lines):
    """(compare, reader, wait states) for every compare whose mask a VALU
    instruction reads in the same basic block before it is written again."""
    out = []
    for k, line in enumerate(lines):
        m = re.match(r"v_cmp\w*_e32 (vcc),", line) or re.match(r"v_cmp\w*_e64 (s\[\d+:\d+\]),", line)
        if not m:
            continue
        reg = re.compile(r"(?<![\w\[:])" + re.escape(m.group(1)) + r"(?![\w\]])")
        waits = 0
        for x in lines[k + 1:k + 24]:
            if not x or x.startswith(";"):
                continue
            if x.endswith(":") or x.startswith((".", "s_cbranch", "s_branch", "s_setpc", "s_endpgm")):
                break
            op, _, args = x.partition(" ")
            srcs = args.split(",", 1)[1] if "," in args else ""
            if op.startswith("v_") and reg.search(srcs):
                out.append((line, x, waits))
                break
            if reg.match(args):                            # the mask written again first
                break
            waits += int(args) + 1 if op == "s_nop" else 1
    return out


def test_compare_masks_read_two_wait_states_later(tmp_path):
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not installed")
    asm = b.device_asm(str(tmp_path / "kernels.s"))
    with open(asm) as f:
        lines = [ln.strip() for ln in f]
    pairs = _pairs(lines)
    assert len(pairs) > 500, len(pairs)                   # the scan finds the compares it is meant to
    short = [p for p in pairs if p[2] < 2]
    assert not short, short[:5]


def test_scan_flags_a_short_pair():
    """The scan itself: one instruction between a compare and a select that
    reads its mask is flagged, two are not, a redefinition ends the search."""
    one = ["v_cmp_ge_u32_e32 vcc, v1, v2", "s_mov_b64 s[4:5], vcc",
           "v_cndmask_b32_sdwa v0, v1, v1, vcc dst_sel:DWORD"]
    two = one[:2] + ["s_nop 0"] + one[2:]
    redef = ["v_cmp_gt_u32_e64 s[0:1], v1, v2", "v_cmp_lt_u32_e64 s[0:1], v3, v4",
             "v_cndmask_b32_e64 v0, v1, v2, s[0:1]"]
    assert [p[2] for p in _pairs(one)] == [1]
    assert [p[2] for p in _pairs(two)] == [2]
    assert [p[2] for p in _pairs(redef)] == [0]           # only the second compare's pair
