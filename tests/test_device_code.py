"""Static checks of the gfx950 device code the kernels compile to (no GPU needed).

A direct load whose 64-bit base comes from SGPRs (global_load_lds_dwordx4 with an
SGPR address) may read those SGPRs only five wait states after a vector-ALU
instruction wrote them (v_readfirstlane of a base held in VGPRs). The compiler
keeps that distance before memory instructions it emits itself, but the direct
loads are inline assembly it cannot see into, so the helper inserts the wait
before the first load from each newly formed base. This test compiles the
kernels to assembly with the library's own flags and checks every such load:
walking back from it, five wait states (an s_nop n counts n + 1, any other
instruction 1) must pass before any vector instruction that writes one of its
base SGPRs, and before any label (an unknown predecessor counts as a failure).
"""
import os
import re
import shutil
import subprocess

import pytest

from block_sparse_attention_causal_amd import build as hip_build

CSRC = os.path.join(os.path.dirname(hip_build.__file__), "csrc")
SADDR_LOAD = re.compile(r"global_load_lds_dwordx4\s+v\d+,\s*s\[(\d+):(\d+)\]")


def _device_asm(src, tmp_path):
    out = str(tmp_path / (os.path.basename(src) + ".s"))
    cmd = [hip_build.HIPCC, *hip_build.FLAGS, "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def _violations(asm):
    bad, checked = [], 0
    for m in re.finditer(r"^(_Z\w+):", asm, re.M):
        end = asm.index(".Lfunc_end", m.end())
        lines = [l.strip() for l in asm[m.end():end].splitlines()]
        lines = [l for l in lines if l and not l.startswith((";", ".cfi", ".loc", ".file"))]
        for k, line in enumerate(lines):
            mm = SADDR_LOAD.match(line)
            if not mm:
                continue
            checked += 1
            regs = {"s" + mm.group(1), "s" + mm.group(2)}
            states, ok = 0, False
            for back in range(k - 1, -1, -1):
                x = lines[back]
                if states >= 5:
                    ok = True
                    break
                if x.endswith(":") or x.startswith("s_cbranch") or x.startswith("s_branch"):
                    break                               # another path may reach the load
                if x.startswith("."):
                    continue
                op = x.split()[0]
                if op == "s_nop":
                    states += int(x.split()[1], 0) + 1
                    continue
                if op.startswith("v_") and x.split()[1].rstrip(",") in regs:
                    break
                states += 1
            if not ok and states >= 5:
                ok = True
            if not ok:
                bad.append("%s: %s (%d wait states)" % (m.group(1)[:60], line, states))
    return bad, checked


@pytest.mark.skipif(not (os.path.exists(hip_build.HIPCC) or shutil.which("hipcc")),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", ["attention.hip", "backward.hip"])
def test_sgpr_based_direct_loads_wait_after_vector_writes(src, tmp_path):
    bad, checked = _violations(_device_asm(os.path.join(CSRC, src), tmp_path))
    assert checked > 0, "no SGPR-based direct loads found: the check no longer applies"
    assert not bad, "\n".join(bad[:10])


def test_checker_flags_a_short_distance():
    """The scan itself: a readfirstlane right before the load is caught, and an
    s_nop 4 in between clears it."""
    body = ("_Zk:\n\tv_readfirstlane_b32 s2, v4\n\ts_mov_b32 m0, s5\n"
            "\tglobal_load_lds_dwordx4 v6, s[2:3]\n.Lfunc_end0:\n")
    bad, checked = _violations(body)
    assert checked == 1 and len(bad) == 1
    fixed = body.replace("\ts_mov_b32 m0, s5\n", "\ts_mov_b32 m0, s5\n\ts_nop 4\n")
    bad, checked = _violations(fixed)
    assert checked == 1 and not bad
