"""Checks on the compiled gfx950 code of the attention kernels (CPU only: hipcc
cross-compiles).

The direct tile copies of the ping-pong kernel are inline assembly that loads M0
(the LDS address of a global -> LDS copy) without saving it: M0 is a register the
compiler reserves, so it cannot honour a clobber of it.  That is correct only while
no compiler-generated instruction of a kernel holding those copies uses M0.
"""
import pathlib
import re
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
CSRC = ROOT / "segmented_attention_seq_amd" / "csrc"
HIPCC = "/opt/rocm/bin/hipcc"


def _kernels(asm):
    """(name, body) of every kernel function in an assembly listing (a body runs
    from the function's label to its .Lfunc_end marker, past any early exits)."""
    out = []
    for m in re.finditer(r"^(_Z\S+):\s*;\s*@\1\n(.*?)^\.Lfunc_end\d+:", asm, re.S | re.M):
        out.append((m.group(1), m.group(2)))
    return out


def _outside_inline_asm(body):
    keep, inside = [], False
    for line in body.splitlines():
        if ";;#ASMSTART" in line:
            inside = True
        elif ";;#ASMEND" in line:
            inside = False
        elif not inside:
            keep.append(line.split(";")[0])
    return keep


@pytest.mark.skipif(not shutil.which(HIPCC) and not pathlib.Path(HIPCC).exists(), reason="hipcc not available")
def test_direct_copy_kernels_leave_m0_to_their_inline_asm(tmp_path):
    out = tmp_path / "attention.s"
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", str(ROOT / "include"), "-I", str(CSRC), str(CSRC / "attention.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    bad = m0_conflicts(out.read_text())
    assert not bad, f"compiler code uses M0 beside the inline-asm copies: {bad}"


def m0_conflicts(asm):
    """Kernels holding the inline-asm copies whose compiler-generated code also
    uses M0, with the first offending lines."""
    kernels = _kernels(asm)
    assert kernels, "no kernels found in the listing"
    with_copies = [(n, b) for n, b in kernels
                   if re.search(r";;#ASMSTART\s*\n\s*s_mov_b32 m0,[^\n]*\n\s*s_nop 0\s*\n\s*global_load_lds_dwordx4", b)]
    assert with_copies, "no kernel holds the inline-asm tile copies"
    bad = {}
    for name, body in with_copies:
        uses = [l.strip() for l in _outside_inline_asm(body) if re.search(r"\bm0\b", l)]
        if uses:
            bad[name] = uses[:5]
    return bad
