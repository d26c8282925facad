"""A lint over the compiled gfx950 assembly of every kernel source (CPU
only: hipcc cross-compiles).

The kernels read matrix-core results across lanes (DPP row operations,
v_permlane*, ds_bpermute/ds_swizzle) in a few places.  Such a read must not
issue before the MFMA that writes its source registers has landed; the
kernels pad every such read with an explicit fence of 20 wait states, since
the compiler's own hazard padding has not been enough for it on gfx950.  A
missing fence gives wrong values without any error, so this test checks the
compiled code: within each basic block, no lane-crossing instruction reads a
VGPR that an MFMA wrote fewer than MIN_WAIT_STATES wait states earlier
(every instruction counts one, `s_nop n` counts n + 1)."""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import __graft_entry__ as ge  # noqa: E402

MIN_WAIT_STATES = 18   # a 16-pass MFMA's result, with the margin the fences keep
HIP_SOURCES = [s for s in ge.SOURCES if s.endswith(".hip")]

_REG = re.compile(r"\bv(\d+)\b|\bv\[(\d+):(\d+)\]")
_LANE_CROSSING = re.compile(r"^(v_permlane|ds_bpermute|ds_permute|ds_swizzle)|"
                            r"\b(row_shl|row_shr|row_ror|row_mirror|row_half_mirror|row_bcast|row_newbcast|"
                            r"row_share|row_xmask|quad_perm|wave_shl|wave_shr|wave_ror|wave_rol)\b")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1) is not None:
            out.add(int(m.group(1)))
        else:
            out.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def hazards(asm: str):
    """(line number, instruction, distance) of every lane-crossing read of an
    MFMA destination closer than MIN_WAIT_STATES wait states."""
    found = []
    pending = {}   # VGPR -> wait-state clock at which its MFMA issued
    clock = 0
    for no, raw in enumerate(asm.splitlines(), 1):
        line = raw.split(";")[0].strip()
        if not line:
            continue
        if line.endswith(":"):   # a label: a new basic block
            pending.clear()
            continue
        if line.startswith("."):   # a directive
            continue
        op, _, args = line.partition(" ")
        if op.startswith("s_nop"):
            clock += int(args.strip() or 0, 0) + 1
            continue
        clock += 1
        if op.startswith("v_mfma"):
            dst = args.split(",")[0]
            for r in _regs(dst):
                pending[r] = clock
            continue
        if _LANE_CROSSING.search(line):
            srcs = args.split(",", 1)[1] if "," in args else args
            if op.startswith("v_permlane"):   # both operands are read
                srcs = args
            for r in _regs(srcs):
                if r in pending and clock - pending[r] < MIN_WAIT_STATES:
                    found.append((no, line, clock - pending[r]))
        if op.startswith("v_") and "," in args:
            for r in _regs(args.split(",")[0]):   # overwritten: no longer an MFMA result
                pending.pop(r, None)
    return found


def test_lint_flags_a_planted_hazard():
    """The lint itself: an unfenced permlane and DPP read of an MFMA result are
    flagged; fenced ones, and reads of other registers, are not."""
    bad = "\n".join([
        "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",
        "v_permlane32_swap_b32_e32 v3, v40",
        "v_add_f32_dpp v41, v5, v42 row_shr:1 row_mask:0xf bank_mask:0xf",
        "v_add_f32_dpp v43, v44, v45 row_shr:1 row_mask:0xf bank_mask:0xf",
    ])
    assert [h[2] for h in hazards(bad)] == [1, 2]
    good = "\n".join([
        "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",
        "s_nop 7", "s_nop 7", "s_nop 3",
        "v_permlane32_swap_b32_e32 v3, v40",
    ])
    assert hazards(good) == []
    block = "\n".join([
        "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",
        ".LBB0_1:",
        "v_permlane32_swap_b32_e32 v3, v40",
    ])
    assert hazards(block) == []


@pytest.mark.skipif(shutil.which(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")) is None, reason="no hipcc")
@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_unfenced_lane_crossing_read_of_mfma_results(src, tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    flags = [f for f in ge.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    out = tmp_path / (src + ".s")
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", "-I" + os.path.join(ROOT, "include"), "-I" + ge.CSRC,
           os.path.join(ge.CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    asm = out.read_text()
    # the matrix-core sources must have been linted on their MFMAs
    assert "v_mfma" in asm or src in ("kda_api.hip", "kda_backward.hip"), src
    found = hazards(asm)
    assert not found, found[:10]
