"""Static check of the compiled kernels (CPU only): no vector instruction may
touch a register that a matrix instruction writes before that instruction
has finished writing it.

gfx950 does not interlock a VALU read or write of an MFMA's destination
registers: software must leave enough issue slots between them (`s_nop n`
counts n + 1). The compiler pads these gaps itself; in the minimal case (an
MFMA followed at once by a dependent multiply) it pads
  v_mfma_f32_32x32x64_f8f6f4 (16 passes with fp8 operands): 20 slots,
  v_mfma_f32_32x32x16_f16: 12 slots,
  v_mfma_f32_16x16x32_fp8_fp8: 8 slots,
which is the requirement this test enforces. In two instantiations of the
few-token GEMM the compiler once left 19 slots before the first multiply
of the last result register of a 32 x 32 x 64 MFMA; the GPU then read a
stale value there (a parity test saw exactly that register wrong in every
tile). The kernel was restructured so that no rescale reads the MFMA issued
just before it; this test keeps any kernel from regressing into such a gap.

The scan follows the straight-line fall-through path after each MFMA (up to
an unconditional branch or the end of the program), counting every issued
instruction as one slot. A gap across a taken branch is not seen.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

REQUIRED = {
    "v_mfma_f32_32x32x64_f8f6f4": 20,
    "v_mfma_scale_f32_32x32x64_f8f6f4": 20,
    "v_mfma_f32_32x32x16_f16": 12,
    "v_mfma_f32_16x16x32_fp8_fp8": 8,
}
SOURCES = ["rrs_gemm.hip", "rrs_gemm_small.hip", "rrs_frontend.hip", "rrs_frontend_kron.hip"]

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def _regs(text):
    out = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", text):
        if m.group(3) is not None:
            out.add(int(m.group(3)))
        else:
            out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def scan(lines):
    """(slots, mfma line, instruction) for every VALU touch of an MFMA's
    destination closer than the requirement, on the fall-through path."""
    bad = []
    for i, line in enumerate(lines):
        s = line.strip()
        op = s.split()[0] if s else ""
        if op not in REQUIRED:
            continue
        need = REQUIRED[op]
        pending = _regs(s.split(None, 1)[1].split(",")[0])
        slots = 0
        for t in lines[i + 1:]:
            t = t.strip()
            if not t or t.startswith((";", ".")) or t.endswith(":"):
                continue
            top = t.split()[0]
            if top in ("s_branch", "s_endpgm", "s_setpc_b64") or slots >= need or not pending:
                break
            if top == "s_nop":
                slots += int(t.split()[1], 0) + 1
                continue
            if top.startswith("v_") and " " in t:
                touched = _regs(t.split(None, 1)[1]) & pending
                if touched and not top.startswith("v_mfma"):
                    bad.append((slots, s[:70], t[:70]))
                    pending -= touched
                elif touched:
                    pending -= touched  # chained into another MFMA: its own rule, padded by the compiler
            slots += 1
    return bad


def _asm(src, outdir):
    import rotated_runtime_activation_amd.build as b
    out = os.path.join(outdir, src + ".s")
    cmd = [b.hipcc(), *b.flags(), "--cuda-device-only", "-S", os.path.join(b.CSRC, src), "-o", out]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    return out


def test_scan_flags_a_short_gap():
    """The scan itself: 19 slots before a read of a 32 x 32 x 64 result is
    flagged, 20 are not."""
    mf = "v_mfma_f32_32x32x64_f8f6f4 v[0:15], v[16:23], v[24:31], v[0:15]"
    short = [mf, "s_nop 15", "s_nop 2", "v_mul_f32_e32 v15, v40, v15"]
    ok = [mf, "s_nop 15", "s_nop 3", "v_mul_f32_e32 v15, v40, v15"]
    assert scan(short) and not scan(ok)
    # an intervening redefinition by another MFMA ends the watch
    chained = [mf, "v_mfma_f32_32x32x64_f8f6f4 v[0:15], v[16:23], v[24:31], v[0:15]", "s_nop 15", "s_nop 3",
               "v_mul_f32_e32 v15, v40, v15"]
    assert not scan(chained[:1] + chained[1:2])  # no VALU touch at all


def test_no_short_mfma_to_valu_gaps(tmp_path):
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        paths = list(ex.map(lambda s: _asm(s, str(tmp_path)), SOURCES))
    problems = []
    for path in paths:
        lines = open(path).read().split("\n")
        starts = [(i, l.split(":")[0]) for i, l in enumerate(lines) if re.match(r"^_Z\S+:", l)]
        for k, (i, name) in enumerate(starts):
            end = starts[k + 1][0] if k + 1 < len(starts) else len(lines)
            for slots, mf, instr in scan(lines[i:end]):
                problems.append(f"{os.path.basename(path)} {name[:80]}: {slots} slots: {mf} -> {instr}")
    assert not problems, "\n".join(problems[:20])
