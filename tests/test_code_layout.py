"""Instruction-line offsets of the backward's tile loops (no GPU).

Where a tile loop starts within the 64-byte lines the instructions are
fetched in changes the backward kernels' speed: an earlier dQ kernel ran 3 %
slower with its loop 44 bytes into a line than at 24 (identical loop code).
dkdv_kernel pads its prologue (UL_CODE_PAD) to reach its measured-good offset;
dq_kernel_1w has no pad and keeps the offset it was timed with (a sweep of its
eight 8-byte offsets put all of them within the run-to-run spread).  Any change to
a prologue moves the loop; this test compiles attn_bwd.hip for gfx950 with the
library's flags, disassembles the device code and checks that the loops still
start at those offsets, so such a change cannot slip in unnoticed.

The offsets are a performance guard, not a functional property: they hold for
the compiler they were measured with (MEASURED_WITH).  With another compiler
the test is skipped and reports the offsets it found instead of failing.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "ulysses_sequence_parallelism_ul_amd", "csrc", "attn_bwd.hip")
OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
WANT = {"dkdv_kernelILi128": 40, "dq_kernel_1wILi128": 32}
# `hipcc --version` of the toolchain the padding was measured with
MEASURED_WITH = "roc-7.2.0 26014 7b800a19466229b8479a78de19143dc33c3ab9b5"


def _loop_offsets(dis_lines):
    """Byte offset (mod 64) of the target of the longest backward branch in each kernel."""
    out = {}
    for kern in WANT:
        inside, best = False, None
        for ln in dis_lines:
            if re.match(r"^[0-9a-f]+ <", ln):
                inside = kern in ln
            if not inside:
                continue
            m = re.search(r"(s_cbranch\w*|s_branch)\s+(-?\d+)\s+//\s+([0-9A-F]+):", ln)
            if m:
                addr, simm = int(m.group(3), 16), int(m.group(2))
                if simm > 32767:
                    simm -= 65536
                tgt = addr + 4 + 4 * simm
                if tgt < addr and addr - tgt > 1000 and (best is None or tgt < best):
                    best = tgt
        out[kern] = None if best is None else best % 64
    return out


def test_backward_tile_loops_start_at_their_padded_offsets(tmp_path):
    from ulysses_sequence_parallelism_ul_amd import build as B

    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if not os.path.exists(OBJDUMP) and shutil.which("llvm-objdump") is None:
        pytest.skip("llvm-objdump not available")
    objdump = OBJDUMP if os.path.exists(OBJDUMP) else shutil.which("llvm-objdump")
    version = subprocess.run([hipcc, "--version"], capture_output=True, text=True).stdout
    obj = str(tmp_path / "attn_bwd_device.o")
    flags = [f for f in B.HIPCC_FLAGS if f != "-fPIC"]
    r = subprocess.run([hipcc] + flags + ["--cuda-device-only", "--no-gpu-bundle-output", "-c", SRC, "-o", obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    dis = subprocess.run([objdump, "-d", obj], capture_output=True, text=True, check=True).stdout.splitlines()
    got = _loop_offsets(dis)
    if MEASURED_WITH not in version:
        pytest.skip(f"padding measured with {MEASURED_WITH}; this compiler places the loops at {got} (want {WANT})")
    assert got == WANT
