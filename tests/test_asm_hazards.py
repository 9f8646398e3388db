"""Wait states around the inline-asm MFMAs of dq_kernel_1w (no GPU).

dq_kernel_1w issues its MFMAs as inline assembly so that its operands and
accumulators stay in AGPRs.  The compiler then does not know that these
instructions are MFMAs, so it neither inserts the wait states the hardware
requires around them nor avoids reusing their registers too early: the
kernel places the fences and register keep-alives itself.  A compiler
change, or an edit of the kernel, can undo that without any error.  This
test compiles attn_bwd.hip for gfx950 with the library's flags and scans the
kernel's machine code, following branches, for the two hazards that matter
(CDNA3/CDNA4 instruction set reference, section on dependency wait states
for MFMA):

  * a VALU instruction writes a register that an MFMA reads (A, B or C) with
    fewer than VALU_TO_MFMA wait states between them;
  * an instruction other than the next MFMA of the same accumulation chain
    reads or overwrites an MFMA's result with fewer than MFMA_TO_READ wait
    states after the MFMA (an 8-pass 32x32x16 MFMA needs 11; the margin is
    deliberate).

Both scans are checked on planted cases first, so that a scanner that finds
nothing because it is broken fails too.
"""

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "ulysses_sequence_parallelism_ul_amd", "csrc", "attn_bwd.hip")
KERNEL = "dq_kernel_1wILi128"
VALU_TO_MFMA = 3
MFMA_TO_READ = 20


def _regs(tok):
    """Vector / accumulator registers named by one operand token."""
    out = set()
    for f, lo, hi in re.findall(r"(?<!\w)([va])\[(\d+):(\d+)\]", tok):
        out |= {(f, r) for r in range(int(lo), int(hi) + 1)}
    for f, r in re.findall(r"(?<!\w)([va])(\d+)(?![\w\[])", tok):
        out.add((f, int(r)))
    return out


class Code:
    """One function's instructions with their control-flow edges."""

    def __init__(self, lines):
        self.ins, self.ops, label_at = [], [], {}
        pending = []
        for raw in lines:
            ln = raw.split(";")[0].strip()
            if not ln:
                continue
            if ln.endswith(":"):
                pending.append(ln[:-1])
                continue
            if ln.startswith("."):
                continue
            for lab in pending:
                label_at[lab] = len(self.ins)
            pending = []
            op, _, rest = ln.partition(" ")
            self.ins.append(op)
            self.ops.append([t.strip() for t in rest.split(",")] if rest.strip() else [])
        n = len(self.ins)
        self.succ = [[] for _ in range(n)]
        for i, op in enumerate(self.ins):
            if op.startswith("s_cbranch") or op == "s_branch":
                tgt = label_at.get(self.ops[i][0]) if self.ops[i] else None
                if tgt is not None:
                    self.succ[i].append(tgt)
                if op == "s_branch":
                    continue
            if op == "s_endpgm":
                continue
            if i + 1 < n:
                self.succ[i].append(i + 1)
        self.pred = [[] for _ in range(n)]
        for i, ss in enumerate(self.succ):
            for j in ss:
                self.pred[j].append(i)

    def wait_states(self, i):
        if self.ins[i] == "s_nop":
            return int(self.ops[i][0], 0) + 1
        return 1

    def is_mfma(self, i):
        return self.ins[i].startswith("v_mfma")


def valu_to_mfma_hazards(code, need=VALU_TO_MFMA):
    """(writer, mfma) index pairs: a VALU write of an MFMA source with fewer than `need` wait states between."""
    bad = []
    for i in range(len(code.ins)):
        if not code.is_mfma(i):
            continue
        srcs = set().union(*(_regs(t) for t in code.ops[i][1:4]))
        stack, seen = [(p, 0) for p in code.pred[i]], set()
        while stack:
            j, ws = stack.pop()
            if (j, ws) in seen or ws >= need:
                continue
            seen.add((j, ws))
            op = code.ins[j]
            if op.startswith("v_") and not code.is_mfma(j) and code.ops[j] and _regs(code.ops[j][0]) & srcs:
                bad.append((j, i))
            stack.extend((p, ws + code.wait_states(j)) for p in code.pred[j])
    return bad


def mfma_result_hazards(code, need=MFMA_TO_READ):
    """(mfma, reader) index pairs: a read or overwrite of an MFMA's result within `need` wait states, other
    than the next MFMA of the same accumulation chain (SrcC equal to the destination)."""
    bad = []
    for i in range(len(code.ins)):
        if not code.is_mfma(i):
            continue
        dst = _regs(code.ops[i][0])
        stack, seen = [(s, 0) for s in code.succ[i]], set()
        while stack:
            j, ws = stack.pop()
            if (j, ws) in seen or ws >= need:
                continue
            seen.add((j, ws))
            op = code.ins[j]
            if code.is_mfma(j):
                o = code.ops[j]
                if (_regs(o[1]) | _regs(o[2])) & dst or (_regs(o[3]) & dst and _regs(o[3]) != dst):
                    bad.append((i, j))
            elif not op.startswith("s_") and set().union(*(_regs(t) for t in code.ops[j])) & dst:
                bad.append((i, j))
            stack.extend((s, ws + code.wait_states(j)) for s in code.succ[j])
    return bad


def _code(text):
    return Code(text.strip().splitlines())


MFMA = "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], v[0:15]"


def test_scanners_find_planted_hazards():
    # a VALU write of the accumulator right before the MFMA; enough wait states clear it
    assert valu_to_mfma_hazards(_code(f"v_mov_b32 v3, 0\n{MFMA}")) == [(0, 1)]
    assert valu_to_mfma_hazards(_code(f"v_mov_b32 v17, 0\ns_nop 0\n{MFMA}")) == [(0, 2)]
    assert valu_to_mfma_hazards(_code(f"v_mov_b32 v17, 0\ns_nop 2\n{MFMA}")) == []
    assert valu_to_mfma_hazards(_code(f"v_accvgpr_write_b32 a2, v40\n{MFMA}")) == [(0, 1)]
    assert valu_to_mfma_hazards(_code(f"v_mov_b32 v20, 0\n{MFMA}")) == []  # not an operand
    # across a loop's back edge: the write at the end of the body, the MFMA at its top
    loop = f".LBB0_1:\n{MFMA}\ns_nop 7\ns_nop 7\ns_nop 7\nv_mov_b32 v18, 1\ns_cbranch_scc1 .LBB0_1\ns_endpgm"
    assert valu_to_mfma_hazards(_code(loop)) == [(4, 0)]
    # a read of the result too early, also behind a branch; the accumulation chain is allowed
    assert mfma_result_hazards(_code(f"{MFMA}\ns_nop 7\nv_add_f32 v40, v5, v41")) == [(0, 2)]
    assert mfma_result_hazards(_code(f"{MFMA}\ns_nop 7\ns_nop 7\ns_nop 7\nv_add_f32 v40, v5, v41")) == []
    assert mfma_result_hazards(_code(f"{MFMA}\n{MFMA}")) == []
    assert mfma_result_hazards(_code(f"{MFMA}\nv_mfma_f32_32x32x16_bf16 v[20:35], v[0:3], a[0:3], 0")) == [(0, 1)]
    assert mfma_result_hazards(_code(f"{MFMA}\ns_branch .LBB0_2\nv_mov_b32 v1, 0\n.LBB0_2:\n"
                                     f"global_store_dwordx4 v[40:41], v[4:7], off")) == [(0, 3)]


def test_dq_kernel_1w_mfma_wait_states(tmp_path):
    from ulysses_sequence_parallelism_ul_amd import build as B

    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    asm = str(tmp_path / "attn_bwd.s")
    flags = [f for f in B.HIPCC_FLAGS if f != "-fPIC"]
    r = subprocess.run([hipcc] + flags + ["--cuda-device-only", "--no-gpu-bundle-output", "-S", SRC, "-o", asm],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = open(asm).read().splitlines()
    start = [i for i, ln in enumerate(lines) if re.match(r"^_Z\S*" + KERNEL + r"\S*:", ln)]
    assert len(start) == 1, f"{KERNEL} not found in the device code"
    end = next(i for i in range(start[0], len(lines)) if lines[i].startswith(".Lfunc_end"))
    code = Code(lines[start[0] + 1:end])
    n_mfma = sum(code.is_mfma(i) for i in range(len(code.ins)))
    assert n_mfma >= 96, n_mfma  # the key loop's MFMAs of one tile at least
    show = lambda pairs: [(code.ins[a], code.ops[a], code.ins[b], code.ops[b]) for a, b in pairs[:5]]
    vw = valu_to_mfma_hazards(code)
    assert vw == [], show(vw)
    rr = mfma_result_hazards(code)
    assert rr == [], show(rr)
