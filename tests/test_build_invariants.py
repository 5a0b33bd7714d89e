"""Invariants of the compiled gfx950 kernels, checked on the assembly that
hipcc emits for the kernel sources (no GPU needed).

* Matrix-core instructions write all 64 lanes of their destination registers
  whatever the exec mask, so they must never be issued while exec is partial
  (inside a lane-dependent branch): the compiler assumes masked lanes keep
  their register values and may reuse such registers.
* Every store and atomic is a vector-memory instruction: nothing writes
  through the scalar data cache.
* Inline assembly carries no instructions (only empty register pins): the
  compiler inserts the wait states between dependent instructions (e.g. a
  compare writing a lane mask and a writelane reading it) only for code it
  emits itself."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_tq_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
         "-Xclang", "-packed-fp32-ops", "--offload-device-only", "-S"]


def _functions(asm: str):
    """(name, lines) of each kernel in the assembly text."""
    funcs, name, body = [], None, []
    for i, line in enumerate(asm.splitlines()):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            if name:
                funcs.append((name, body))
            name, body = m.group(1), []
        elif name:
            body.append((i + 1, line.strip()))
            if line.strip().startswith("s_endpgm"):
                funcs.append((name, body))
                name, body = None, []
    return funcs


def _exec_step(stack: tuple, ins: str) -> tuple:
    """Stack of (register, narrows) entries: the saved masks a later restore
    can return to, and whether exec was narrowed when each was pushed.  An
    if's s_and_saveexec pushes its save register (narrowing), a plain copy of
    exec (s_mov_b64 X, exec) pushes X (not narrowing), a loop's lane exit
    (s_andn2_b64 exec, exec, X) pushes X once, and restoring a saved mask
    (s_or_b64 exec, exec, X) pops X and everything above it.  An if/else
    moves its saved mask to the register that restores it
    (s_xor_b64 Y, exec, X renames X to Y).  Else-switches keep the stack;
    any other write of exec is a narrowing with no known restore register."""
    regs = [r for r, _ in stack]
    # if/else: the saved mask moves to another register, which then restores
    m = re.match(r"s_xor_b64 (s\[\d+:\d+\]), exec, (s\[\d+:\d+\])$", ins)
    if m and m.group(2) in regs:
        i = len(regs) - 1 - regs[::-1].index(m.group(2))
        return stack[:i] + ((m.group(1), stack[i][1]),) + stack[i + 1:]
    m = re.match(r"s_and_saveexec_b64 (\S+),", ins)
    if m:
        return stack + ((m.group(1), True),)
    m = re.match(r"s_mov_b64 (s\[\d+:\d+\]), exec$", ins)
    if m:
        return stack + ((m.group(1), False),)
    m = re.match(r"s_andn2_b64 exec, exec, (\S+)", ins)
    if m:
        return stack if m.group(1) in regs else stack + ((m.group(1), True),)
    m = re.match(r"s_or_b64 exec, exec, (\S+)", ins)
    if m:
        r = m.group(1)
        return stack[:len(regs) - 1 - regs[::-1].index(r)] if r in regs else stack
    if re.match(r"s_(andn2|or|xor)_saveexec_b64 ", ins) or re.match(r"s_xor_b64 exec, exec,", ins):
        return stack
    if re.match(r"s_\w+ exec(_lo|_hi)?,", ins):
        return stack + (("?", True),)
    return stack


def _narrowed(stack: tuple) -> bool:
    return any(n for _, n in stack)


def mfma_under_partial_exec(asm: str, max_states: int = 64):
    """(function, line) of each MFMA that some path reaches with exec
    narrowed.  Basic blocks and their edges (fall-through, s_branch,
    s_cbranch_*) form the control-flow graph; each block keeps the set of
    narrowing stacks it can be entered with, iterated to a fixpoint, so a
    block reached both by a loop's back edge (after lanes left) and from
    outside counts as narrowed."""
    found = []
    for fname, body in _functions(asm):
        blocks, labels, cur = [], {}, []
        for ln, ins in body:
            if not ins or ins.startswith(";") or ins.startswith("."):
                m = re.match(r"^(\.LBB\S+):", ins)
                if m:
                    if cur:
                        blocks.append(cur)
                    cur = []
                    labels[m.group(1)] = len(blocks)
                continue
            cur.append((ln, ins))
            if ins.startswith("s_branch") or ins.startswith("s_cbranch") or ins.startswith("s_endpgm"):
                blocks.append(cur)
                cur = []
        if cur:
            blocks.append(cur)
        if not blocks:
            continue
        succ = []
        for bi, blk in enumerate(blocks):
            last = blk[-1][1]
            out = []
            m = re.match(r"s_c?branch\S*\s+(\.LBB\S+)", last)
            if m and m.group(1) in labels:
                out.append(labels[m.group(1)])
            if not (last.startswith("s_branch") or last.startswith("s_endpgm")) and bi + 1 < len(blocks):
                out.append(bi + 1)
            succ.append(out)
        entry = [set() for _ in blocks]
        entry[0].add(())
        work = [(0, ())]
        while work:
            bi, st = work.pop()
            for _, ins in blocks[bi]:
                st = _exec_step(st, ins)
            for t in succ[bi]:
                if st not in entry[t]:
                    assert len(entry[t]) < max_states, f"{fname}: too many exec states"
                    entry[t].add(st)
                    work.append((t, st))
        for bi, blk in enumerate(blocks):
            for st0 in entry[bi]:
                st = st0
                for ln, ins in blk:
                    st = _exec_step(st, ins)
                    if ins.startswith("v_mfma") and _narrowed(st) and (fname, ln) not in found:
                        found.append((fname, ln))
    return found


def inline_asm_instructions(asm: str):
    """Non-comment lines between ;;#ASMSTART and ;;#ASMEND."""
    found, inside = [], False
    for line in asm.splitlines():
        s = line.strip()
        if s == ";;#ASMSTART":
            inside = True
        elif s == ";;#ASMEND":
            inside = False
        elif inside and s and not s.startswith(";"):
            found.append(s)
    return found


def test_checker_flags_inline_instructions():
    asm = "\n".join([";;#ASMSTART", ";;#ASMEND", "v_cmp_le_f32_e32 vcc, 0, v84",
                     ";;#ASMSTART", "v_writelane_b32 v0, vcc_lo, 0", ";;#ASMEND"])
    assert inline_asm_instructions(asm) == ["v_writelane_b32 v0, vcc_lo, 0"]


def test_checker_flags_a_masked_mfma():
    asm = "\n".join(["_Zfoo:", "s_and_saveexec_b64 s[6:7], vcc",
                     "v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0",
                     "s_or_b64 exec, exec, s[6:7]", "v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0",
                     "s_endpgm"])
    assert mfma_under_partial_exec(asm) == [("_Zfoo", 3)]


def test_checker_follows_out_of_order_blocks():
    # an if whose restore sits textually before its saveexec (reached by a
    # branch back): the matrix op after the uniform branch runs at full exec
    asm = "\n".join([
        "_Zbar:",
        "s_cbranch_scc0 .LBB0_2",
        ".LBB0_1:",
        "s_or_b64 exec, exec, s[2:3]",
        "s_branch .LBB0_3",
        ".LBB0_2:",
        "s_and_saveexec_b64 s[2:3], vcc",
        "s_cbranch_execnz .LBB0_4",
        "s_branch .LBB0_1",
        ".LBB0_4:",
        "v_add_f32_e32 v0, v1, v2",
        "s_branch .LBB0_1",
        ".LBB0_3:",
        "v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0",
        "s_endpgm"])
    assert mfma_under_partial_exec(asm) == []
    # the same matrix op placed inside the guarded block is flagged
    masked = asm.replace("v_add_f32_e32 v0, v1, v2", "v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0")
    assert [ln for _, ln in mfma_under_partial_exec(masked)] == [11]


def test_checker_flags_a_loop_with_lane_exits():
    asm = "\n".join([
        "_Zloop:",
        "s_mov_b64 s[0:1], 0",
        ".LBB0_1:",
        "v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0",
        "s_andn2_b64 exec, exec, s[0:1]",
        "s_cbranch_execnz .LBB0_1",
        "s_or_b64 exec, exec, s[0:1]",
        "v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0",
        "s_endpgm"])
    assert [ln for _, ln in mfma_under_partial_exec(asm)] == [4]


def test_checker_follows_copied_exec_saves():
    asm = "\n".join([
        "_Zmov:",
        "s_mov_b64 s[74:75], exec",
        "s_and_b64 s[0:1], s[74:75], s[10:11]",
        "s_mov_b64 exec, s[0:1]",
        "s_cbranch_execz .LBB0_1",
        "v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0",
        ".LBB0_1:",
        "s_or_b64 exec, exec, s[74:75]",
        "v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0",
        "s_endpgm"])
    assert [ln for _, ln in mfma_under_partial_exec(asm)] == [6]


def test_checker_follows_if_else_mask_moves():
    # outer if/else saved in s[28:29], moved to s[14:15]; s[28:29] is reused by
    # an inner if; the outer restore goes through s[14:15], inside a loop
    asm = "\n".join([
        "_Zife:",
        ".LBB0_1:",
        "s_and_saveexec_b64 s[28:29], s[14:15]",
        "s_xor_b64 s[14:15], exec, s[28:29]",
        "s_cbranch_execz .LBB0_2",
        "s_and_saveexec_b64 s[28:29], vcc",
        "v_add_f32_e32 v0, v1, v2",
        "s_or_b64 exec, exec, s[28:29]",
        ".LBB0_2:",
        "s_andn2_saveexec_b64 s[14:15], s[14:15]",
        "s_or_b64 exec, exec, s[14:15]",
        "v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0",
        "s_cbranch_scc1 .LBB0_1",
        "s_endpgm"])
    assert mfma_under_partial_exec(asm) == []


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["tq_encode.hip", "tq_decode.hip", "tq_prefill.hip"])
def test_no_matrix_op_under_partial_exec(src, tmp_path):
    out = tmp_path / (src + ".s")
    r = subprocess.run([HIPCC, *FLAGS, os.path.join(CSRC, src), "-o", str(out)],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    assert "v_mfma" in asm
    assert mfma_under_partial_exec(asm) == []
    # all stores and atomics go through the vector memory path
    scalar_writes = [l.strip() for l in asm.splitlines()
                     if re.match(r"\s*s_(store|atomic|buffer_store|buffer_atomic|dcache_wb|dcache_discard)", l)]
    assert scalar_writes == []
    assert inline_asm_instructions(asm) == []
