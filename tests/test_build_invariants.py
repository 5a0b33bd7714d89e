"""Invariants of the compiled gfx950 kernels, checked on the assembly that
hipcc emits for the kernel sources (no GPU needed).

* Matrix-core instructions write all 64 lanes of their destination registers
  whatever the exec mask, so they must never be issued while exec is partial
  (inside a lane-dependent branch): the compiler assumes masked lanes keep
  their register values and may reuse such registers.
* Every store and atomic is a vector-memory instruction: nothing writes
  through the scalar data cache."""
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


def mfma_under_partial_exec(asm: str):
    """(function, line) of each MFMA issued at a nonzero nesting depth of exec
    narrowing: s_and_saveexec and loop-exit s_andn2_b64 exec open a level,
    s_or_b64 exec closes one; else-switches keep the level."""
    found = []
    func, depth = None, 0
    for i, line in enumerate(asm.splitlines()):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            func, depth = m.group(1), 0
        s = line.strip()
        if s.startswith("s_and_saveexec_b64") or s.startswith("s_andn2_b64 exec"):
            depth += 1
        elif s.startswith("s_or_b64 exec, exec"):
            depth -= 1
        if s.startswith("v_mfma") and depth > 0:
            found.append((func, i + 1))
    return found


def test_checker_flags_a_masked_mfma():
    asm = "\n".join(["_Zfoo:", "s_and_saveexec_b64 s[6:7], vcc",
                     "v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0",
                     "s_or_b64 exec, exec, s[6:7]", "v_mfma_f32_16x16x32_f16 v[0:3], v[4:7], v[8:11], 0"])
    assert mfma_under_partial_exec(asm) == [("_Zfoo", 3)]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["tq_encode.hip", "tq_decode.hip"])
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
