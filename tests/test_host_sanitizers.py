"""The host half of the library (tq_host.cpp: codebooks, projection, plans,
argument checks) built alone with AddressSanitizer and
UndefinedBehaviorSanitizer and driven through its C ABI on the CPU
(tests/sanitize/host_driver.cpp); the device entry points are stubs that
abort if reached."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not os.path.exists(CLANG), reason="clang++ of the ROCm toolchain not found")
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = tmp_path / "host_driver"
    src = [os.path.join(ROOT, "decode_attention_tq_amd", "csrc", "tq_host.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp")]
    # host-only C++ (no device code): the sanitizers instrument the CPU code
    cmd = [CLANG, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "decode_attention_tq_amd", "csrc"),
           "-I", "/opt/rocm/include", *src, "-o", str(exe), "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "host driver ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
