"""The host library (validation, planner, plan description, the entry points' host-side
checks) under the address and undefined-behaviour sanitizers: planner.cpp and api.cpp
are compiled with g++ together with tests/c/sanitize_host.cpp, which sweeps seeded
valid and invalid problems, and tests/c/kernel_stubs.cpp, which stands in for the
device launchers. Runs on the CPU; no GPU is touched."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None or
                    not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")),
                    reason="g++ or the HIP runtime library is not installed")
def test_host_library_under_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitize_host")
    csrc = os.path.join(ROOT, "decode_attention_verify_amd", "csrc")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "sanitize_host.cpp"),
           os.path.join(ROOT, "tests", "c", "kernel_stubs.cpp"),
           os.path.join(csrc, "planner.cpp"), os.path.join(csrc, "api.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert res.stdout.strip().splitlines()[-1].startswith("ok"), res.stdout[-2000:]
