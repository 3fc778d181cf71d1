"""The C ABI from a plain C program (host only): compile tests/c/abi_host_check.c with gcc
against include/rattn.h, link librattn.so, run it."""

import os
import shutil
import subprocess

import pytest

from decode_attention_verify_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_c_program_uses_the_abi(tmp_path):
    binding.load()                                  # the library is built
    lib_dir = os.path.dirname(binding.LIB_PATH)
    exe = str(tmp_path / "abi_host_check")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host_check.c"), "-o", exe,
                    "-L", lib_dir, "-lrattn", "-Wl,-rpath," + lib_dir],
                   check=True, capture_output=True, text=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "FAIL" not in res.stdout
