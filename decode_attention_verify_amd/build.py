"""Build librattn.so (HIP kernels for gfx950 + the C-ABI host library) in-tree.

Usage: ``python -m decode_attention_verify_amd.build`` or ``build()`` from Python.
The library lands next to this file; ``binding`` loads it from there.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "librattn.so")
BUILD_DIR = os.path.join(HERE, "_build")

ARCH = "gfx950"
# packed fp32 VALU ops stay off for the device code; hipcc's host pass warns that it
# does not know the feature, which is harmless
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-I", INCLUDE]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: cannot build librattn.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("build step failed (%d):\n%s\n%s" % (res.returncode, " ".join(cmd), out))
    if verbose and out.strip():
        print(out)


def build(verbose=False, save_temps=False):
    """Compile every source under csrc/ for gfx950 and link librattn.so. Always rebuilds."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for name in ("kernels.hip", "scratch.hip", "api.cpp", "planner.cpp"):
        src = os.path.join(CSRC, name)
        obj = os.path.join(BUILD_DIR, name + ".o")
        cmd = [hipcc, "--offload-arch=" + ARCH] + COMMON + DEVICE_FLAGS
        if name.endswith(".hip"):
            cmd += ["-x", "hip"]
            if save_temps:
                cmd += ["-save-temps=obj"]
        cmd += ["-c", src, "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, save_temps="--save-temps" in sys.argv)
    print("built", LIB)
