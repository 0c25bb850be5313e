"""Builds libfp8mot.so (the HIP kernels and the C ABI) in-tree for gfx950.

Compiler flags:
  --offload-arch=gfx950          the only target (no other architecture);
  -ffp-contract=off              arithmetic as written: no implicit FMA, so
                                 the observer update and the epilogue round
                                 exactly where the code says;
  -target-feature -packed-fp32-ops
                                 no packed FP32 instructions are generated;
  no fast-math                   FP32 division stays correctly rounded.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libfp8mot.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["elementwise.hip", "gemm.hip", "mfma_ceiling.hip", "verify.hip", "capi.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("command failed: " + " ".join(cmd))
    return r


def build(verbose=False, jobs=4) -> str:
    """Compile every source and link libfp8mot.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def device_assembly(src) -> str:
    """gfx950 assembly text of one source (for inspection by tests)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    out = os.path.join(BUILD_DIR, src.replace(".hip", ".gfx950.s"))
    _run([HIPCC, *FLAGS, "--cuda-device-only", "-S",
          os.path.join(CSRC, src), "-o", out])
    with open(out) as f:
        return f.read()


if __name__ == "__main__":
    print(build(verbose=True))
