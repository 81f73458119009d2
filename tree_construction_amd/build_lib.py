"""Compile the HIP library (libkdt.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", "kdt.hip"), os.path.join(PKG, "csrc", "knn.hip")]
LIB_PATH = os.path.join(PKG, "libkdt.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-FP32 instruction selection anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False, out_path: str = LIB_PATH) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, "-I" + os.path.join(ROOT, "include"), "-o", tmp, *SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed (exit %d)" % r.returncode)
    if verbose:
        sys.stderr.write(r.stderr)
    os.replace(tmp, out_path)
    return out_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
