"""Build the HIP library libmoe.so for gfx950, in place."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-fvisibility=hidden",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out_tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), *sources(), "-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libmoe.so")
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
