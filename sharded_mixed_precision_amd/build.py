"""Build libdopt.so (host mapper + gfx950 kernels) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SO = os.path.join(HERE, "libdopt.so")
SOURCES = [os.path.join(HERE, "csrc", "mapper.cpp"), os.path.join(HERE, "csrc", "step.hip"),
           os.path.join(HERE, "csrc", "vmm.cpp")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # IEEE fp32 step: no contraction into FMA, correctly rounded sqrt and
    # division, denormals kept.
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # no packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", os.path.join(HERE, "csrc"),
]


def build(verbose: bool = False) -> str:
    tmp = SO + ".tmp"
    cmd = [HIPCC, *FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libdopt.so")
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
