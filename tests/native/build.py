"""Build the native program of tests/native: abi_step, a C++ consumer of
libdopt.so (host code only: it calls the C ABI with hipMalloc'd buffers, no
Python)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "abi_step")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, what: str, verbose: bool):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed building {what}")


def build(verbose: bool = False) -> str:
    common = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    _run(common + ["-I", os.path.join(ROOT, "include"), os.path.join(HERE, "abi_step.cpp"),
                   "-L", os.path.join(ROOT, "sharded_mixed_precision_amd"), "-ldopt",
                   "-Wl,-rpath,$ORIGIN/../../sharded_mixed_precision_amd", "-o", EXE + ".tmp"],
         "tests/native/abi_step", verbose)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
