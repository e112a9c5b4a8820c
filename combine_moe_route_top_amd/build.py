"""Build libmoe.so (the HIP kernels + C ABI) in-tree with hipcc for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmoe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 arithmetic off: plain v_fma_f32 / v_add_f32 only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every csrc/*.hip into libmoe.so (always recompiles).  `defines` (NAME=VALUE)
    override launch-shape constants for an alternative build written to `out`."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *["-D" + d for d in defines], "-I", os.path.join(ROOT, "include"),
           *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import sys
    args = sys.argv[1:]
    out = LIB
    if args and args[0].endswith(".so"):
        out, args = args[0], args[1:]
    print(build(verbose=True, out=out, defines=args))
