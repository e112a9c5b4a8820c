"""Build tests/c/moe_c_abi (a plain C program driving libmoe.so through include/moe.h and
checking it against the C oracle).  Test infrastructure: links liboracle.so."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "moe_c_abi.c")
EXE = os.path.join(HERE, "moe_c_abi")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    """Compile with gcc against the built libmoe.so and liboracle.so (always recompiles)."""
    pkg = os.path.join(ROOT, "combine_moe_route_top_amd")
    orc = os.path.join(ROOT, "oracle")
    tmp = EXE + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           SRC, "-o", tmp, "-L", pkg, "-lmoe", "-L", orc, "-loracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../combine_moe_route_top_amd:$ORIGIN/../../oracle:" +
           os.path.join(ROCM, "lib")]
    subprocess.check_call(cmd)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build())
