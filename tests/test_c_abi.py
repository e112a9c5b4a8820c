"""The library driven from a plain C program (tests/c/moe_c_abi.c) through include/moe.h, with
the HIP runtime API for memory and streams and no Python or torch in the process: host-only
checks on the CPU, the decode and prefill paths against the C oracle on the GPU."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "c"))
EXE = os.path.join(HERE, "c", "moe_c_abi")


def test_c_program_builds_and_host_checks_pass():
    import build_c_abi
    import oracle
    oracle.build()
    build_c_abi.build()
    p = subprocess.run([EXE, "--host"], capture_output=True, text=True, timeout=60)
    assert p.returncode == 0 and p.stdout.strip().endswith("ok"), p.stdout + p.stderr


@pytest.mark.gpu
def test_c_program_on_gpu():
    print("\ncase C program: decode and prefill paths", flush=True)
    assert os.path.exists(EXE), "tests/c/moe_c_abi is not built (run __graft_entry__.build())"
    p = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(p.stdout, p.stderr, flush=True)
    assert p.returncode == 0 and p.stdout.strip().endswith("ok")
