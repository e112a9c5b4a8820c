"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/c/oracle_sanitize.c drives every oracle function through small seeded shapes (bf16 and
e4m3 payloads, per-rank token counts, both combine modes, the send-side sum, the prefill path)
with every buffer allocated at exactly its contract size; it is built with gcc and both
sanitizers, with recovery off, so an out-of-bounds access, a use of freed memory, a leak, a
signed overflow or a bad shift ends the run with a report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not available")
    exe = os.path.join(str(tmp_path), "oracle_sanitize")
    build = ["gcc", "-O1", "-g", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
             "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "tests", "c", "oracle_sanitize.c"),
             "-lm", "-o", exe]
    r = subprocess.run(build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-1000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
    assert "cases passed" in r.stdout
