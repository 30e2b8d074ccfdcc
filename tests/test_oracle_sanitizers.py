"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/sanitize_check.c calls every function of oracle/tq_oracle.c on small
inputs in exactly sized heap buffers (packing at odd counts, the transform at
2 ... 16384 points, TQ3 with zero and overflowing vectors, OrbitQuant at
d = 32 ... 12288 with a zero row, both bit orders, rotated and full
dequantization). Built here with gcc -fsanitize=address,undefined and
-fno-sanitize-recover, any out-of-bounds access, leak or undefined operation
fails the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize_check")
    src = [os.path.join(ROOT, "oracle", "sanitize_check.c"), os.path.join(ROOT, "oracle", "tq_oracle.c")]
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp",
           *src, "-o", exe, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "ok" in run.stdout
