"""The codec kernels divide by a shared divisor with its correctly rounded
reciprocal and one correction step from the exact remainder (three fp32
operations). This checks, on the host with the same IEEE fp32 operations,
that the sequence rounds exactly like IEEE division for every numerator of 8
(bf16) and 11 (fp16) significant bits and every divisor mantissa, and that
the check sees the errors of the uncorrected product. (The device check in
test_gpu_arith_checks.py covers every fp32 numerator.)"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("div") / "division_check")
    subprocess.run([cc, "-O2", "-std=c99", "-mfma", "-ffp-contract=off", "-fno-fast-math",
                    "-fopenmp", os.path.join(HERE, "division_check.c"), "-o", exe, "-lm"],
                   check=True)
    return exe


@pytest.mark.parametrize("bits", [8, 11])
def test_short_numerator_division_is_correctly_rounded(checker, bits):
    r = subprocess.run([checker, str(bits)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 of " in r.stdout


def test_uncorrected_product_is_caught(checker):
    r = subprocess.run([checker, "8", "uncorrected"], capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 1, r.stdout + r.stderr
    assert " 0 of " not in r.stdout
