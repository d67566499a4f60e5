"""The quantizers divide by a constant (the code ranges 3, 15, 127 and 255, the
Oaken magnitude range 31) without a division instruction: q0 = fl(x c), c = fl(1/D), then
one step corrected by the exact fused-multiply-add residual.  This checks,
on the CPU, that the sequence gives the IEEE quotient fl(x / D) for every
non-negative binary32 x of the binades `tests/constdiv/const_division.c`
lists (all subnormals and the binades where the residual can be subnormal;
every other binade is a scaled copy).  (The FP8 divisors 448 and 57344 fail
this check in some binades, so the FP8 scales keep the division.)  Infinite
and NaN x are not claimed:
the kernels pass those through unchanged, as the division would.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "constdiv")


@pytest.mark.timeout(300)
def test_constant_division_is_correctly_rounded(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "const_division")
    src = os.path.join(HERE, "const_division.c")
    base = [cc, "-O2", "-ffp-contract=off", "-o", exe, src, "-lm"]
    if subprocess.run(base + ["-fopenmp"], capture_output=True).returncode != 0:
        subprocess.run(base, check=True)  # one thread
    r = subprocess.run([exe, "3", "15", "31", "127", "255"], capture_output=True, text=True)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count(" 0 mismatches") == 5
