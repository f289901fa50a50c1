"""The quantizers' reciprocal-and-correction quotient against IEEE division.

The row quantizer and the tgmm operand quantization compute x / s as
q0 = x*r, e' = fma(q0, s, -x), fma(-e', r, q0) with r = 1/s, which costs
three operations where an IEEE f32 division costs about ten.  Their
codes stay bit-exact only if that quotient equals the IEEE one wherever an
8-bit code can tell them apart.  This test runs the check over every input
pair the quantizers can see (bf16 x, |x| <= amax, s = f32(max(amax, 1e-12) /
FMAX) for both FMAX), compiled with gcc: about 2 * 10^9 pairs, a few seconds
on 8 cores."""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_div_by_scale_exhaustive(tmp_path):
    exe = tmp_path / "div_by_scale_check"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    os.path.join(HERE, "div_by_scale_check.c"), "-o", str(exe), "-lm"], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=600).stdout
    rows = re.findall(r"FMAX (\S+) pairs (\d+) differ (\d+) differ_coded (\d+) differ_old (\d+)", out)
    assert len(rows) == 2, out
    for fm, pairs, differ, coded, old in rows:
        print(f"FMAX {fm}: {int(pairs)} pairs, {int(differ)} differ below half the smallest code, {int(coded)} above, "
              f"{int(old)} differ from the copysign form")
        assert int(pairs) > 10 ** 9 and int(coded) == 0 and int(old) == 0, out
