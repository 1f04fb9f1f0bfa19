"""Host check of the division identity the quantize kernels use (CPU only).

The kernels replace the IEEE fp32 division x / s by r = RN(1/s); q0 = RN(x r);
e = fma(q0, s, -x); q = fma(-e, r, q0) (Markstein's theorem).  tests/csrc/division_identity.c
compares that sequence with x / s bit for bit, on the host with a correctly rounded fmaf, for every
finite BF16 x and for random FP32 x, over many scales drawn like the quantizer's; mismatches are
allowed only where both quotients are below 2^-60 with the same sign (they encode to the same signed
zero).  Built here with gcc; it shares no code with the kernels.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "csrc", "division_identity.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_division_identity(tmp_path):
    exe = str(tmp_path / "division_identity")
    subprocess.run(["gcc", "-O2", "-mfma", "-std=c11", "-o", exe, SRC, "-lm"], check=True)
    r = subprocess.run([exe, "2000", "3"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    checked = int(r.stdout.split()[1])
    assert checked > 50_000_000
    assert " mismatches 0 " in r.stdout
