"""The quantisers form the correctly rounded quotient x / s from a per-block
reciprocal (Markstein's FMA correction) and the scale amax / 448 as
(amax / 7) * 2^-6; scales outside [2^-80, 2^100] are first brought into
that range by an exact power of two applied to x and s alike. These are
IEEE 754 facts, independent of the GPU: this test compiles
tests/native/division_identities.c with the host C compiler and runs it
exhaustively (every amax >= 2^-100; every x in the e4m3-relevant quotient
range for 12 ordinary and 16 extreme scales, subnormal ones down to 2^-149
and the largest a finite amax gives). The GPU side is checked against the
oracle by test_gpu_quantize.py."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a host C compiler")
def test_division_identities_exhaustive(tmp_path):
    exe = tmp_path / "division_identities"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", str(exe),
                    os.path.join(HERE, "native", "division_identities.c"), "-lm"], check=True)
    res = subprocess.run([str(exe), "4"], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "total mismatches 0" in res.stdout
