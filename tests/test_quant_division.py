"""The quantizers' reciprocal path gives the IEEE division's codes (CPU only).

The activation and weight quantizers replace fl(x / s) by a reciprocal and
two fused corrections for rows with s >= 2^-96.  tests/native/
fast_division_check.c walks every (amax, x) pair of bf16 inputs with
|x| <= amax for Q = 127 and 448 and counts code mismatches; there must be
none at or above the threshold.  (The GPU parity tests then check the kernels
themselves bit-exactly against the oracle, including tiny-scale rows.)
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_reciprocal_division_gives_identical_codes_exhaustively(tmp_path):
    exe = str(tmp_path / "fast_division_check")
    src = os.path.join(HERE, "native", "fast_division_check.c")
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", src, "-o", exe, "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    lines = [l for l in r.stdout.splitlines() if l.startswith("Q=")]
    assert len(lines) == 2, r.stdout
    for l in lines:
        assert "code_mismatches_at_or_above_2^-96=0 " in l, r.stdout
    assert r.returncode == 0, r.stdout
