"""The fast activation encoder replaces its two correctly rounded divisions
(t = bmax / 6 and g_enc / s_dec) by a reciprocal multiply plus one fused
multiply-add correction.  This builds and runs an exhaustive host check of
that identity (tests/exact_division_check.c) with the system C compiler; the
GPU parity tests then confirm the encoder bit for bit against the oracle."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_markstein_division_is_exact(tmp_path):
    exe = tmp_path / "exact_division_check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", os.path.join(HERE, "exact_division_check.c"),
                    "-o", str(exe), "-lm"], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "mismatches 0\n" in res.stdout
