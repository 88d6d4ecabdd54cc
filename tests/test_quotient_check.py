"""The quantizer's element division (|x| / d with one rounding, x's sign
kept) is taken as q = x r, then q - (q d - x) r with two fmas, r = 1/d once
per block.  tests/quotient_check.c compares that, for x and -x, with the
correctly rounded division on the host; here it runs on every bf16
significand against every 61st fp32 significand (the full 2^30-pair run
takes about 20 s: QUOTIENT_CHECK_STEP=1)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_quotient_shortcut_matches_division(tmp_path):
    exe = str(tmp_path / "quotient_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, os.path.join(HERE, "quotient_check.c"), "-lm"],
                   check=True)
    step = os.environ.get("QUOTIENT_CHECK_STEP", "61")
    p = subprocess.run([exe, step], capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, p.stdout
    checked, bad = (int(t) for t in p.stdout.split()[1::2][-2:])
    assert bad == 0 and checked == 128 * len(range(0, 1 << 23, int(step)))
