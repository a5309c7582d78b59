"""Arithmetic the writer's quantizer relies on, checked on the CPU with the
same IEEE fp32 operations the GPU performs.

The scale of a group is span / levels (levels 3 or 15), correctly rounded
(RAQ-MLA appendix Table 5: FP16 scale per group).  The writer forms it as a
product with rn(1 / levels) and one fused correction; this holds for every
fp32 span from 0 to 2^20 (run with QUOTIENT_CHECK_ALL=1 for all 1.2e9
spans of each divisor, about a minute; by default every 29th bit pattern)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_scale_quotient_by_fused_correction(tmp_path):
    exe = tmp_path / "quotient_check"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe), os.path.join(HERE, "quotient_check.c"), "-lm"],
                   check=True)
    stride = "1" if os.environ.get("QUOTIENT_CHECK_ALL") else "29"
    bad, n = map(int, subprocess.run([str(exe), stride], check=True, capture_output=True, text=True).stdout.split())
    assert n > 2 * (0x49800000 // int(stride))
    assert bad == 0, f"{bad} of {n} spans differ from the IEEE quotient"
