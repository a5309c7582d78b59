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


def _f16_directed(x, up):
    """Nearest fp16 at or above (up) / at or below x, as float32 (finite x,
    |x| <= 65504)."""
    import numpy as np
    h = x.astype(np.float16)
    hf = h.astype(np.float32)
    if up:
        fix = hf < x
        h = np.where(fix, np.nextafter(h, np.float16(np.inf)), h)
    else:
        fix = hf > x
        h = np.where(fix, np.nextafter(h, np.float16(-np.inf)), h)
    return h.astype(np.float32)


@pytest.mark.parametrize("levels", [3, 15])
def test_codes_stay_in_range_without_a_clamp(levels):
    """The writer stores rint(fl(fl(x - min_h) * r)) without clamping it to
    [0, levels], where min_h is the group minimum rounded down to fp16, the
    scale s_h the correctly rounded fl(span / levels) rounded up to fp16
    (span = fl(max - min_h)) and r its reciprocal within one ulp (or the
    IEEE quotient for values near a tie).  Over groups of finite bf16 inputs
    with |x| <= 65280 (random, tiny spans, spans across the whole range,
    constant groups), every such quotient must round into [0, levels]."""
    import numpy as np
    rng = np.random.default_rng(7)
    groups = []
    for _ in range(4000):
        kind = rng.integers(0, 6)
        if kind == 0:
            g = rng.standard_normal(128) * 10.0 ** rng.uniform(-6, 4)
        elif kind == 1:
            g = rng.uniform(-65280, 65280, 128)
        elif kind == 2:
            c = rng.uniform(-65280, 65280)
            g = c + rng.standard_normal(128) * abs(c) * 1e-3
        elif kind == 3:
            g = np.full(128, rng.uniform(-65280, 65280))
        elif kind == 4:
            g = np.where(rng.random(128) < 0.5, -65280.0, 65280.0)
        else:
            g = rng.standard_normal(128) * 1e-4 + rng.uniform(-3, 3)
        groups.append(np.clip(g, -65280, 65280))
    x = np.asarray(groups, dtype=np.float32)
    # bf16 inputs (round to nearest even on the top 16 bits)
    b = x.view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    x = b.astype(np.uint32).view(np.float32)
    x = np.clip(x, np.float32(-65280), np.float32(65280))
    mn, mx = x.min(axis=1), x.max(axis=1)
    mh = _f16_directed(mn, up=False)
    span = (mx - mh).astype(np.float32)
    s = (span / np.float32(levels)).astype(np.float32)
    sh = _f16_directed(s, up=True)
    ok = sh > 0
    d = (x - mh[:, None]).astype(np.float32)
    assert (d >= 0).all()
    r = (np.float32(1) / sh[ok]).astype(np.float32)
    for rr in (r, np.nextafter(r, np.float32(np.inf)), np.nextafter(r, np.float32(0))):
        q = (d[ok] * rr[:, None]).astype(np.float32)
        assert np.rint(q).max() <= levels and np.rint(q).min() >= 0
    q = (d[ok] / sh[ok][:, None]).astype(np.float32)
    assert np.rint(q).max() <= levels
    # zero scale: every value equals min_h, so every code is 0
    assert (d[~ok] == 0).all()
