"""Planted mistakes in the oracle must be caught by the pins.

Each case copies ``oracle/mla_oracle.c``, plants one plausible mistake by a
textual substitution, builds the copy with gcc into a temporary library and
runs the pin tests against it in a subprocess.  The pins must fail.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mla_oracle.c")

MUTANTS = {
    "round_down_is_nearest": ("if (g_f16_sorted[mid] <= x) {", "if (g_f16_sorted[mid] <= x + ldexp(1.0, -12) * fabs(x)) {"),
    "quantile_off_by_one": ("int32_t l = (int32_t)floor(h);", "int32_t l = (int32_t)floor(h) + 1;"),
    "clip_frac_dropped": ("float c = a[lo] + p;", "float c = a[lo] + 0.0f * p;"),
    "scale_levels_plus_one": ("float s = span / (float)levels;", "float s = span / (float)(levels + 1);"),
    "round_half_up": ("float r = rintf(t);", "float r = floorf(t + 0.5f);"),
    "pack_high_nibble_first": ("row[bit / 8] |= (uint8_t)(code << (bit % 8));",
                               "row[bit / 8] |= (uint8_t)(code << ((8 - bits - bit % 8)));"),
    "rope_scale_min_swapped": ("put_f16(meta + 2 * c, sh);", "put_f16(meta + 2 * c, mh);"),
    "protected_window_off_by_one": ("j >= Lb - L->local)", "j > Lb - L->local)"),
    "rope_term_dropped": ("for (int c = 0; c < W; ++c) acc += q[h * W + c] * tok[c];",
                          "for (int c = 0; c < D; ++c) acc += q[h * W + c] * tok[c];"),
    "page_complete_wrong": ("int page_complete = (int64_t)(pidx + 1) * P <= Lb;",
                            "int page_complete = (int64_t)(pidx + 1) * P < Lb;"),
    "softmax_not_max_subtracted": ("s += exp(z[(int64_t)h * Lb + j] - m);", "s += exp(z[(int64_t)h * Lb + j] - m) * 1.0001;"),
    "bf16_cache_slot_off_by_one": ("bt[j / page_size] * page_size + j % page_size) * W;\n        double acc",
                                   "bt[j / page_size] * page_size + (j + 1) % page_size) * W;\n        double acc"),
    "bf16_cache_rope_dropped": ("for (int c = 0; c < W; ++c) acc += q[c] * bf16_to_f32(row[c]);",
                                "for (int c = 0; c < D; ++c) acc += q[c] * bf16_to_f32(row[c]);"),
    "transform_ties_away": ("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))",
                            "if (dropped >= 0x8000u)"),
    "transform_matrix_transposed": ("acc = fmaf(bf16_to_f32(a_c[(int64_t)c * dim + k])",
                                    "acc = fmaf(bf16_to_f32(a_c[(int64_t)k * dim + c])"),
    "transform_double_accumulation": ("      float acc = 0.0f;\n      for (int32_t k = 0; k < dim; ++k)\n        acc = fmaf(",
                                      "      double acc = 0.0;\n      for (int32_t k = 0; k < dim; ++k)\n        acc = fma("),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found for {name}"
    with tempfile.TemporaryDirectory() as d:
        csrc = os.path.join(d, "m.c")
        lib = os.path.join(d, "libm.so")
        open(csrc, "w").write(src.replace(old, new, 1))
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", csrc, "-o", lib, "-lm"])
        env = dict(os.environ, MLA_ORACLE_LIB=lib)
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        assert r.returncode != 0, f"planted mistake {name} passed every pin:\n{r.stdout[-2000:]}"
