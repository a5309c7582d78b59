"""Host-side checks of bench.py's measurement arithmetic (no GPU): the
algorithmic bytes and useful flops per decode call that every roofline figure
divides by, against the per-workload totals derived by hand from the layout
(C4R4 304 B / C2R4 176 B per packed token, 256 B of k_R metadata per page
read, 1152 B per BF16-path token, 1152 B of queries and 2052 B of output + lse
per (sequence, head); 2176 flops per cached token and head), and the one-GPU
contract of the command line."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from bit_kv_cache_writer_amd import workloads as wl  # noqa: E402

# (workload, algorithmic MB per call, binding roofline): the totals of the
# hot-path measurement table, rounded as printed there
EXPECTED = [
    ("tiny_c4r4", 0.161, "hbm"),
    ("c4r4_h16_b8", 11.33, "hbm"),
    ("c4r4_h16_b32", 45.32, "hbm"),
    ("c2r4_h20", 49.74, "hbm"),
    ("c4r4_h128", 679.3, "mfma"),
    ("c2r4_h64_long", 95.71, "mfma"),
]


@pytest.mark.parametrize("name,mb,bound", EXPECTED, ids=[e[0] for e in EXPECTED])
def test_algorithmic_bytes_and_bound(name, mb, bound):
    w = wl.WORKLOADS[name]
    total = bench.algorithmic_decode_bytes(w, w.seqlen)["total"] * w.batch
    digits = 3 if mb < 1 else (2 if mb < 100 else 1)
    assert round(total / 1e6, digits) == pytest.approx(mb, abs=10 ** -digits)
    flops = bench.FLOPS_PER_TOKEN_HEAD * w.seqlen * w.heads * w.batch
    hbm_s = total / (bench.HBM_PEAK_GBS * 1e9)
    mfma_s = flops / (bench.MFMA_F16_PEAK_TFLOPS * 1e12)
    assert ("hbm" if hbm_s >= mfma_s else "mfma") == bound


def test_packed_token_bytes_by_hand():
    # 32 x 4096, P = 128, sink 4, local 128: 3964 packed tokens in pages 0..30
    # (31 pages), 132 BF16-path tokens
    w = wl.WORKLOADS["c4r4_h16_b32"]
    a = bench.algorithmic_decode_bytes(w, 4096)
    assert a["packed_tokens"] == 4096 - 128 - 4
    assert a["cache"] == 3964 * 304 + 31 * 256 + 132 * 1152
    assert a["q"] == 16 * 1152 and a["out"] == 16 * 2052


def test_flops_per_token_head():
    assert bench.FLOPS_PER_TOKEN_HEAD == 2 * (512 + 64) + 2 * 512 == 2176


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
