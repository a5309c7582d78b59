"""Host-side checks of the C ABI (no GPU): the library loads and exports every
entry point of include/mla_lowbit.h, the layout query matches the oracle's
independent byte geometry, and bad arguments are rejected before anything is
launched."""
import ctypes
import os
import re

import pytest

from bit_kv_cache_writer_amd import mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "mla_lowbit.h")).read()
    return sorted(set(re.findall(r"\b(mla_lowbit_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert set(names) == set(mla.EXPORTS)
    lib = mla.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_exports_every_probe_symbol():
    text = open(os.path.join(ROOT, "include", "mla_lowbit_probe.h")).read()
    names = set(re.findall(r"\b(mla_lowbit_\w+)\s*\(", text))
    assert names == set(mla.PROBE_EXPORTS)
    lib = mla.lib()
    for n in names:
        assert hasattr(lib, n), n
    # argument errors are found on the host
    flops = ctypes.c_double()
    assert lib.mla_lowbit_probe_mfma(None, 10, ctypes.byref(flops), None) == -2
    assert lib.mla_lowbit_probe_mfma(256, 0, ctypes.byref(flops), None) == -2
    assert lib.mla_lowbit_probe_read(256, 100, 256, None) == -2   # not a multiple of 64
    assert lib.mla_lowbit_probe_read(None, 64, 256, None) == -2


@pytest.mark.parametrize("P", [32, 64, 128, 256])
@pytest.mark.parametrize("bits", [2, 4])
def test_layout_query_matches_oracle(orc, P, bits):
    s = mla.mla_lowbit_layout_query(mla.Layout(P, bits, 0.94 if bits == 2 else 0.0, 4, 128))
    off = orc.page_offsets(orc.Layout(P, bits, 0.0, 4, 128))
    assert s["page_bytes"] == off["page_bytes"]
    assert s["latent_meta_offset"] == off["latent_meta"]
    assert s["rope_codes_offset"] == off["rope_codes"]
    assert s["rope_meta_offset"] == off["rope_meta"]
    assert s["latent_row_bytes"] == off["latent_row"]
    assert s["sink_bytes_per_seq"] == 4 * 1152 and s["ring_bytes_per_seq"] == 128 * 1152
    assert s["tail_bytes_per_seq"] == P * 128


@pytest.mark.parametrize("bad", [
    dict(page_size=48), dict(page_size=16), dict(latent_bits=3), dict(latent_clip_q=1.5),
    dict(latent_clip_q=-0.1), dict(latent_clip_q=float("nan")), dict(sink=65), dict(local=5000),
    dict(latent_dim=256), dict(rope_dim=128), dict(rope_bits=2), dict(latent_group=64), dict(version=2),
])
def test_bad_layouts_rejected(bad):
    base = dict(page_size=64, latent_bits=4, latent_clip_q=0.0, sink=4, local=128)
    base.update(bad)
    with pytest.raises(mla.MlaError) as e:
        mla.mla_lowbit_layout_query(mla.Layout(**base))
    assert e.value.code == -1


def test_workspace_query_and_errors():
    lay = mla.Layout(128, 4, 0.0, 4, 128)
    part = 16 * 512 * 2 + 32 * 4  # one split's partial: 16 heads x 512 fp16 outputs + fp32 max, sum
    n = mla.mla_lowbit_decode_workspace(lay, 32, 16, 4096)
    assert n > 0 and n % (32 * part) == 0  # whole partials for each of the 32 sequences
    assert mla.mla_lowbit_decode_workspace(lay, 1, 16, 0) == 0  # one split: no partials
    for args in [(0, 0, 4096), (32, 129, 4096), (32, 16, -1)]:
        with pytest.raises(mla.MlaError) as e:
            mla.mla_lowbit_decode_workspace(lay, *args)
        assert e.value.code == -2


# The work split the decode chooses, seen through the workspace it needs
# (groups x splits x one partial).  Two workgroups per CU (512), at most 512
# splits, the BF16-path count minimizing the longer of the two kinds of
# workgroup: the headline batch keeps 16 splits (3 BF16-path + 13 packed, five
# rounds of packed tiles), one long sequence fills the chip with 512, 128 heads
# need 3 per (sequence, head block) (1 BF16-path + 2 packed, a 512-page window
# each).
SPLITS = [
    # (P, bits, batch, heads, max_seqlen, splits per (sequence, head block))
    (128, 4, 32, 16, 4096, 16),
    (128, 4, 8, 16, 4096, 35),
    (128, 4, 1, 16, 1 << 20, 512),
    (64, 4, 64, 128, 32768, 3),
    (64, 2, 4, 64, 131072, 32),
]


@pytest.mark.parametrize("P,bits,batch,heads,L,splits", SPLITS)
def test_decode_split_plan(P, bits, batch, heads, L, splits):
    lay = mla.Layout(P, bits, 0.94 if bits == 2 else 0.0, 4, 128)
    part = 16 * 512 * 2 + 32 * 4
    groups = batch * ((heads + 15) // 16)
    assert mla.mla_lowbit_decode_workspace(lay, batch, heads, L) == groups * splits * part


def _write(lay, **kw):
    a = dict(c_kv=16, k_r=16, cu_new=16, seqlens_before=16, batch=1, total_new=1, max_new_per_seq=1,
             block_table=16, max_pages=1, num_pool_pages=1, page_pool=16, sink_buf=16, ring_buf=16,
             rope_tail=16)
    a.update(kw)
    L = mla.lib()
    return L.mla_lowbit_write(ctypes.byref(lay.c()), a["c_kv"], a["k_r"], a["cu_new"], a["seqlens_before"],
                              a["batch"], a["total_new"], a["max_new_per_seq"], a["block_table"],
                              a["max_pages"], a["num_pool_pages"], a["page_pool"], a["sink_buf"],
                              a["ring_buf"], a["rope_tail"], None)


def test_write_rejects_bad_arguments_without_launch():
    lay = mla.Layout(64, 4, 0.0, 4, 32)
    assert _write(lay, c_kv=None) == -2
    assert _write(lay, rope_tail=None) == -2
    assert _write(lay, sink_buf=None) == -2
    assert _write(lay, c_kv=24) == -2          # misaligned
    assert _write(lay, batch=-1) == -2
    assert _write(lay, max_pages=0) == -2
    assert _write(lay, batch=0) == 0           # nothing to do
    assert _write(lay, total_new=0) == 0
    bad = mla.Layout(64, 4, 0.0, 4, 32, version=7)
    assert _write(bad) == -1


def _decode(lay, **kw):
    a = dict(q_lat=256, q_rope=256, batch=1, heads=16, scale=0.07, pool=256, num_pool_pages=4,
             block_table=256, max_pages=4, seqlens=256, max_seqlen=100, sink=256, ring=256, tail=256,
             out=256, lse=256, ws=256, ws_bytes=1 << 30)
    a.update(kw)
    L = mla.lib()
    return L.mla_lowbit_decode(ctypes.byref(lay.c()), a["q_lat"], a["q_rope"], a["batch"], a["heads"],
                               a["scale"], a["pool"], a["num_pool_pages"], a["block_table"],
                               a["max_pages"], a["seqlens"], a["max_seqlen"], a["sink"], a["ring"],
                               a["tail"], a["out"], a["lse"], a["ws"], a["ws_bytes"], None)


def test_decode_rejects_bad_arguments_without_launch():
    lay = mla.Layout(64, 4, 0.0, 4, 32)
    assert _decode(lay, q_lat=None) == -2
    assert _decode(lay, heads=0) == -2
    assert _decode(lay, heads=129) == -2
    assert _decode(lay, max_seqlen=4 * 64 + 1) == -2     # beyond the block table
    # 256 tokens of one sequence split in two: partials need a 16-B aligned workspace
    assert _decode(lay, max_seqlen=256, ws=512 + 8) == -2
    assert _decode(lay, max_seqlen=256, ws_bytes=16) == -4
    assert _decode(lay, max_seqlen=256, ws=None) == -4
    assert _decode(lay, scale=float("inf")) == -2
    assert _decode(lay, out=258) == -2
    assert _decode(lay, batch=0) == 0
    assert _decode(mla.Layout(64, 3, 0.0, 4, 32)) == -1


def _decode_noalloc(lay, **kw):
    a = dict(q_lat=256, q_rope=256, batch=1, heads=16, scale=0.07, pool=256, num_pool_pages=4,
             block_table=256, max_pages=4, seqlens=256, max_seqlen=100, sink=256, ring=256, tail=256,
             out=256, lse=256)
    a.update(kw)
    L = mla.lib()
    return L.mla_lowbit_decode_noalloc(ctypes.byref(lay.c()), a["q_lat"], a["q_rope"], a["batch"], a["heads"],
                                       a["scale"], a["pool"], a["num_pool_pages"], a["block_table"],
                                       a["max_pages"], a["seqlens"], a["max_seqlen"], a["sink"], a["ring"],
                                       a["tail"], a["out"], a["lse"], None)


def test_decode_noalloc_rejects_without_launch():
    """Argument errors and shapes whose partials exceed the fixed scratch are
    refused on the host, before any HIP call."""
    lay = mla.Layout(64, 4, 0.0, 4, 128)
    assert _decode_noalloc(lay, q_lat=None) == -2
    assert _decode_noalloc(lay, heads=0) == -2
    assert _decode_noalloc(lay, batch=0) == 0
    assert _decode_noalloc(mla.Layout(64, 3, 0.0, 4, 32)) == -1
    # 512 sequences x 32768 tokens x 128 heads: the split partials need far
    # more than the scratch array
    need = mla.mla_lowbit_decode_workspace(lay, 512, 128, 32768)
    assert need > mla.NOALLOC_SCRATCH_BYTES
    assert _decode_noalloc(lay, batch=512, heads=128, max_seqlen=32768, max_pages=512, num_pool_pages=512 * 512) == -6
    assert "NOALLOC" in mla.strerror(-6)


def test_strerror():
    for c in (0, -1, -2, -3, -4, -5, -6, 99):
        assert isinstance(mla.strerror(c), str) and mla.strerror(c)


# ----------------------------------------------------------------------------
# the plain BF16 paged cache (include/mla_bf16.h)

def test_exports_every_bf16_symbol():
    text = open(os.path.join(ROOT, "include", "mla_bf16.h")).read()
    names = set(re.findall(r"\b(mla_bf16_\w+)\s*\(", text))
    assert names == set(mla.BF16_EXPORTS)
    lib = mla.lib()
    for n in names:
        assert hasattr(lib, n), n


# Work split of the BF16 decode, seen through its workspace: two workgroups
# per CU (512) over (sequence, head block, split), at least 4 tiles of 16
# tokens per split, at most 510 pages per split, at most 512 splits.
BF16_SPLITS = [
    # (P, batch, heads, max_seqlen, splits per (sequence, head block))
    (64, 32, 16, 4096, 16),       # 512 / 32
    (64, 8, 16, 65536, 64),       # 512 / 8
    (64, 1, 16, 1 << 20, 512),    # one sequence fills the chip
    (16, 1, 16, 1 << 20, 512),    # 65536 tiles over 510-page windows: 129 at least, 512 taken
    (64, 64, 128, 32768, 2),      # 512 groups already, but 512 pages pass the window
    (64, 4, 16, 100, 2),          # 7 tiles: at least 4 per split
]


@pytest.mark.parametrize("P,batch,heads,L,splits", BF16_SPLITS)
def test_bf16_decode_split_plan(P, batch, heads, L, splits):
    part = 16 * 512 * 2 + 32 * 4
    groups = batch * ((heads + 15) // 16)
    n = mla.mla_bf16_decode_workspace(P, batch, heads, L)
    assert n == (0 if splits == 1 else groups * splits * part)


def test_bf16_argument_errors():
    lib = mla.lib()
    for args in [(8, 32, 16, 4096), (64, 32, 0, 4096), (64, 32, 129, 4096), (64, 32, 16, -1), (48, 1, 16, 64),
                 (2048, 1, 16, 64)]:
        with pytest.raises(mla.MlaError) as e:
            mla.mla_bf16_decode_workspace(*args)
        assert e.value.code == -2
    # decode: bad page size, max_seqlen beyond the block table, missing pool
    f = lib.mla_bf16_decode
    assert f(256, 256, 1, 16, 0.1, 256, 1, 40, 256, 1, 256, 16, 256, 256, None, 0, None) == -2
    assert f(256, 256, 1, 16, 0.1, 256, 1, 64, 256, 1, 256, 65, 256, 256, None, 0, None) == -2
    assert f(256, 256, 1, 16, 0.1, None, 1, 64, 256, 1, 256, 64, 256, 256, None, 0, None) == -2
    assert f(256, 256, 1, 16, float("nan"), 256, 1, 64, 256, 1, 256, 64, 256, 256, None, 0, None) == -2
    # a missing workspace where one is needed
    assert f(256, 256, 8, 16, 0.1, 256, 1, 64, 256, 64, 256, 4096, 256, 256, None, 0, None) == -4
    # append: bad page size, misaligned rows, missing block table
    g = lib.mla_bf16_append
    assert g(256, 256, 256, 256, 1, 4, 4, 40, 256, 1, 1, 256, None) == -2
    assert g(257, 256, 256, 256, 1, 4, 4, 64, 256, 1, 1, 256, None) == -2
    assert g(256, 256, 256, 256, 1, 4, 4, 64, None, 1, 1, 256, None) == -2
    assert g(None, None, None, None, 1, 0, 0, 64, None, 0, 0, None, None) == 0  # nothing to append
