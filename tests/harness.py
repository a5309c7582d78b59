"""Shared helpers of the tests: build the same cache on the GPU (through the C
ABI) and in the CPU oracle from the same seeded inputs, and compare them."""
from __future__ import annotations

import math
import sys

import numpy as np

from bit_kv_cache_writer_amd import workloads as wl

TOL_REL = 2e-3   # per (sequence, head) row: max |o - r| / max |r|
TOL_LSE = 2e-3   # absolute, natural-log units


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def layouts(P, bits, clip, sink, local):
    import oracle
    from bit_kv_cache_writer_amd import mla
    return (mla.Layout(P, bits, clip, sink, local), oracle.Layout(P, bits, clip, sink, local))


class OracleCache:
    def __init__(self, lay, batch, max_pages, block_table, n_pool):
        import oracle
        self.orc, self.lay = oracle, lay
        self.pb = oracle.page_bytes(lay)
        self.bt = np.ascontiguousarray(block_table, dtype=np.int32)
        self.pool = np.zeros(n_pool * self.pb, np.uint8)
        self.sink = np.zeros((batch, max(lay.sink, 1), 576), np.uint16)
        self.ring = np.zeros((batch, max(lay.local, 1), 576), np.uint16)
        self.tail = np.zeros((batch, lay.page_size, 64), np.uint16)
        self.len = np.zeros(batch, np.int32)

    def append(self, ckv, kr, counts):
        cu = wl.cu_from_counts(counts)
        self.orc.write(self.lay, np.ascontiguousarray(ckv), np.ascontiguousarray(kr), cu,
                       self.len.copy(), self.bt, self.pool, self.sink, self.ring, self.tail)
        self.len += np.asarray(counts, np.int32)

    def decode(self, ql, qr, scale):
        return self.orc.decode(self.lay, np.ascontiguousarray(ql), np.ascontiguousarray(qr), scale,
                               self.pool, self.bt, self.len.copy(), self.sink, self.ring, self.tail)


def compare_cache(gpu, ref: OracleCache, seqs=None):
    """Bit-exact comparison of every region the writer defines (codes and
    metadata of complete pages, written rows of the unfinished page, sink rows,
    window ring slots, k_R tail rows)."""
    lay = ref.lay
    P, pb = lay.page_size, ref.pb
    pool = gpu.pool.cpu().numpy()
    sink = gpu.sink.cpu().numpy().view(np.uint16)
    ring = gpu.ring.cpu().numpy().view(np.uint16)
    tail = gpu.tail.cpu().numpy().view(np.uint16)
    off = ref.orc.page_offsets(lay)
    lat_row = off["latent_row"]
    seqs = range(len(ref.len)) if seqs is None else seqs
    for b in seqs:
        L = int(ref.len[b])
        for i in range((L + P - 1) // P):
            pid = int(ref.bt[b, i])
            g = pool[pid * pb:(pid + 1) * pb]
            r = ref.pool[pid * pb:(pid + 1) * pb]
            if (i + 1) * P <= L:
                if not np.array_equal(g, r):
                    bad = np.nonzero(g != r)[0]
                    raise AssertionError(f"seq {b} page {i}: {bad.size} bytes differ, first at {bad[:8]}")
            else:
                n = L - i * P
                np.testing.assert_array_equal(g[: n * lat_row], r[: n * lat_row],
                                              err_msg=f"seq {b} tail page latent codes")
                mo = off["latent_meta"]
                np.testing.assert_array_equal(g[mo:mo + n * 16], r[mo:mo + n * 16],
                                              err_msg=f"seq {b} tail page latent metadata")
        ns = min(lay.sink, L)
        np.testing.assert_array_equal(sink[b, :ns], ref.sink[b, :ns], err_msg=f"seq {b} sink rows")
        if lay.local > 0:
            slots = [t % lay.local for t in range(max(0, L - lay.local), L)]
            np.testing.assert_array_equal(ring[b, slots], ref.ring[b, slots], err_msg=f"seq {b} ring")
        nt = L % P
        np.testing.assert_array_equal(tail[b, :nt], ref.tail[b, :nt], err_msg=f"seq {b} k_R tail rows")


def compare_decode(out, lse, ref_out, ref_lse, heads=None, seqs=None):
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    worst = 0.0
    seqs = range(ref_out.shape[0]) if seqs is None else seqs
    for bi, b in enumerate(seqs):
        for hi in range(ref_out.shape[1]):
            r = ref_out[bi, hi]
            o = out[bi, hi]
            denom = np.abs(r).max()
            if denom == 0.0:
                assert np.abs(o).max() == 0.0, f"seq {b} head {hi}: expected zero output"
                assert np.isneginf(lse[bi, hi]) and np.isneginf(ref_lse[bi, hi])
                continue
            err = np.abs(o - r).max() / denom
            worst = max(worst, err)
            assert err <= TOL_REL, f"seq {b} head {hi}: max rel err {err:.3e} > {TOL_REL}"
            d = abs(lse[bi, hi] - ref_lse[bi, hi])
            assert d <= TOL_LSE, f"seq {b} head {hi}: lse diff {d:.3e}"
    return worst


def random_tokens(seed, n, outliers=(7, 23, 39, 55), mult=20.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 576)).astype(np.float32)
    x[:, [512 + c for c in outliers]] *= mult
    return wl.f32_to_bf16_bits(x[:, :512]), wl.f32_to_bf16_bits(x[:, 512:])


def random_queries(seed, batch, heads):
    rng = np.random.default_rng(seed)
    return (wl.f32_to_bf16_bits(rng.standard_normal((batch, heads, 512)).astype(np.float32)),
            wl.f32_to_bf16_bits(rng.standard_normal((batch, heads, 64)).astype(np.float32)))


def perm_block_table(seed, batch, max_pages):
    n_pool = int(math.ceil(batch * max_pages * 1.25)) + 1
    bt = np.random.default_rng(seed).permutation(n_pool)[: batch * max_pages]
    return bt.astype(np.int32).reshape(batch, max_pages), n_pool
