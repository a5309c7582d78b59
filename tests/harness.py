"""Shared helpers of the tests: build the same cache on the GPU (through the C
ABI) and in the CPU oracle from the same seeded inputs, and compare them."""
from __future__ import annotations

import math
import sys

import numpy as np

from bit_kv_cache_writer_amd import workloads as wl

TOL_REL = 2e-3   # per (sequence, head) row: max |o - r| / max |r|
TOL_LSE = 2e-3   # absolute, natural-log units, plus the fp32 slack below
# An fp32 dot product of n terms carries rounding errors that scale with
# u * sum_i |a_i b_i| (u = 2^-24; the classical bound is n u sum |a_i b_i|),
# not with the size of the result, and the lse of a peaked softmax is the top
# score itself.  So the lse bar adds 2^-17 = 128 u times the score's L1 size
# S = scale * max_j sum_c |q_c x_jc| (x the oracle's dequantized tokens): at
# unit-scale inputs this is ~2e-4, at latents scaled by 10^3 it is what any
# fp32 score computation needs.  The output bar (TOL_REL) is unchanged.
LSE_FP32_FRACTION = 2.0 ** -17


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


# worst errors of every decode comparison of the session, printed in the
# terminal summary (tests/conftest.py) so that the margin to the 2e-3 bar
# shows even in a quiet run
PARITY_LOG: list = []


def record(case: str, worst_rel: float, worst_lse: float, rows: int, lse_use: float = 0.0) -> None:
    """lse_use: the largest |d lse| / bar over the case's rows (the bar
    includes the fp32 slack where one is given)."""
    PARITY_LOG.append((case, worst_rel, worst_lse, rows, lse_use))


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

    def lse_slack(self, ql, qr, scale, chunk=8192):
        """LSE_FP32_FRACTION * scale * max_j sum_c |q_c x_jc| per (sequence, head),
        x_j the oracle's dequantized tokens (as its decode reads them)."""
        B, H, _ = ql.shape
        q = np.abs(np.concatenate([wl.bf16_bits_to_f32(ql), wl.bf16_bits_to_f32(qr)], axis=2)).astype(np.float64)
        S = np.zeros((B, H))
        for b in range(B):
            L = int(self.len[b])
            for j0 in range(0, L, chunk):
                X = np.stack([self.orc.read_token(self.lay, self.pool, self.bt, self.sink, self.ring, self.tail,
                                                  b, L, j)[0] for j in range(j0, min(L, j0 + chunk))])
                S[b] = np.maximum(S[b], (np.abs(X) @ q[b].T).max(axis=0))
        return LSE_FP32_FRACTION * abs(scale) * S


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


def compare_decode(out, lse, ref_out, ref_lse, heads=None, seqs=None, case=None, lse_slack=None):
    """Per (sequence, head) row: max |o - r| / max |r| <= TOL_REL and
    |lse - lse_ref| <= TOL_LSE + lse_slack (OracleCache.lse_slack); outputs
    must be finite.  Returns the worst row error; with `case`, the worst
    errors are recorded for the summary."""
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    assert np.all(np.isfinite(out)), "non-finite decode output"
    worst, worst_lse, lse_use, rows = 0.0, 0.0, 0.0, 0
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
            rows += 1
            assert err <= TOL_REL, f"seq {b} head {hi}: max rel err {err:.3e} > {TOL_REL}"
            d = abs(lse[bi, hi] - ref_lse[bi, hi])
            worst_lse = max(worst_lse, d)
            bar = TOL_LSE + (0.0 if lse_slack is None else float(lse_slack[bi, hi]))
            lse_use = max(lse_use, d / bar)
            assert d <= bar, f"seq {b} head {hi}: lse diff {d:.3e} > {bar:.3e}"
    if case is not None:
        record(case, worst, worst_lse, rows, lse_use)
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
