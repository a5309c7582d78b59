"""Pins of the CPU oracle against things other than itself (no GPU).

Each test ties one part of the oracle to the pages' printed numbers, a closed
form, a library routine (numpy float16 conversion, numpy.quantile, torch's
scaled-dot-product attention) or brute force on tiny inputs.
"""
import json
import os

import numpy as np
import pytest
import torch

from bit_kv_cache_writer_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# fp16 directed rounding of the metadata

def _numpy_directed(x):
    rn = x.astype(np.float16)
    back = rn.astype(np.float32)
    with np.errstate(over="ignore"):  # nextafter(+-65504) -> inf, never selected
        down = np.where(back > x, np.nextafter(rn, np.float16(-np.inf)), rn)
        up = np.where(back < x, np.nextafter(rn, np.float16(np.inf)), rn)
    return down, up


def test_f16_directed_rounding_matches_numpy(orc):
    rng = np.random.default_rng(0)
    parts = [rng.standard_normal(4000) * s for s in (1e-8, 1e-6, 1e-4, 1e-2, 1, 100, 2e4)]
    exact = rng.integers(0, 0x7C00, 3000).astype(np.uint16).view(np.float16).astype(np.float32)
    mids = (exact[:-1].astype(np.float64) + exact[1:]) / 2
    x = np.concatenate(parts + [exact, -exact, mids, [0.0, 65504.0, -65504.0, 6e-8, -6e-8]])
    x = x.astype(np.float32)
    x = x[np.abs(x) <= 65504]
    down, up = _numpy_directed(x)
    rd = orc.f16_round_down(x).view(np.float16)
    ru = orc.f16_round_up(x).view(np.float16)
    np.testing.assert_array_equal(rd.astype(np.float64), down.astype(np.float64))
    np.testing.assert_array_equal(ru.astype(np.float64), up.astype(np.float64))
    # invariants: rd <= x <= ru, no fp16 strictly between
    assert np.all(rd.astype(np.float64) <= x) and np.all(ru.astype(np.float64) >= x)
    # a zero result is always +0
    assert np.all(orc.f16_round_down(np.float32([1e-9, 0.0]))[:2] == 0)


# ----------------------------------------------------------------------------
# 0.94-quantile clipping (RAQ-MLA Table 5)

def test_quantile_params_closed_form(orc):
    lo, hi, frac = orc.quantile_params(512, 0.94)
    assert (lo, hi) == (480, 481)
    assert frac == np.float32(0.34)
    assert orc.quantile_params(512, 1.0)[:2] == (511, 511)


def test_clip_of_permutation_is_481_34(orc):
    rng = np.random.default_rng(1)
    x = rng.permutation(np.arange(1, 513, dtype=np.float32)) * rng.choice([-1, 1], 512)
    c = orc.clip_value(x.astype(np.float32), 0.94)
    assert abs(c - 481.34) <= 2 ** -15


@pytest.mark.parametrize("q", [0.5, 0.9, 0.94, 0.99, 1.0])
def test_clip_matches_numpy_quantile(orc, q):
    rng = np.random.default_rng(2)
    for _ in range(50):
        x = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(rng.standard_normal(512).astype(np.float32)))
        c = orc.clip_value(x, q)
        ref = np.quantile(np.abs(x).astype(np.float64), q)
        assert abs(c - ref) <= 2 * np.spacing(np.float32(ref)), (c, ref)


# ----------------------------------------------------------------------------
# asymmetric min/scale quantizer

def _dequant(codes, sh, mh):
    s = np.uint16(sh).view(np.float16).astype(np.float64)
    m = np.uint16(mh).view(np.float16).astype(np.float64)
    return codes.astype(np.float64) * s + m, s, m


@pytest.mark.parametrize("levels", [3, 15])
def test_quantizer_round_trip_and_argmin(orc, levels):
    rng = np.random.default_rng(3 + levels)
    for trial in range(300):
        scale = 10.0 ** rng.uniform(-3, 3)
        x = (rng.standard_normal(128) * scale + rng.uniform(-1, 1) * scale).astype(np.float32)
        x = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(x))
        codes, sh, mh = orc.quantize_group(x, levels)
        xh, s, m = _dequant(codes, sh, mh)
        assert codes.max() <= levels
        xd = x.astype(np.float64)
        # the fp16 grid covers the group
        assert m <= xd.min()
        assert m + levels * s >= xd.max() - 4 * np.spacing(np.float32(abs(xd).max()))
        # round trip: |x - x_hat| <= s/2 (fp32 slack on the division)
        assert np.all(np.abs(xd - xh) <= s * (0.5 + 2.0 ** -18))
        # brute force: nearest grid point, ties broken towards the even code
        t = (xd - m) / s
        ks = np.arange(levels + 1)
        dist = np.abs(t[:, None] - ks[None, :])
        best = ks[np.argmin(dist, axis=1)]
        frac = t - np.floor(t)
        clear = np.abs(frac - 0.5) > 1e-5
        np.testing.assert_array_equal(codes[clear], best[clear])
        # monotone in x
        order = np.argsort(x, kind="stable")
        assert np.all(np.diff(codes[order].astype(int)) >= 0)


def test_quantizer_exact_grid(orc):
    k = np.arange(16)
    x = (-1.0 + k / 8.0).astype(np.float32)
    codes, sh, mh = orc.quantize_group(np.tile(x, 8), 15)
    xh, s, m = _dequant(codes, sh, mh)
    assert s == 0.125 and m == -1.0
    np.testing.assert_array_equal(codes[:16], k)
    np.testing.assert_array_equal(xh, np.tile(x, 8).astype(np.float64))
    # exact midpoints between grid points: ties go to the even code, as numpy's
    # round (IEEE round-half-even) does
    mid = (-1.0 + (np.arange(15) + 0.5) / 8.0).astype(np.float32)
    g = np.concatenate([x, mid, np.tile(x, 6)[: 128 - 31]]).astype(np.float32)
    codes, sh, mh = orc.quantize_group(g, 15)
    t = (g.astype(np.float64) + 1.0) * 8.0
    np.testing.assert_array_equal(codes, np.round(t).astype(np.uint8))
    assert list(codes[16:31]) == [0, 2, 2, 4, 4, 6, 6, 8, 8, 10, 10, 12, 12, 14, 14]


def test_quantizer_degenerate_groups(orc):
    codes, sh, mh = orc.quantize_group(np.zeros(128, np.float32), 3)
    assert sh == 0 and mh == 0 and not codes.any()
    c = np.full(128, 0.3, np.float32)
    codes, sh, mh = orc.quantize_group(c, 15)
    xh, s, m = _dequant(codes, sh, mh)
    assert np.all(np.abs(xh - np.float64(np.float32(0.3))) <= 2 ** -12)


# ----------------------------------------------------------------------------
# packing: channel c in byte c*b/8, lower channels in lower bits

def test_pack_closed_form(orc):
    assert list(orc.pack_row(np.arange(16), 4)) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert list(orc.pack_row([0, 1, 2, 3], 2)) == [0xE4]
    rng = np.random.default_rng(5)
    for bits in (2, 4):
        c = rng.integers(0, 1 << bits, 512).astype(np.uint8)
        np.testing.assert_array_equal(orc.unpack_row(orc.pack_row(c, bits), 512, bits), c)


# ----------------------------------------------------------------------------
# effective bits (RAQ-MLA Table 5, Table 1 BPE, abstract)

def test_effective_bits_match_pages(orc):
    g = json.load(open(os.path.join(GOLDEN, "effective_bits.json")))
    for P in (64, 128):
        for bits in (2, 4):
            off = orc.page_offsets(orc.Layout(P, bits, 0.0, 4, 128))
            lat = off["rope_codes"] * 8 / (P * 512)
            rope = (off["page_bytes"] - off["rope_codes"]) * 8 / (P * 64)
            assert lat == bits + 32 / 128
            assert rope == 4 + 32 / P
            if bits == 2:
                assert lat == g["latent_bits_2bit_g128"]
            assert rope == g["rope_bits_4bit_per_page"][str(P)]
    tot128 = orc.page_bytes(orc.Layout(128, 2, 0.94, 4, 128)) * 8 / (128 * 576)
    tot64 = orc.page_bytes(orc.Layout(64, 2, 0.94, 4, 128)) * 8 / (64 * 576)
    pr = g["printed_precision"]
    assert abs(tot128 - g["bpe_c2r4_page128_printed"]) <= pr["bpe_c2r4_page128_printed"]
    assert abs(tot64 - g["bpe_c2r4_about"]) <= pr["bpe_c2r4_about"]
    assert abs(16 / tot128 - g["capacity_vs_bf16_about"]) <= pr["capacity_vs_bf16_about"]


# ----------------------------------------------------------------------------
# writer + decode on small synthetic sequences

class Cache:
    """A tiny cache driven through the oracle writer."""

    def __init__(self, orc, P, bits, clip, sink, local, batch, cap):
        self.orc = orc
        self.lay = orc.Layout(P, bits, clip, sink, local)
        self.P, self.batch = P, batch
        self.max_pages = (cap + P - 1) // P
        self.pb = orc.page_bytes(self.lay)
        rng = np.random.default_rng(11)
        n_pool = batch * self.max_pages + 3
        self.bt = rng.permutation(n_pool)[: batch * self.max_pages].astype(np.int32).reshape(batch, -1)
        self.pool = np.zeros(n_pool * self.pb, np.uint8)
        self.sink = np.zeros((batch, max(sink, 1), 576), np.uint16)
        self.ring = np.zeros((batch, max(local, 1), 576), np.uint16)
        self.tail = np.zeros((batch, P, 64), np.uint16)
        self.len = np.zeros(batch, np.int32)

    def append(self, ckv, kr, counts):
        cu = wl.cu_from_counts(counts)
        self.orc.write(self.lay, np.ascontiguousarray(ckv), np.ascontiguousarray(kr), cu,
                       self.len.copy(), self.bt, self.pool, self.sink, self.ring, self.tail)
        self.len += np.asarray(counts, np.int32)

    def decode(self, ql, qr, scale):
        return self.orc.decode(self.lay, ql, qr, scale, self.pool, self.bt, self.len.copy(),
                               self.sink, self.ring, self.tail)

    def page(self, b, i):
        p = self.bt[b, i]
        return self.pool[p * self.pb:(p + 1) * self.pb]


def _rand_bf16(rng, shape, outliers=()):
    x = rng.standard_normal(shape).astype(np.float32)
    if outliers:
        x[..., list(outliers)] *= 20
    return wl.f32_to_bf16_bits(x)


def _sdpa(ql, qr, toks, scale):
    """torch scaled-dot-product attention in fp64 over token rows [L][576]."""
    H = ql.shape[0]
    q = torch.from_numpy(np.concatenate([ql, qr], -1).astype(np.float64)).view(1, H, 1, 576)
    k = torch.from_numpy(toks).view(1, 1, -1, 576).expand(1, H, -1, 576)
    v = torch.from_numpy(toks[:, :512].copy()).view(1, 1, -1, 512).expand(1, H, -1, 512)
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
    lse = torch.logsumexp((q @ k.transpose(-1, -2)).squeeze(2) * scale, dim=-1)
    return out.view(H, 512).numpy(), lse.view(H).numpy()


def test_decode_all_protected_equals_sdpa(orc):
    rng = np.random.default_rng(20)
    L, H = 37, 5
    c = Cache(orc, 16, 4, 0.0, 4, 40, 1, 64)
    ckv, kr = _rand_bf16(rng, (L, 512)), _rand_bf16(rng, (L, 64), (7, 23))
    c.append(ckv, kr, [L])
    ql, qr = _rand_bf16(rng, (1, H, 512)), _rand_bf16(rng, (1, H, 64))
    out, lse = c.decode(ql, qr, 0.07)
    toks = wl.bf16_bits_to_f32(np.concatenate([ckv, kr], -1)).astype(np.float64)
    ref, rlse = _sdpa(wl.bf16_bits_to_f32(ql[0]), wl.bf16_bits_to_f32(qr[0]), toks, 0.07)
    np.testing.assert_allclose(out[0], ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse[0], rlse, rtol=1e-12)


def _grid_tokens(rng, L, bits):
    """Tokens whose latent groups and page k_R columns sit exactly on an fp16
    grid, so quantization is lossless: INT4 grid -1 + k/8, INT2 grid -1 + k/2."""
    if bits == 4:
        lv, step = 15, 1 / 8
    else:
        lv, step = 3, 1 / 2
    k = rng.integers(0, lv + 1, (L, 512))
    # make every group hold both ends of the grid, and >= 32 channels at -1 so
    # that the 0.94-quantile clip of |x| is 1 and clips nothing
    for g in range(4):
        k[:, g * 128] = 0
        k[:, g * 128 + 1] = lv
        k[:, g * 128 + 2: g * 128 + 12] = 0
    ckv = (-1.0 + k * step).astype(np.float32)
    kk = rng.integers(0, 16, (L, 64))
    kr = (-1.0 + kk / 8.0).astype(np.float32)
    return wl.f32_to_bf16_bits(ckv), wl.f32_to_bf16_bits(kr)


@pytest.mark.parametrize("bits,clip", [(4, 0.0), (2, 0.94)])
def test_decode_exact_grid_equals_sdpa(orc, bits, clip):
    rng = np.random.default_rng(21 + bits)
    P, L, H = 16, 64, 4
    c = Cache(orc, P, bits, clip, 0, 0, 1, L)
    ckv, kr = _grid_tokens(rng, L, bits)
    # every page column of k_R holds both ends of its grid
    kr_f = wl.bf16_bits_to_f32(kr)
    for p in range(L // P):
        kr_f[p * P] = -1.0
        kr_f[p * P + 1] = 0.875
    kr = wl.f32_to_bf16_bits(kr_f)
    c.append(ckv, kr, [L])
    ql, qr = _rand_bf16(rng, (1, H, 512)), _rand_bf16(rng, (1, H, 64))
    out, lse = c.decode(ql, qr, 0.05)
    toks = wl.bf16_bits_to_f32(np.concatenate([ckv, kr], -1)).astype(np.float64)
    ref, rlse = _sdpa(wl.bf16_bits_to_f32(ql[0]), wl.bf16_bits_to_f32(qr[0]), toks, 0.05)
    np.testing.assert_allclose(out[0], ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse[0], rlse, rtol=1e-12)


def _qdq_tokens(orc, ckv, kr, L, P, bits, clip, sink, local):
    """Expected reconstructed tokens assembled from the original inputs and the
    (separately pinned) quantizer, clip and packing pieces."""
    lv = (1 << bits) - 1
    out = np.zeros((L, 576))
    x_all = wl.bf16_bits_to_f32(ckv)
    k_all = wl.bf16_bits_to_f32(kr)
    for j in range(L):
        if j < sink or j >= L - local:
            out[j, :512] = x_all[j]
            out[j, 512:] = k_all[j]
            continue
        x = x_all[j].copy()
        if clip > 0:
            cl = orc.clip_value(x, clip)
            x = np.clip(x, -cl, cl).astype(np.float32)
        for g in range(4):
            codes, sh, mh = orc.quantize_group(x[g * 128:(g + 1) * 128], lv)
            out[j, g * 128:(g + 1) * 128] = _dequant(codes, sh, mh)[0]
        p0 = (j // P) * P
        if p0 + P <= L:
            for ch in range(64):
                codes, sh, mh = orc.quantize_group(k_all[p0:p0 + P, ch].copy(), 15)
                out[j, 512 + ch] = _dequant(codes[j - p0:j - p0 + 1], sh, mh)[0][0]
        else:
            out[j, 512:] = k_all[j]
    return out


@pytest.mark.parametrize("bits,clip,sink,local,L", [
    (4, 0.0, 4, 8, 60),      # local < P-1: unprotected tokens in the unfinished page
    (2, 0.94, 4, 8, 60),
    (4, 0.0, 0, 0, 48),      # nothing protected, every page complete
    (2, 0.94, 3, 20, 41),
])
def test_decode_matches_qdq_assembly(orc, bits, clip, sink, local, L):
    rng = np.random.default_rng(30 + L + bits)
    P, H = 16, 3
    c = Cache(orc, P, bits, clip, sink, local, 1, 64)
    ckv, kr = _rand_bf16(rng, (L, 512)), _rand_bf16(rng, (L, 64), (7, 23, 39, 55))
    c.append(ckv, kr, [L])
    toks = _qdq_tokens(orc, ckv, kr, L, P, bits, clip, sink, local)
    ql, qr = _rand_bf16(rng, (1, H, 512)), _rand_bf16(rng, (1, H, 64))
    out, lse = c.decode(ql, qr, 0.07)
    ref, rlse = _sdpa(wl.bf16_bits_to_f32(ql[0]), wl.bf16_bits_to_f32(qr[0]), toks, 0.07)
    np.testing.assert_allclose(out[0], ref, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(lse[0], rlse, rtol=1e-12)


def test_decode_special_cases(orc):
    rng = np.random.default_rng(40)
    P, L, H = 16, 40, 2
    c = Cache(orc, P, 4, 0.0, 2, 5, 1, 64)
    ckv, kr = _rand_bf16(rng, (L, 512)), _rand_bf16(rng, (L, 64))
    c.append(ckv, kr, [L])
    toks = _qdq_tokens(orc, ckv, kr, L, P, 4, 0.0, 2, 5)
    zq = np.zeros((1, H, 512), np.uint16), np.zeros((1, H, 64), np.uint16)
    out, lse = c.decode(zq[0], zq[1], 0.1)
    np.testing.assert_allclose(out[0], np.tile(toks[:, :512].mean(0), (H, 1)), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[0], np.log(L), rtol=1e-14)
    # a single cached token: the output is that token
    c1 = Cache(orc, P, 4, 0.0, 0, 0, 1, 64)
    c1.append(ckv[:1], kr[:1], [1])
    ql, qr = _rand_bf16(rng, (1, H, 512)), _rand_bf16(rng, (1, H, 64))
    out1, lse1 = c1.decode(ql, qr, 0.1)
    t0 = _qdq_tokens(orc, ckv[:1], kr[:1], 1, P, 4, 0.0, 0, 0)[0]
    np.testing.assert_allclose(out1[0], np.tile(t0[:512], (H, 1)), rtol=1e-13)
    # no cached token: zero output, lse = -inf
    c0 = Cache(orc, P, 4, 0.0, 0, 0, 1, 64)
    out0, lse0 = c0.decode(ql, qr, 0.1)
    assert not out0.any() and np.all(np.isneginf(lse0))


def test_window_exit_switches_to_existing_packed_copy(orc):
    """QuantMLA Figure 8: a token leaving the recent window is read from the
    packed copy written when it arrived; a completed page never changes."""
    rng = np.random.default_rng(50)
    P, sink, local = 16, 2, 6
    c = Cache(orc, P, 4, 0.0, sink, local, 1, 96)
    ckv, kr = _rand_bf16(rng, (80, 512)), _rand_bf16(rng, (80, 64))
    c.append(ckv[:20], kr[:20], [20])
    snap = c.page(0, 0).copy()
    j = 15
    tok_before, kind_before = orc.read_token(c.lay, c.pool, c.bt, c.sink, c.ring, c.tail, 0, 20, j)
    assert kind_before == 1  # still in the window: BF16
    for step in range(20, 80):
        c.append(ckv[step:step + 1], kr[step:step + 1], [1])
        np.testing.assert_array_equal(c.page(0, 0), snap)
    tok_after, kind_after = orc.read_token(c.lay, c.pool, c.bt, c.sink, c.ring, c.tail, 0, 80, j)
    assert kind_after == 0
    expect = _qdq_tokens(orc, ckv, kr, 80, P, 4, 0.0, sink, local)[j]
    np.testing.assert_array_equal(tok_after, expect)


def test_chunked_appends_equal_one_bulk_append(orc):
    rng = np.random.default_rng(60)
    P, L = 16, 3 * 16 + 7
    ckv, kr = _rand_bf16(rng, (2 * L, 512)), _rand_bf16(rng, (2 * L, 64))
    bulk = Cache(orc, P, 2, 0.94, 4, 8, 2, 64)
    bulk.append(ckv, kr, [L, L])
    inc = Cache(orc, P, 2, 0.94, 4, 8, 2, 64)
    sizes = [1, 5, 16, 3, 17, 13]
    pos = 0
    for s in sizes:
        rows = np.concatenate([ckv[pos:pos + s], ckv[L + pos:L + pos + s]])
        rk = np.concatenate([kr[pos:pos + s], kr[L + pos:L + pos + s]])
        inc.append(rows, rk, [s, s])
        pos += s
    assert pos == L
    np.testing.assert_array_equal(inc.pool, bulk.pool)
    np.testing.assert_array_equal(inc.ring, bulk.ring)
    np.testing.assert_array_equal(inc.sink, bulk.sink)
    np.testing.assert_array_equal(inc.tail[:, : L % P], bulk.tail[:, : L % P])


# ----------------------------------------------------------------------------
# Latent transform y = bf16(fp32 fma chain of A_c x), ascending input order

def _bf16(v):
    return wl.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def _eye_bf16(dim, scale=1.0):
    a = np.zeros((dim, dim), dtype=np.float32)
    np.fill_diagonal(a, scale)
    return _bf16(a)


def _x_rows(seed, n, dim=512):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, dim)).astype(np.float32) * rng.choice([1e-3, 1.0, 30.0], (n, dim))
    x[:, ::97] = 0.0
    x[0, 5] = -0.0
    return _bf16(x)


def test_transform_identity_and_permutation(orc):
    """A_c = I returns x (a -0 input becomes +0: 0 + -0 = +0 to nearest);
    a permutation matrix permutes; 2 I doubles exactly."""
    import oracle as orc_mod
    x = _x_rows(1, 6)
    canon = np.where(x == 0x8000, np.uint16(0), x)
    assert np.array_equal(orc_mod.transform(_eye_bf16(512), x), canon)
    perm = np.random.default_rng(2).permutation(512)
    a = np.zeros((512, 512), dtype=np.float32)
    a[np.arange(512), perm] = 1.0
    assert np.array_equal(orc_mod.transform(_bf16(a), x), canon[:, perm])
    xf = wl.bf16_bits_to_f32(canon)
    assert np.array_equal(orc_mod.transform(_eye_bf16(512, 2.0), x), _bf16(2.0 * xf))


def test_transform_bf16_round_to_nearest_even(orc):
    """Three-term sums that land on, above and below bf16 midpoints (bf16 keeps
    7 fraction bits: its step at 1 is 2^-7)."""
    import oracle as orc_mod
    dim = 512
    a = np.zeros((dim, dim), dtype=np.float32)
    a[:, :3] = 1.0
    cases = [  # (x0, x1, x2, expected sum after rounding)
        (1.0, 2.0**-8, 0.0, 1.0),                              # tie, even below
        (1.0 + 2.0**-7, 2.0**-8, 0.0, 1.0 + 2.0**-6),         # tie, even above
        (1.0, 2.0**-8, 2.0**-16, 1.0 + 2.0**-7),              # just above the tie
        (1.0, 2.0**-8, -(2.0**-17), 1.0),                     # just below the tie
        (-1.0, -(2.0**-8), 0.0, -1.0),                        # negative tie
        (3.0, 2.0**-7, 0.0, 3.0),                             # tie: the step in [2, 4) is 2^-6
    ]
    x = np.zeros((len(cases), dim), dtype=np.float32)
    for i, c in enumerate(cases):
        x[i, :3] = c[:3]
    xb = _bf16(x)
    assert np.array_equal(wl.bf16_bits_to_f32(xb)[:, :3], x[:, :3])  # inputs exact in bf16
    y = wl.bf16_bits_to_f32(orc_mod.transform(_bf16(a), xb))
    assert np.array_equal(y[:, 0], np.array([c[3] for c in cases], dtype=np.float32))


def test_transform_single_precision_input_order(orc):
    """The sum runs in fp32 in ascending input order: after 2^24 every +1
    lands on a tie and rounds back to 2^24 (even), so 2^24, 510 ones and
    -2^24 sum to 0; in any exact or reordered sum they give 510."""
    import oracle as orc_mod
    dim = 512
    a = _bf16(np.ones((dim, dim), dtype=np.float32))
    x = np.ones((1, dim), dtype=np.float32)
    x[0, 0], x[0, -1] = 2.0**24, -(2.0**24)
    y = wl.bf16_bits_to_f32(orc_mod.transform(a, _bf16(x)))
    assert np.all(y == 0.0)
    x2 = x.copy()
    x2[0, 0], x2[0, 1] = -(2.0**24), 2.0**24   # cancellation first: the ones add up
    x2[0, -1] = 1.0
    y2 = wl.bf16_bits_to_f32(orc_mod.transform(a, _bf16(x2)))
    assert np.all(y2 == 510.0)


def test_transform_within_fp32_bound_of_exact(orc):
    """Against the exact product (float64: every bf16 x bf16 product is exact
    and the 512-term sum's error is far below the bound): |y - Ax| is at most
    half a bf16 step of y plus the fp32 chain's bound 512 u sum |a x|."""
    import oracle as orc_mod
    a = wl.random_orthogonal_bf16(11)
    x = _x_rows(3, 8)
    af = wl.bf16_bits_to_f32(a).astype(np.float64)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    exact = xf @ af.T
    absum = np.abs(xf) @ np.abs(af).T
    y = wl.bf16_bits_to_f32(orc_mod.transform(a, x)).astype(np.float64)
    step = np.abs(y) * 2.0**-7 + 2.0**-133
    assert np.all(np.abs(y - exact) <= 0.5 * step + 512 * 2.0**-24 * absum)
    # the transform is (nearly) orthogonal: row norms are kept to bf16 accuracy
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(xf, axis=1), rtol=2e-2)


# ----------------------------------------------------------------------------
# BF16 paged cache (the baseline of QuantMLA Table 9 caption)

def test_bf16_cache_decode_equals_sdpa(orc):
    """Ragged sequences through a permuted block table: each sequence's
    output and lse equal torch attention over its rows in order."""
    rng = np.random.default_rng(31)
    P, H = 16, 3
    lengths = [0, 1, 15, 16, 17, 40]
    max_pages = (max(lengths) + P - 1) // P
    n_pool = len(lengths) * max_pages + 3
    bt = rng.permutation(n_pool)[: len(lengths) * max_pages].astype(np.int32).reshape(len(lengths), max_pages)
    pool = np.zeros((n_pool, P, 576), np.uint16)
    ckv = _rand_bf16(rng, (sum(lengths), 512), (3, 300))
    kr = _rand_bf16(rng, (sum(lengths), 64), (9,))
    orc.append_bf16(pool, P, bt, np.zeros(len(lengths), np.int32), ckv, kr, lengths)
    ql, qr = _rand_bf16(rng, (len(lengths), H, 512)), _rand_bf16(rng, (len(lengths), H, 64))
    out, lse = orc.decode_bf16(ql, qr, 0.06, pool, P, bt, np.asarray(lengths, np.int32))
    start = 0
    for b, L in enumerate(lengths):
        if L == 0:
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        toks = wl.bf16_bits_to_f32(np.concatenate([ckv[start:start + L], kr[start:start + L]], -1))
        ref, rlse = _sdpa(wl.bf16_bits_to_f32(ql[b]), wl.bf16_bits_to_f32(qr[b]), toks.astype(np.float64), 0.06)
        np.testing.assert_allclose(out[b], ref, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse[b], rlse, rtol=1e-12)
        start += L


def test_bf16_cache_single_token_and_appends(orc):
    """One token: out is its latent row exactly and lse its scaled score.
    Rows appended in two calls land where one call puts them."""
    rng = np.random.default_rng(32)
    P = 32
    bt = np.array([[4, 1, 7]], np.int32)
    ckv, kr = _rand_bf16(rng, (70, 512)), _rand_bf16(rng, (70, 64))
    one = orc.append_bf16(np.zeros((8, P, 576), np.uint16), P, bt, np.zeros(1, np.int32), ckv, kr, [70])
    two = orc.append_bf16(np.zeros((8, P, 576), np.uint16), P, bt, np.zeros(1, np.int32), ckv[:33], kr[:33], [33])
    orc.append_bf16(two, P, bt, np.array([33], np.int32), ckv[33:], kr[33:], [37])
    np.testing.assert_array_equal(one, two)
    assert np.array_equal(one[7, 69 - 64, :512], ckv[69]) and np.array_equal(one[1, 0, 512:], kr[32])
    ql, qr = _rand_bf16(rng, (1, 2, 512)), _rand_bf16(rng, (1, 2, 64))
    out, lse = orc.decode_bf16(ql, qr, 0.1, one, P, bt, np.array([1], np.int32))
    x = wl.bf16_bits_to_f32(ckv[0]).astype(np.float64)
    k = wl.bf16_bits_to_f32(kr[0]).astype(np.float64)
    np.testing.assert_array_equal(out[0], np.broadcast_to(x, (2, 512)))
    z = 0.1 * (wl.bf16_bits_to_f32(ql[0]).astype(np.float64) @ x + wl.bf16_bits_to_f32(qr[0]).astype(np.float64) @ k)
    np.testing.assert_allclose(lse[0], z, rtol=1e-13)
