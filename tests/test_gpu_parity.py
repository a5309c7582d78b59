"""GPU parity: the HIP writer and decode (through the C ABI) against the CPU
oracle on the same seeded inputs.  Packed codes, metadata and BF16 copies must
be bit-exact; decode outputs must be within max relative error 2e-3 per
(sequence, head) row and lse within 2e-3."""
import math

import numpy as np
import pytest

from bit_kv_cache_writer_amd import workloads as wl

from harness import (OracleCache, compare_cache, compare_decode, layouts, perm_block_table,
                      random_queries, random_tokens, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_kv_cache_writer_amd import mla
    mla.lib()
    return torch


def _to_dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _build(torch, name, P, bits, clip, sink, local, lengths, seed, chunks=None, a_c=None):
    from bit_kv_cache_writer_amd import mla
    glay, olay = layouts(P, bits, clip, sink, local)
    B = len(lengths)
    cap = max(max(lengths), 1)
    max_pages = (cap + P - 1) // P
    bt, n_pool = perm_block_table(seed, B, max_pages)
    toks = [random_tokens(seed * 1000 + b, max(L, 1)) for b, L in enumerate(lengths)]
    gpu = mla.DeviceCache(glay, B, max_pages, bt, n_pool)
    ref = OracleCache(olay, B, max_pages, bt, n_pool)
    # oracle: one bulk append
    ref_ckv = np.concatenate([t[0][:L] for t, L in zip(toks, lengths)])
    if a_c is not None:  # the oracle caches bf16(A_c x) in place of x
        import oracle
        ref_ckv = oracle.transform(a_c, ref_ckv)
    ref.append(ref_ckv, np.concatenate([t[1][:L] for t, L in zip(toks, lengths)]), lengths)
    a_dev = None if a_c is None else _to_dev(torch, a_c)
    # GPU: bulk, or the given chunk schedule (list of per-sequence count lists)
    chunks = chunks or [lengths]
    pos = [0] * B
    for counts in chunks:
        ckv = np.concatenate([toks[b][0][pos[b]:pos[b] + c] for b, c in enumerate(counts)])
        kr = np.concatenate([toks[b][1][pos[b]:pos[b] + c] for b, c in enumerate(counts)])
        say(name, "GPU append", counts[:8])
        gpu.append(_to_dev(torch, ckv), _to_dev(torch, kr), counts, a_c=a_dev)
        pos = [p + c for p, c in zip(pos, counts)]
    torch.cuda.synchronize()
    assert pos == list(lengths)
    return gpu, ref


CASES = [
    # name, P, bits, clip, sink, local, lengths, heads
    ("tiny_c4r4", 64, 4, 0.0, 4, 32, [256], 16),
    ("tiny_L250_unfinished_page", 64, 4, 0.0, 4, 32, [250], 16),
    ("c2r4_p128_ragged", 128, 2, 0.94, 4, 128, [700, 1000, 129, 5], 20),
    ("c4r4_p128_ragged", 128, 4, 0.0, 4, 128, [0, 1, 127, 128, 129, 600, 1300], 16),
    ("c4r4_p64_h128", 64, 4, 0.0, 4, 128, [300, 513], 128),
    ("c2r4_p64_h64", 64, 2, 0.94, 4, 128, [1000, 2000], 64),
    ("c4r4_p32_noprot_h7", 32, 4, 0.0, 0, 0, [64, 95, 200], 7),
    ("c2r4_p256_allprot", 256, 2, 0.94, 8, 512, [300, 40], 16),
    ("c4r4_p64_local8", 64, 4, 0.0, 2, 8, [150, 64, 63], 33),
    # one long sequence: over 128 splits, so the merge loads the splits'
    # (max, sum) blocks in several rounds
    ("c4r4_p128_b1_long", 128, 4, 0.0, 4, 128, [40000], 16),
    # the layout's largest protection: sink 64 and a 4096-token window, one
    # sequence past both and one inside them
    ("c2r4_p64_maxwin", 64, 2, 0.94, 64, 4096, [4500, 3000], 16),
    # 2-bit latents without the clip (two tokens a wave): odd token counts per
    # page and wave, sink and ring copies from either half-wave
    ("c2r4_p64_noclip_ragged", 64, 2, 0.0, 4, 32, [1, 2, 63, 64, 65, 191, 700], 16),
    ("c4r4_p32_odd_h20", 32, 4, 0.0, 3, 5, [33, 15, 97], 20),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_write_and_decode_parity(torch_cuda, case):
    torch = torch_cuda
    name, P, bits, clip, sink, local, lengths, H = case
    gpu, ref = _build(torch, name, P, bits, clip, sink, local, lengths, seed=len(name))
    say(name, "compare cache bytes")
    compare_cache(gpu, ref)
    ql, qr = random_queries(7 + H, len(lengths), H)
    scale = 1.0 / math.sqrt(192.0)
    say(name, "GPU decode", "heads", H)
    out, lse = gpu.decode(_to_dev(torch, ql), _to_dev(torch, qr), scale)
    torch.cuda.synchronize()
    r_out, r_lse = ref.decode(ql, qr, scale)
    worst = compare_decode(out.cpu().numpy(), lse.cpu().numpy(), r_out, r_lse, case=name,
                           lse_slack=ref.lse_slack(ql, qr, scale))
    say(name, f"worst row rel err {worst:.2e}")


def test_chunked_appends_equal_bulk(torch_cuda):
    """Token-by-token and ragged chunked appends (the decode-step writer) give
    the same bytes as the oracle's single append."""
    torch = torch_cuda
    lengths = [200, 77, 130]
    sched = [[1, 1, 1]] * 3 + [[60, 0, 5], [1, 70, 0], [64, 2, 64], [0, 1, 58]]
    done = np.sum(sched, axis=0)
    sched.append([int(L - d) for L, d in zip(lengths, done)])
    gpu, ref = _build(torch, "chunked_c2r4", 64, 2, 0.94, 4, 32, lengths, seed=91, chunks=sched)
    compare_cache(gpu, ref)
    gpu2, ref2 = _build(torch, "chunked_c4r4", 32, 4, 0.0, 4, 8, lengths, seed=92,
                        chunks=[[1, 1, 1]] * 7 + [[L - 7 for L in lengths]])
    compare_cache(gpu2, ref2)
    gpu3, ref3 = _build(torch, "chunked_c2r4_noclip", 64, 2, 0.0, 4, 32, lengths, seed=93, chunks=sched)
    compare_cache(gpu3, ref3)


TRANSFORM_CASES = [
    # name, P, bits, clip, sink, local, lengths, chunk schedule (None = one bulk append);
    # without the clip the writer runs one workgroup per (page, latent group),
    # with it one per page
    ("xf_c4r4_p64_steps", 64, 4, 0.0, 4, 32, [3, 70, 130, 9],
     [[1, 1, 1, 1]] * 3 + [[0, 67, 127, 6]]),
    ("xf_c2r4_p128_bulk", 128, 2, 0.94, 4, 128, [300, 5, 129], None),
    ("xf_c4r4_p32_noprot", 32, 4, 0.0, 0, 0, [64, 33], [[1, 1], [20, 0], [43, 32]]),
    # INT2 latent without the clip: the per-group workgroups, 2-bit codes
    ("xf_c2r4_p64_noclip", 64, 2, 0.0, 4, 32, [150, 64, 1], [[1, 64, 1], [149, 0, 0]]),
    # the largest page: 300-token calls into 256-token pages, one page left
    # one token short of full
    ("xf_c4r4_p256_bulk", 256, 4, 0.0, 4, 128, [600, 255, 256, 1], [[300, 255, 0, 1], [300, 0, 256, 0]]),
]


@pytest.mark.parametrize("case", TRANSFORM_CASES, ids=[c[0] for c in TRANSFORM_CASES])
def test_transformed_writer_parity(torch_cuda, case):
    """The writer with the latent transform A_c inside it (a seeded random
    orthogonal matrix) caches, bit for bit, what the oracle caches for the
    rows bf16(A_c x); decode over that cache matches the oracle's."""
    torch = torch_cuda
    name, P, bits, clip, sink, local, lengths, chunks = case
    a_c = wl.random_orthogonal_bf16(len(name))
    gpu, ref = _build(torch, name, P, bits, clip, sink, local, lengths, seed=len(name) + 500,
                      chunks=chunks, a_c=a_c)
    say(name, "compare cache bytes")
    compare_cache(gpu, ref)
    ql, qr = random_queries(31, len(lengths), 16)
    scale = 1.0 / math.sqrt(192.0)
    say(name, "GPU decode")
    out, lse = gpu.decode(_to_dev(torch, ql), _to_dev(torch, qr), scale)
    torch.cuda.synchronize()
    r_out, r_lse = ref.decode(ql, qr, scale)
    worst = compare_decode(out.cpu().numpy(), lse.cpu().numpy(), r_out, r_lse, case=name,
                           lse_slack=ref.lse_slack(ql, qr, scale))
    say(name, f"worst row rel err {worst:.2e}")


def test_transformed_writer_identity_equals_plain(torch_cuda):
    """A_c = I through the transforming writer gives the plain writer's bytes
    (the inputs hold no -0, which the fma chain would turn into +0)."""
    torch = torch_cuda
    lengths = [150, 64, 1]
    eye = np.zeros((512, 512), np.float32)
    np.fill_diagonal(eye, 1.0)
    a_c = wl.f32_to_bf16_bits(eye)
    gpu_t, ref = _build(torch, "xf_identity", 64, 4, 0.0, 4, 32, lengths, seed=77, a_c=a_c)
    gpu_p, _ = _build(torch, "xf_identity_plain", 64, 4, 0.0, 4, 32, lengths, seed=77)
    compare_cache(gpu_t, ref)
    for a, b in ((gpu_t.pool, gpu_p.pool), (gpu_t.sink, gpu_p.sink), (gpu_t.ring, gpu_p.ring),
                 (gpu_t.tail, gpu_p.tail)):
        assert torch.equal(a, b)


def test_transformed_writer_rejects_null_matrix(torch_cuda):
    from bit_kv_cache_writer_amd import mla
    torch = torch_cuda
    glay, _ = layouts(64, 4, 0.0, 4, 32)
    c = mla.DeviceCache(glay, 1, 1, [[0]], 1)
    x = torch.zeros((1, 512), dtype=torch.int16, device="cuda")
    k = torch.zeros((1, 64), dtype=torch.int16, device="cuda")
    cu = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    with pytest.raises(mla.MlaError):
        mla.mla_lowbit_write_transformed(glay, None, x, k, cu, c.lengths, 1, 1, 1, c.block_table, 1, 1,
                                         c.pool, c.sink, c.ring, c.tail)


def test_decode_edge_inputs(torch_cuda):
    """Constant groups, all-zero tokens, bf16 subnormals, large outliers and
    codes on exact rounding ties."""
    torch = torch_cuda
    from bit_kv_cache_writer_amd import mla
    P, L = 64, 192
    ckv, kr = random_tokens(5, L)
    ckv[10] = 0
    ckv[11] = wl.f32_to_bf16_bits(np.full(512, 0.3, np.float32))
    ckv[12, :128] = wl.f32_to_bf16_bits(np.full(128, -2.5, np.float32))
    ckv[13] = wl.f32_to_bf16_bits((np.arange(512) % 7 - 3).astype(np.float32) * 1e-39)
    ckv[14, 5] = wl.f32_to_bf16_bits(np.float32(3000.0))
    # exact ties: groups whose step is 1 or 2 with values on the half-integers
    # of the quotient (every code a round-half-to-even case, which the writer
    # settles with the IEEE division), and a k_R channel of the first page
    # likewise
    half = np.concatenate([[0.0, 15.0], np.arange(0.5, 15.0, 1.0)])
    tie = np.resize(half, 128).astype(np.float32)
    ckv[15] = wl.f32_to_bf16_bits(np.concatenate([tie, 2.0 * tie, tie - 8.0, -2.0 * tie]))
    ckv[16] = wl.f32_to_bf16_bits(np.concatenate([tie[::-1], tie, 0.25 * tie, tie + 0.5]))
    kr[0:64, 9] = wl.f32_to_bf16_bits(np.resize(half, 64).astype(np.float32))
    kr[20:40, 3] = wl.f32_to_bf16_bits(np.float32(-0.0))
    for bits, clip in ((4, 0.0), (2, 0.94)):
        glay, olay = layouts(P, bits, clip, 2, 16)
        bt, n_pool = perm_block_table(3, 1, 3)
        gpu = mla.DeviceCache(glay, 1, 3, bt, n_pool)
        ref = OracleCache(olay, 1, 3, bt, n_pool)
        ref.append(ckv, kr, [L])
        say("edge inputs", bits)
        gpu.append(_to_dev(torch, ckv), _to_dev(torch, kr), [L])
        torch.cuda.synchronize()
        compare_cache(gpu, ref)
        ql, qr = random_queries(8, 1, 16)
        out, lse = gpu.decode(_to_dev(torch, ql), _to_dev(torch, qr), 0.07)
        torch.cuda.synchronize()
        r_out, r_lse = ref.decode(ql, qr, 0.07)
        compare_decode(out.cpu().numpy(), lse.cpu().numpy(), r_out, r_lse, case=f"edge_inputs_c{bits}r4",
                       lse_slack=ref.lse_slack(ql, qr, 0.07))


def _clip_rows(seed, n):
    """Latent rows that stress the clip's order statistics: ties, constant
    and all-zero rows, a single non-zero value, eight large values in one
    lane's channels, wide exponent spreads, bf16 subnormals, two-valued and
    all-negative rows, and plain Gaussian rows between them."""
    rng = np.random.default_rng(seed)
    rows = []
    for i in range(n):
        k = i % 12
        x = rng.standard_normal(512)
        if k == 1:
            x = rng.integers(-3, 4, 512).astype(np.float64)
        elif k == 2:
            x = np.full(512, 1.5)
        elif k == 3:
            x = np.zeros(512)
            x[rng.integers(0, 512)] = 2.0
        elif k == 4:
            x = np.zeros(512)
        elif k == 5:
            x[:8] *= 1000.0  # lane 0 holds all eight
        elif k == 6:
            x = rng.choice([-1.0, 1.0], 512) * 2.0 ** rng.integers(-40, 15, 512)
        elif k == 7:
            x = (np.arange(512) % 9 - 4) * 1e-39 + (rng.random(512) < 0.1) * rng.standard_normal(512)
        elif k == 8:
            x = np.where(rng.random(512) < 0.5, 0.75, -3.25)
        elif k == 9:
            x = -np.abs(x) * 40.0
        elif k == 10:
            x = np.linspace(-300.0, 300.0, 512)[rng.permutation(512)]
        rows.append(x.astype(np.float32))
    return wl.f32_to_bf16_bits(np.stack(rows))


# quantiles whose search starts from columns 0, 1, 4, 5 and 7 of the lanes'
# sorted keys (the lower rank's column), both ends, and the 4-bit latent
CLIP_QS = [(2, 0.94), (2, 0.5), (2, 0.999), (2, 1e-4), (2, 1.0), (2, 0.87), (2, 0.3), (4, 0.94)]


@pytest.mark.parametrize("bits,q", CLIP_QS, ids=[f"c{b}r4_q{q}" for b, q in CLIP_QS])
def test_clip_order_statistics(torch_cuda, bits, q):
    """The clip value of every token (and so its codes and metadata) is
    bit-exact on rows built to break an order-statistic search."""
    torch = torch_cuda
    from bit_kv_cache_writer_amd import mla
    P, L = 32, 80
    _, kr = random_tokens(17, L)
    ckv = _clip_rows(18, L)
    glay, olay = layouts(P, bits, q, 2, 16)
    bt, n_pool = perm_block_table(4, 1, 3)
    gpu = mla.DeviceCache(glay, 1, 3, bt, n_pool)
    ref = OracleCache(olay, 1, 3, bt, n_pool)
    ref.append(ckv, kr, [L])
    say("clip order statistics", bits, q)
    gpu.append(_to_dev(torch, ckv), _to_dev(torch, kr), [L])
    torch.cuda.synchronize()
    compare_cache(gpu, ref)


# --------------------------------------------------------------------------
# the configurations at their full sizes, in the launch configuration the
# benchmark times; sampled sequences (and, for the many-head ones, a subset
# of heads) are decoded by the oracle one by one, and the cache bytes of the
# sampled sequences (of every sequence where cache_all) are compared


def _full_size(torch, w, decode_seqs, heads_sub, cache_all=False, latent_mult=1.0, tag=""):
    from bit_kv_cache_writer_amd import mla
    name = w.name + tag
    glay, olay = layouts(w.page_size, w.latent_bits, w.clip_q, w.sink, w.local)
    max_pages = w.pages_per_seq()
    bt, n_pool = wl.block_table(w, max_pages)
    gpu = mla.DeviceCache(glay, w.batch, max_pages, bt, n_pool)
    n = w.seqlen
    ckv_d = torch.empty((w.batch * n, 512), dtype=torch.int16, device="cuda")
    kr_d = torch.empty((w.batch * n, 64), dtype=torch.int16, device="cuda")
    say(name, "generate inputs", w.batch, "x", n, "latent x", latent_mult)
    for b in range(w.batch):
        c, k = wl.seq_tokens(w, b, latent_mult=latent_mult)
        ckv_d[b * n:(b + 1) * n] = _to_dev(torch, c)
        kr_d[b * n:(b + 1) * n] = _to_dev(torch, k)
    say(name, "GPU bulk write")
    gpu.append(ckv_d, kr_d, [n] * w.batch)
    del ckv_d, kr_d
    ql, qr = wl.queries(w)
    say(name, "GPU decode")
    out, lse = gpu.decode(_to_dev(torch, ql), _to_dev(torch, qr), w.softmax_scale)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    if cache_all:  # every sequence's bytes, from one oracle append of the whole batch
        say(name, "oracle cache of all", w.batch, "sequences")
        ref = OracleCache(olay, w.batch, max_pages, bt, n_pool)
        toks = [wl.seq_tokens(w, b, latent_mult=latent_mult) for b in range(w.batch)]
        ref.append(np.concatenate([t[0] for t in toks]), np.concatenate([t[1] for t in toks]), [n] * w.batch)
        del toks
        compare_cache(gpu, ref)
        del ref
    pool = gpu.pool.cpu().numpy()
    ring, sink, tail = (gpu.ring.cpu().numpy().view(np.uint16), gpu.sink.cpu().numpy().view(np.uint16),
                        gpu.tail.cpu().numpy().view(np.uint16))
    hs = list(range(w.heads)) if heads_sub is None else heads_sub
    for b in decode_seqs:
        say(name, "oracle sequence", b)
        ref = OracleCache(olay, 1, max_pages, bt[b:b + 1], n_pool)
        c, k = wl.seq_tokens(w, b, latent_mult=latent_mult)
        ref.append(c, k, [n])

        class View:  # the GPU cache restricted to sequence b
            pass
        v = View()
        v.pool = torch.from_numpy(pool)
        v.sink = torch.from_numpy(sink[b:b + 1].view(np.int16))
        v.ring = torch.from_numpy(ring[b:b + 1].view(np.int16))
        v.tail = torch.from_numpy(tail[b:b + 1].view(np.int16))
        compare_cache(v, ref)
        qlb, qrb = np.ascontiguousarray(ql[b:b + 1, hs]), np.ascontiguousarray(qr[b:b + 1, hs])
        r_out, r_lse = ref.decode(qlb, qrb, w.softmax_scale)
        worst = compare_decode(out[b:b + 1, hs], lse[b:b + 1, hs], r_out, r_lse, seqs=[b],
                               case=f"{name} seq {b}", lse_slack=ref.lse_slack(qlb, qrb, w.softmax_scale))
        say(name, f"seq {b} worst row rel err {worst:.2e}")


FULL = [("tiny_c4r4", [0], None, True), ("c4r4_h16_b8", [0, 7], None, False),
        ("c4r4_h16_b32", [5, 31], None, True), ("c2r4_h20", [3], None, True),
        ("c4r4_h128", [17], [0, 1, 64, 127], False), ("c2r4_h64_long", [2], [0, 33, 63], False)]


@pytest.mark.parametrize("wname,seqs,heads_sub,cache_all", FULL, ids=[f[0] for f in FULL])
def test_full_size_sampled(torch_cuda, wname, seqs, heads_sub, cache_all):
    _full_size(torch_cuda, wl.WORKLOADS[wname], seqs, heads_sub, cache_all=cache_all)


# Large latent magnitudes in the same launch configurations: C2R4 latents
# x300 and x3000 (clip on, and a clip-free variant) and C4R4 latents x1500
# (group spans of several thousand, so fp16 weights p s_g would pass the fp16
# range without the scale headroom of the running max).
LARGE = [("c2r4_h20", 300.0, None, [3, 12], [0, 7, 19]),
         ("c2r4_h20", 3000.0, None, [5], [0, 11, 19]),
         ("c2r4_h64_long", 3000.0, 0.0, [1], [0, 40, 63]),
         ("c4r4_h16_b32", 1500.0, None, [0, 17], None),
         ("c4r4_h128", 1500.0, None, [9], [0, 77, 127])]


@pytest.mark.parametrize("wname,mult,clip,seqs,heads_sub", LARGE,
                         ids=[f"{w}_x{int(m)}" + ("_noclip" if c == 0.0 else "") for w, m, c, _, _ in LARGE])
def test_large_latents(torch_cuda, wname, mult, clip, seqs, heads_sub):
    import dataclasses
    w = wl.WORKLOADS[wname]
    tag = f"_x{int(mult)}"
    if clip is not None:
        w = dataclasses.replace(w, clip_q=clip)
        tag += "_noclip"
    _full_size(torch_cuda, w, seqs, heads_sub, latent_mult=mult, tag=tag)
