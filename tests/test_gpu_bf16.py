"""GPU parity of the plain BF16 paged cache (include/mla_bf16.h) against the
CPU oracle: appended rows must be bit-exact, decode outputs within max
relative error 2e-3 per (sequence, head) row and lse within 2e-3."""
import math

import numpy as np
import pytest

from harness import compare_decode, perm_block_table, random_queries, random_tokens, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from bit_kv_cache_writer_amd import mla
    mla.lib()
    return torch


def _dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def _build(torch, P, lengths, seed, chunks=None, mult=1.0):
    """The same seeded rows appended to the GPU cache (in the given chunks)
    and to the oracle's pool."""
    import oracle
    from bit_kv_cache_writer_amd import mla
    B = len(lengths)
    max_pages = max(1, (max(lengths) + P - 1) // P)
    bt, n_pool = perm_block_table(seed, B, max_pages)
    toks = [random_tokens(seed * 1000 + b, max(L, 1)) for b, L in enumerate(lengths)]
    if mult != 1.0:
        from bit_kv_cache_writer_amd import workloads as wl
        toks = [(wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(c) * np.float32(mult)), k) for c, k in toks]
    gpu = mla.Bf16Cache(P, B, max_pages, bt, n_pool)
    ref = np.zeros((n_pool, P, 576), np.uint16)
    oracle.append_bf16(ref, P, bt, np.zeros(B, np.int32), np.concatenate([t[0][:L] for t, L in zip(toks, lengths)]),
                       np.concatenate([t[1][:L] for t, L in zip(toks, lengths)]), lengths)
    pos = [0] * B
    for counts in chunks or [lengths]:
        ckv = np.concatenate([toks[b][0][pos[b]:pos[b] + c] for b, c in enumerate(counts)])
        kr = np.concatenate([toks[b][1][pos[b]:pos[b] + c] for b, c in enumerate(counts)])
        gpu.append(_dev(torch, ckv), _dev(torch, kr), counts)
        pos = [p + c for p, c in zip(pos, counts)]
    torch.cuda.synchronize()
    return gpu, ref, bt


def _lse_slack(ql, qr, pool, bt, lengths, scale):
    """fp32 slack of the lse comparison: 2^-17 scale max_j sum_c |q_c x_jc|
    (the scores are fp32 dot products of that L1 size)."""
    from harness import LSE_FP32_FRACTION
    from bit_kv_cache_writer_amd import workloads as wl
    P = pool.shape[1]
    out = np.zeros(ql.shape[:2])
    for b, L in enumerate(lengths):
        if L == 0:
            continue
        rows = np.stack([pool[bt[b][j // P], j % P] for j in range(L)])
        x = np.abs(wl.bf16_bits_to_f32(rows).astype(np.float64))
        q = np.abs(np.concatenate([wl.bf16_bits_to_f32(ql[b]), wl.bf16_bits_to_f32(qr[b])], -1).astype(np.float64))
        out[b] = LSE_FP32_FRACTION * scale * (q @ x.T).max(axis=1)
    return out


CASES = [
    # name, P, lengths, heads
    ("p16_ragged", 16, [0, 1, 15, 16, 17, 100, 1000], 16),
    ("p64_h20", 64, [513, 2048, 3000], 20),
    ("p128_h128", 128, [300, 700], 128),
    ("p256_h7", 256, [5, 600, 256], 7),
    # one long sequence: over 32 splits, so the merge takes its many-split shape
    ("p64_b1_long", 64, [40000], 16),
    # the largest page and a single head
    ("p1024_h1", 1024, [2000, 5, 1024], 1),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bf16_cache_parity(torch_cuda, case):
    import oracle
    torch = torch_cuda
    name, P, lengths, H = case
    seed = 50 + len(name)
    say(name, "append", lengths)
    gpu, ref, bt = _build(torch, P, lengths, seed)
    np.testing.assert_array_equal(gpu.pool.cpu().numpy().view(np.uint16), ref)
    ql, qr = random_queries(seed + 1, len(lengths), H)
    scale = 1.0 / math.sqrt(192.0)
    say(name, "decode, heads", H)
    out, lse = gpu.decode(_dev(torch, ql), _dev(torch, qr), scale)
    torch.cuda.synchronize()
    r_out, r_lse = oracle.decode_bf16(ql, qr, scale, ref, P, bt, np.asarray(lengths, np.int32))
    worst = compare_decode(out.cpu().numpy(), lse.cpu().numpy(), r_out, r_lse, case=f"bf16 {name}",
                           lse_slack=_lse_slack(ql, qr, ref, bt, lengths, scale))
    say(name, f"worst row rel err {worst:.2e}")


def test_bf16_cache_chunked_appends_and_large_values(torch_cuda):
    """Rows appended over several calls equal one append; latents x3000
    (spans near the range limit) decode within the bar."""
    import oracle
    torch = torch_cuda
    lengths = [130, 77, 300]
    chunks = [[1, 0, 5], [64, 13, 100], [0, 64, 1], [65, 0, 194]]
    say("bf16 chunked appends", chunks)
    gpu, ref, bt = _build(torch, 64, lengths, 77, chunks=chunks, mult=3000.0)
    np.testing.assert_array_equal(gpu.pool.cpu().numpy().view(np.uint16), ref)
    ql, qr = random_queries(78, 3, 16)
    out, lse = gpu.decode(_dev(torch, ql), _dev(torch, qr), 0.01)
    torch.cuda.synchronize()
    r_out, r_lse = oracle.decode_bf16(ql, qr, 0.01, ref, 64, bt, np.asarray(lengths, np.int32))
    compare_decode(out.cpu().numpy(), lse.cpu().numpy(), r_out, r_lse, case="bf16 latents x3000",
                   lse_slack=_lse_slack(ql, qr, ref, bt, lengths, 0.01))
