"""The no-allocation decode entry point (split partials in the library's fixed
per-GPU scratch array) against mla_lowbit_decode with a caller workspace, on
the same cache: outputs and lse must be bit-identical (same kernels, same
work split).  Two calls in a row, the second on a smaller input, so the
second reuses the scratch the first left behind."""
import math

import numpy as np
import pytest

from harness import OracleCache, compare_decode, layouts, perm_block_table, random_queries, random_tokens, say

pytestmark = pytest.mark.gpu


def _cache(torch, P, bits, clip, lengths, seed):
    from bit_kv_cache_writer_amd import mla
    glay, olay = layouts(P, bits, clip, 4, 128)
    B = len(lengths)
    max_pages = (max(lengths) + P - 1) // P
    bt, n_pool = perm_block_table(seed, B, max_pages)
    gpu = mla.DeviceCache(glay, B, max_pages, bt, n_pool)
    toks = [random_tokens(seed * 100 + b, L) for b, L in enumerate(lengths)]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    gpu.append(dev(np.concatenate([t[0] for t in toks])), dev(np.concatenate([t[1] for t in toks])), lengths)
    ref = OracleCache(olay, B, max_pages, bt, n_pool)
    ref.append(np.concatenate([t[0] for t in toks]), np.concatenate([t[1] for t in toks]), lengths)
    return gpu, ref


def _both(torch, gpu, heads, seed):
    from bit_kv_cache_writer_amd import mla
    B = gpu.batch
    ql, qr = random_queries(seed, B, heads)
    q_lat = torch.from_numpy(ql.view(np.int16)).cuda()
    q_rope = torch.from_numpy(qr.view(np.int16)).cuda()
    scale = 1.0 / math.sqrt(192.0)
    ws = gpu.workspace_bytes(heads)
    assert 0 < ws <= mla.NOALLOC_SCRATCH_BYTES  # the shape needs split partials
    out_w, lse_w = gpu.decode(q_lat, q_rope, scale)
    out_n = torch.full_like(out_w, float("nan"))
    lse_n = torch.full_like(lse_w, float("nan"))
    mla.mla_lowbit_decode_noalloc(gpu.layout, q_lat, q_rope, B, heads, scale, gpu.pool, gpu.num_pool_pages,
                                  gpu.block_table, gpu.max_pages, gpu.lengths, max(gpu.host_lengths), gpu.sink,
                                  gpu.ring, gpu.tail, out_n, lse_n)
    torch.cuda.synchronize()
    return (ql, qr, scale), (out_w.cpu().numpy(), lse_w.cpu().numpy()), (out_n.cpu().numpy(), lse_n.cpu().numpy())


def test_noalloc_equals_workspace_decode_twice():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # first call: 8 x 4096 tokens, 16 heads (several splits per sequence)
    say("noalloc", "call 1: C4R4 P128 8 x 4096, 16 heads")
    gpu, ref = _cache(torch, 128, 4, 0.0, [4096] * 8, seed=41)
    q, (ow, lw), (on, ln) = _both(torch, gpu, 16, seed=42)
    assert np.array_equal(ow, on) and np.array_equal(lw, ln)
    r_out, r_lse = ref.decode(*q[:2], q[2])
    compare_decode(on, ln, r_out, r_lse, case="noalloc call 1 (8 x 4096, 16 heads)",
                   lse_slack=ref.lse_slack(*q[:2], q[2]))
    # second call, smaller: 3 sequences of C2R4, 20 heads
    say("noalloc", "call 2: C2R4 P64 3 sequences, 20 heads")
    gpu2, ref2 = _cache(torch, 64, 2, 0.94, [1500, 700, 2100], seed=43)
    q, (ow, lw), (on, ln) = _both(torch, gpu2, 20, seed=44)
    assert np.array_equal(ow, on) and np.array_equal(lw, ln)
    r_out, r_lse = ref2.decode(*q[:2], q[2])
    compare_decode(on, ln, r_out, r_lse, case="noalloc call 2 (3 seqs, 20 heads)",
                   lse_slack=ref2.lse_slack(*q[:2], q[2]))
