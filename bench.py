"""Benchmark: one MLA decode step over the dual-path low-bit cache, per layer.

A step is what one decode step of a model does to every layer's cache: the
fused writer appends the incoming token of each sequence (its latent and
positional key are quantized and packed; this token completes a cache page,
so the page's k_R is quantized too) and the decode attends over the N cached
tokens.  The step is repeated over `--layers` distinct caches so that the
256 MB Infinity Cache cannot hold them (the packed bytes of all layers exceed
1 GB).  The reported value is the decode's microseconds per layer (attention
and split merge, timed with events on the launch stream); the writer's share
and the whole step are reported beside it.

`--calibrate-copy` instead times a plain 1 GiB device copy (the reference
kernel for scaling the FETCH_SIZE / WRITE_SIZE counters to bytes).

Workload (the headline; the largest configuration): C4R4 decode, 128 heads,
latent 512 + rope 64, batch 64 x 32768 cached tokens, page 64, sink 4 + local
128 in BF16 (synthetic, seeded inputs); 64 new tokens per step.  The same run
also times every other workload (inputs drawn on the GPU, same
distributions) into the line's "configs" table, and measures the HBM read,
device copy and fp16 matrix-core rates the GPU sustains ("probes").

Prints one JSON line.  Run on one GPU: python bench.py [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak
FLOPS_PER_TOKEN_HEAD = 2 * 576 + 2 * 512  # QK over 576 channels + PV over 512
PROFILES = os.path.join(ROOT, "profiles")
# the decode translation unit: its source and the headers it includes
DECODE_SRCS = [os.path.join(ROOT, "bit_kv_cache_writer_amd", "csrc", f)
               for f in ("decode.hip", "decode_plan.h", "decode_bf16.h", "geometry.h")]


def decode_source_sha256() -> str:
    """sha256 over the decode sources in a fixed order (a profile taken with
    other sources no longer describes the kernels)."""
    import hashlib
    h = hashlib.sha256()
    for path in DECODE_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per decode call from the committed counter summary, or None
    when there is none or the decode source changed since it was taken."""
    path = os.path.join(PROFILES, f"decode_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("decode_source_sha256") != decode_source_sha256() or "traffic_bytes_per_call" not in fields:
        return None
    return int(float(fields["traffic_bytes_per_call"]))


def calibrate_copy() -> int:
    """Plain device copy of known size (1 GiB read + 1 GiB written), 5 times."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": round(ms, 4),
                      "gbs_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)
    return 0


def algorithmic_decode_bytes(w, L: int) -> dict:
    """Bytes the decode must move for one sequence of L tokens (layout sizes:
    C4R4 304 B / C2R4 176 B per packed token, 256 B k_R metadata per page read,
    1152 B per BF16 token, 1152 B of queries and 2052 B of output per head)."""
    lat_row = 512 * w.latent_bits // 8
    per_packed = lat_row + 16 + 32
    lo_p = min(w.sink, L)
    full = (L // w.page_size) * w.page_size
    hi_p = max(lo_p, min(L - w.local, full))
    n_packed = hi_p - lo_p
    pages = 0 if n_packed == 0 else (hi_p - 1) // w.page_size - lo_p // w.page_size + 1
    n_bf16 = L - n_packed
    cache = n_packed * per_packed + pages * 256 + n_bf16 * 1152
    return {"cache": cache, "q": w.heads * 1152, "out": w.heads * 2052,
            "total": cache + w.heads * 1152 + w.heads * 2052, "packed_tokens": n_packed}


def cpu_baseline(w, n_seq_sample: int, budget_s: float = 12.0) -> dict:
    """The CPU oracle doing the same work for a sample of sequences: the
    decode over the N cached tokens (microseconds per layer for the whole
    batch) and the one-token append before it.  Timed on one thread (a
    budget-bounded sample of sequences, scaled to the batch) and, as the
    reported value, on T host threads decoding T sequences at once (the oracle
    is unchanged; its C entry points run outside the interpreter lock), scaled
    by ceil(batch / T)."""
    import concurrent.futures as cf

    import oracle
    from bit_kv_cache_writer_amd import workloads as wl

    olay = oracle.Layout(w.page_size, w.latent_bits, w.clip_q, w.sink, w.local)
    max_pages = w.pages_per_seq()
    pb = oracle.page_bytes(olay)
    ql, qr = wl.queries(w)
    n = w.seqlen
    threads = max(1, min(16, os.cpu_count() or 1, w.batch))
    built = {}

    def build(b):
        c, k = wl.seq_tokens(w, b)
        bt = np.arange(max_pages, dtype=np.int32).reshape(1, max_pages)
        pool = np.zeros(max_pages * pb, np.uint8)
        sink = np.zeros((1, max(w.sink, 1), 576), np.uint16)
        ring = np.zeros((1, max(w.local, 1), 576), np.uint16)
        tail = np.zeros((1, w.page_size, 64), np.uint16)
        oracle.write(olay, c[: n - 1], k[: n - 1], np.array([0, n - 1], np.int32),
                     np.zeros(1, np.int32), bt, pool, sink, ring, tail)
        t0 = time.perf_counter()
        oracle.write(olay, np.ascontiguousarray(c[n - 1:]), np.ascontiguousarray(k[n - 1:]),
                     np.array([0, 1], np.int32), np.array([n - 1], np.int32), bt, pool, sink, ring, tail)
        built[b] = (bt, pool, sink, ring, tail)
        return time.perf_counter() - t0

    def dec(b):
        bt, pool, sink, ring, tail = built[b]
        t0 = time.perf_counter()
        oracle.decode(olay, np.ascontiguousarray(ql[b:b + 1]), np.ascontiguousarray(qr[b:b + 1]),
                      w.softmax_scale, pool, bt, np.array([n], np.int32), sink, ring, tail)
        return time.perf_counter() - t0

    t_dec, t_app, done = 0.0, 0.0, 0
    for b in range(n_seq_sample):
        t_app += build(b)
        t_dec += dec(b)
        done += 1
        if t_app + t_dec > budget_s:
            break
    scale1 = w.batch / done
    for b in range(done, threads):
        build(b)
    with cf.ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(dec, range(threads)))
        wall = time.perf_counter() - t0
    rounds = -(-w.batch // threads)
    return {"value": wall * rounds * 1e6, "unit": "us/layer", "cores": threads, "kind": "oracle",
            "sample": f"{threads} sequences decoded at once on {threads} threads (fp64 C oracle, each over "
                      f"{n} cached tokens), scaled x{rounds} to {w.batch} sequences; one thread: "
                      f"{done} of {w.batch} sequences, scaled x{scale1:.1f}",
            "single_thread_us_per_layer": t_dec * scale1 * 1e6,
            "append_us_per_layer": t_app * scale1 * 1e6, "sample_seconds": round(t_app + t_dec + wall, 3)}


def sweep(steps: int) -> int:
    """Context sweep (timing only; parity is covered by the tests): C4R4
    decode, 16 heads, page 128, sink 4 + local 128, batch 1 and 8, N = 1K to
    1M cached tokens.  Inputs are drawn on the GPU from a seeded generator
    (N(0,1) latent and queries, k_R N(0,1) with channels 7, 23, 39, 55 x20,
    rounded to bf16); each configuration uses enough layer caches for >= 1 GB
    of packed pages.  One JSON line per configuration."""
    import torch

    from bit_kv_cache_writer_amd import mla

    mla.lib()
    lay = mla.Layout(128, 4, 0.0, 4, 128)
    page_bytes = mla.mla_lowbit_layout_query(lay)["page_bytes"]
    heads, scale = 16, 1.0 / math.sqrt(192.0)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    outl = torch.ones(64, device="cuda")
    outl[[7, 23, 39, 55]] = 20.0

    def bf16_rows(n, width, mult=None):
        x = torch.randn((n, width), generator=gen, device="cuda", dtype=torch.float32)
        if mult is not None:
            x *= mult
        return x.to(torch.bfloat16).view(torch.int16)

    class W:  # the shape algorithmic_decode_bytes reads
        latent_bits, page_size, sink, local = 4, 128, 4, 128

    for B in (1, 8):
        for N in (1024, 4096, 16384, 65536, 262144, 1048576):
            W.heads = heads
            max_pages = (N + 127) // 128
            rng = np.random.default_rng(np.random.SeedSequence([7, B, N]))
            n_pool = int(math.ceil(B * max_pages * 1.25))
            bt = rng.permutation(n_pool)[: B * max_pages].astype(np.int32).reshape(B, max_pages)
            layers = min(64, max(2, math.ceil(1.0e9 / (B * max_pages * page_bytes))))
            caches = []
            for _ in range(layers):
                c = mla.DeviceCache(lay, B, max_pages, bt, n_pool)
                done = 0
                while done < N:
                    t = min(65536, N - done)
                    c.append(bf16_rows(B * t, 512), bf16_rows(B * t, 64, outl), [t] * B)
                    done += t
                caches.append(c)
            q_lat = bf16_rows(B * heads, 512).view(B, heads, 512).contiguous()
            q_rope = bf16_rows(B * heads, 64).view(B, heads, 64).contiguous()
            stream = torch.cuda.current_stream()
            for c in caches:
                c.decode(q_lat, q_rope, scale, stream=stream)
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(steps * layers)]
            for st in range(steps):
                for li, c in enumerate(caches):
                    e = evs[st * layers + li]
                    e[0].record(stream)
                    c.decode(q_lat, q_rope, scale, stream=stream)
                    e[1].record(stream)
            torch.cuda.synchronize()
            us = float(np.mean([a.elapsed_time(b) for a, b in evs]) * 1000.0)
            alg = algorithmic_decode_bytes(W, N)
            byts = alg["total"] * B
            gbs = byts / (us * 1e-6) / 1e9
            print(json.dumps({"sweep": "C4R4 decode, 16 heads, page 128, sink 4 + local 128",
                              "batch": B, "cached_tokens": N, "layers": layers, "decode_us": round(us, 3),
                              "algorithmic_bytes": byts, "hbm_gbs": round(gbs, 1),
                              "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                              "workspace_bytes": mla.mla_lowbit_decode_workspace(lay, B, heads, N)}), flush=True)
            del caches
            torch.cuda.empty_cache()
    return 0


def bf16_compare(steps: int) -> int:
    """Low-bit cache against the plain BF16 paged cache (QuantMLA Table 9
    caption: BF16 with native partitioning; Delta = t_low / t_BF16 - 1), timing
    only (parity of both is covered by the tests).  (1) Context sweep: C4R4
    page 128 sink 4 + local 128 against BF16 page 64, 16 heads, batch 1 and 8,
    N = 1K to 1M; (2) the six workloads at their shapes (BF16 page = the
    workload's page).  Inputs drawn on the GPU (N(0,1) latent and queries,
    k_R N(0,1) with channels 7, 23, 39, 55 x20, bf16); each side gets enough
    layer caches for >= 1 GB (at least 2).  One JSON line per configuration."""
    import torch

    from bit_kv_cache_writer_amd import mla
    from bit_kv_cache_writer_amd import workloads as wl

    mla.lib()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    outl = torch.ones(64, device="cuda")
    outl[[7, 23, 39, 55]] = 20.0

    def bf16_rows(n, width, mult=None):
        out = torch.empty((n, width), dtype=torch.int16, device="cuda")
        for a in range(0, n, 1 << 21):
            e = min(n, a + (1 << 21))
            x = torch.randn((e - a, width), generator=gen, device="cuda", dtype=torch.float32)
            if mult is not None:
                x *= mult
            out[a:e] = x.to(torch.bfloat16).view(torch.int16)
        return out

    def timed(calls):
        stream = torch.cuda.current_stream()
        for c in calls:
            c(stream)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps * len(calls))]
        for st in range(steps):
            for i, c in enumerate(calls):
                e = evs[st * len(calls) + i]
                e[0].record(stream)
                c(stream)
                e[1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]) * 1000.0)

    def one(tag, B, N, H, P_low, bits, clip, sink, local, P_bf, scale):
        lay = mla.Layout(P_low, bits, clip, sink, local)
        page_bytes = mla.mla_lowbit_layout_query(lay)["page_bytes"]
        rng = np.random.default_rng(np.random.SeedSequence([11, B, N, H]))
        q_lat = bf16_rows(B * H, 512).view(B, H, 512).contiguous()
        q_rope = bf16_rows(B * H, 64).view(B, H, 64).contiguous()
        # low-bit side
        mp = (N + P_low - 1) // P_low
        n_pool = int(math.ceil(B * mp * 1.25))
        bt = rng.permutation(n_pool)[: B * mp].astype(np.int32).reshape(B, mp)
        layers = min(64, max(2, math.ceil(1.0e9 / (B * mp * page_bytes))))
        caches = []
        for _ in range(layers):
            c = mla.DeviceCache(lay, B, mp, bt, n_pool)
            done = 0
            while done < N:
                t = min(1 << 17, N - done)
                c.append(bf16_rows(B * t, 512), bf16_rows(B * t, 64, outl), [t] * B)
                done += t
            caches.append(c)
        t_low = timed([lambda s, c=c: c.decode(q_lat, q_rope, scale, stream=s) for c in caches])
        alg = algorithmic_decode_bytes(type("W", (), {"latent_bits": bits, "page_size": P_low, "sink": sink,
                                                      "local": local, "heads": H})(), N)
        low_bytes = alg["total"] * B
        del caches
        torch.cuda.empty_cache()
        # BF16 side
        mpb = (N + P_bf - 1) // P_bf
        n_pool_b = int(math.ceil(B * mpb * 1.25))
        btb = rng.permutation(n_pool_b)[: B * mpb].astype(np.int32).reshape(B, mpb)
        bf_layer = B * N * 1152
        layers_b = min(64, max(2, math.ceil(1.0e9 / bf_layer)))
        bcs = []
        for _ in range(layers_b):
            c = mla.Bf16Cache(P_bf, B, mpb, btb, n_pool_b)
            done = 0
            while done < N:
                t = min(1 << 17, N - done)
                c.append(bf16_rows(B * t, 512), bf16_rows(B * t, 64, outl), [t] * B)
                done += t
            bcs.append(c)
        t_bf = timed([lambda s, c=c: c.decode(q_lat, q_rope, scale, stream=s) for c in bcs])
        del bcs
        torch.cuda.empty_cache()
        gbs = bf_layer / (t_bf * 1e-6) / 1e9
        print(json.dumps({"compare": tag, "batch": B, "cached_tokens": N, "heads": H,
                          "lowbit": f"{'C4R4' if bits == 4 else 'C2R4'} page {P_low} sink {sink} local {local}",
                          "bf16_page": P_bf, "lowbit_us": round(t_low, 3), "bf16_us": round(t_bf, 3),
                          "delta_pct": round((t_low / t_bf - 1.0) * 100.0, 1),
                          "speedup_vs_bf16": round(t_bf / t_low, 3),
                          "lowbit_hbm_gbs": round(low_bytes / (t_low * 1e-6) / 1e9, 1),
                          "bf16_bytes": bf_layer, "bf16_hbm_gbs": round(gbs, 1),
                          "bf16_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                          "layers": [layers, layers_b]}), flush=True)

    for B in (1, 8):
        for N in (1024, 4096, 16384, 65536, 262144, 1048576):
            one("context sweep", B, N, 16, 128, 4, 0.0, 4, 128, 64, 1.0 / math.sqrt(192.0))
    for name, w in wl.WORKLOADS.items():
        one(name, w.batch, w.seqlen, w.heads, w.page_size, w.latent_bits, w.clip_q, w.sink, w.local,
            w.page_size, w.softmax_scale)
    return 0


def ragged(steps: int) -> int:
    """Ragged decode and chunked prefill (timing only; parity of both is
    covered by the tests): (1) C4R4 decode, 16 heads, page 128, sink 4 + local
    128, 32 sequences with seeded lengths uniform in [1024, 8192]; (2) the
    writer appending four 128K-token prompts in 8K-token chunks.  Inputs drawn
    on the GPU from a seeded generator.  One JSON line each."""
    import torch

    from bit_kv_cache_writer_amd import mla

    mla.lib()
    lay = mla.Layout(128, 4, 0.0, 4, 128)
    page_bytes = mla.mla_lowbit_layout_query(lay)["page_bytes"]
    heads, scale = 16, 1.0 / math.sqrt(192.0)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    outl = torch.ones(64, device="cuda")
    outl[[7, 23, 39, 55]] = 20.0

    def bf16_rows(n, width, mult=None):
        x = torch.randn((n, width), generator=gen, device="cuda", dtype=torch.float32)
        if mult is not None:
            x *= mult
        return x.to(torch.bfloat16).view(torch.int16)

    class W:  # the shape algorithmic_decode_bytes reads
        latent_bits, page_size, sink, local, heads = 4, 128, 4, 128, 16

    # (1) ragged decode
    B = 32
    rng = np.random.default_rng(np.random.SeedSequence([11, B]))
    lengths = [int(x) for x in rng.integers(1024, 8193, size=B)]
    max_pages = (max(lengths) + 127) // 128
    n_pool = int(math.ceil(B * max_pages * 1.25))
    bt = rng.permutation(n_pool)[: B * max_pages].astype(np.int32).reshape(B, max_pages)
    layers = max(2, math.ceil(1.0e9 / (sum((L + 127) // 128 for L in lengths) * page_bytes)))
    caches = []
    for _ in range(layers):
        c = mla.DeviceCache(lay, B, max_pages, bt, n_pool)
        n_tok = sum(lengths)
        c.append(bf16_rows(n_tok, 512), bf16_rows(n_tok, 64, outl), lengths)
        caches.append(c)
    q_lat = bf16_rows(B * heads, 512).view(B, heads, 512).contiguous()
    q_rope = bf16_rows(B * heads, 64).view(B, heads, 64).contiguous()
    stream = torch.cuda.current_stream()
    for c in caches:
        c.decode(q_lat, q_rope, scale, stream=stream)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps * layers)]
    for st in range(steps):
        for li, c in enumerate(caches):
            e = evs[st * layers + li]
            e[0].record(stream)
            c.decode(q_lat, q_rope, scale, stream=stream)
            e[1].record(stream)
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in evs]) * 1000.0)
    byts = sum(algorithmic_decode_bytes(W, L)["total"] for L in lengths)
    gbs = byts / (us * 1e-6) / 1e9
    print(json.dumps({"ragged": "C4R4 decode, 16 heads, page 128, sink 4 + local 128, 32 sequences, "
                                "lengths uniform in [1024, 8192]",
                      "mean_tokens": round(float(np.mean(lengths)), 1), "max_tokens": max(lengths),
                      "layers": layers, "decode_us": round(us, 3), "algorithmic_bytes": byts,
                      "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}), flush=True)
    del caches
    torch.cuda.empty_cache()

    # (2) chunked prefill: 4 prompts of 131072 tokens in chunks of 8192
    B, N, chunk = 4, 131072, 8192
    max_pages = N // 128
    n_pool = B * max_pages
    bt = np.arange(n_pool, dtype=np.int32).reshape(B, max_pages)
    c = mla.DeviceCache(lay, B, max_pages, bt, n_pool)
    ckv = bf16_rows(B * chunk, 512)
    kr = bf16_rows(B * chunk, 64, outl)
    # the entry point itself, every argument already on the device (the
    # DeviceCache helper would also time its small host-to-device copies)
    cu_new = torch.arange(0, (B + 1) * chunk, chunk, dtype=torch.int32, device="cuda")
    before = [torch.full((B,), k * chunk, dtype=torch.int32, device="cuda") for k in range(N // chunk)]
    torch.cuda.synchronize()
    evs = []
    for k in range(N // chunk):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        mla.mla_lowbit_write(lay, ckv, kr, cu_new, before[k], B, B * chunk, chunk, c.block_table, max_pages, n_pool,
                             c.pool, c.sink, c.ring, c.tail, stream)
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs[1:]]
    per_tok = 1152 + 304  # read bf16 row, write codes + metadata (C4R4)
    gbs = B * chunk * per_tok / (float(np.median(ms)) * 1e-3) / 1e9
    print(json.dumps({"chunked_prefill": "writer, C4R4 page 128, 4 prompts of 131072 tokens in chunks of 8192",
                      "chunk_us_median": round(float(np.median(ms)) * 1000.0, 2),
                      "tokens_per_s": round(B * chunk / (float(np.median(ms)) * 1e-3), 1),
                      "algorithmic_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}), flush=True)
    return 0


def transform_cost(steps: int) -> int:
    """Per-layer cost of the latent transform A_c (RAQ-MLA appendix Table 9:
    one GLM-shaped MLA layer, 2K cached tokens, decode batch 1..64): the
    writer with A_c fused in against the plain writer, and a standalone bf16
    GEMM (the library's, x A_c^T) that a separate transform would run before
    the plain writer.  C4R4, page 64, sink 4 + local 128, 20 heads; one new
    token per sequence at position 2053 (a step that completes no page).
    A_c is a seeded random orthogonal matrix.  Times are GPU times per call
    from events, with the calls queued behind a sleep kernel so that the host
    does not pace them.  One JSON line per batch."""
    import torch

    from bit_kv_cache_writer_amd import mla
    from bit_kv_cache_writer_amd import workloads as wl

    mla.lib()
    lay = mla.Layout(64, 4, 0.0, 4, 128)
    heads, scale, pos = 20, 1.0 / math.sqrt(192.0), 2053
    a_c = torch.from_numpy(wl.random_orthogonal_bf16(5).view(np.int16)).cuda()
    a_t = a_c.view(torch.bfloat16).t().contiguous()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(17)
    stream = torch.cuda.current_stream()
    reps = max(20, steps * 20)

    def bf16_rows(n, width):
        return torch.randn((n, width), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        try:
            torch.cuda._sleep(50_000_000)  # the queue fills while this runs
        except (AttributeError, RuntimeError):
            pass
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in evs]) * 1000.0)

    for B in (1, 2, 4, 8, 64):
        max_pages = (pos + 1 + 63) // 64
        n_pool = B * max_pages
        bt = np.arange(n_pool, dtype=np.int32).reshape(B, max_pages)
        caches = []
        for _ in range(2):
            c = mla.DeviceCache(lay, B, max_pages, bt, n_pool)
            c.append(bf16_rows(B * pos, 512), bf16_rows(B * pos, 64), [pos] * B)
            caches.append(c)
        plain, fused = caches
        x = bf16_rows(B, 512)
        kr = bf16_rows(B, 64)
        cu_new = torch.arange(B + 1, dtype=torch.int32, device="cuda")
        before = torch.full((B,), pos, dtype=torch.int32, device="cuda")
        seqlens = torch.full((B,), pos + 1, dtype=torch.int32, device="cuda")
        ws_bytes = mla.mla_lowbit_decode_workspace(lay, B, heads, pos + 1)
        ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
        out = torch.empty((B, heads, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, heads), dtype=torch.float32, device="cuda")
        q_lat = bf16_rows(B * heads, 512)
        q_rope = bf16_rows(B * heads, 64)
        y = torch.empty((B, 512), dtype=torch.bfloat16, device="cuda")

        def w_plain():
            mla.mla_lowbit_write(lay, x, kr, cu_new, before, B, B, 1, plain.block_table, max_pages, n_pool,
                                 plain.pool, plain.sink, plain.ring, plain.tail, stream)

        def w_fused():
            mla.mla_lowbit_write_transformed(lay, a_c, x, kr, cu_new, before, B, B, 1, fused.block_table,
                                             max_pages, n_pool, fused.pool, fused.sink, fused.ring, fused.tail,
                                             stream)

        def gemm():
            torch.matmul(x.view(torch.bfloat16), a_t, out=y)

        def dec():
            mla.mla_lowbit_decode(lay, q_lat, q_rope, B, heads, scale, plain.pool, n_pool, plain.block_table,
                                  max_pages, seqlens, pos + 1, plain.sink, plain.ring, plain.tail, out, lse, ws,
                                  ws_bytes, stream)

        t_plain, t_fused, t_gemm, t_dec = timed(w_plain), timed(w_fused), timed(gemm), timed(dec)
        cost = t_fused - t_plain
        print(json.dumps({"transform": "latent transform A_c (512 x 512) per new token, C4R4 page 64, "
                                       "2054 cached tokens, 20 heads",
                          "batch": B, "plain_write_us": round(t_plain, 2), "fused_write_us": round(t_fused, 2),
                          "fused_cost_us": round(cost, 2), "standalone_gemm_us": round(t_gemm, 2),
                          "decode_us": round(t_dec, 2),
                          "fused_share": round(cost / (t_plain + t_dec), 4)}), flush=True)
        del caches, plain, fused
        torch.cuda.empty_cache()
    return 0


def probes() -> dict:
    """Measured peaks beside the published ones: a 4 GiB read stream and the
    fp16 matrix-core probe (include/mla_lowbit_probe.h), and a plain 1 GiB
    device copy (read + write)."""
    import torch

    from bit_kv_cache_writer_amd import mla

    stream = torch.cuda.current_stream()
    n = 4 << 30
    src = torch.ones(n // 2, dtype=torch.int16, device="cuda")
    sink_u = torch.empty(mla.PROBE_BLOCKS * 256, dtype=torch.int32, device="cuda")
    sink_f = torch.empty(mla.PROBE_BLOCKS * 256, dtype=torch.float32, device="cuda")

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    t_read = timed(lambda: mla.mla_lowbit_probe_read(src, n, sink_u, stream), 5)
    flops = [0.0]

    def mf():
        flops[0] = mla.mla_lowbit_probe_mfma(sink_f, 10000, stream)
    t_mfma = timed(mf, 3)
    del src
    cp_src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    cp_dst = torch.empty_like(cp_src)
    t_copy = timed(lambda: cp_dst.copy_(cp_src), 5)
    del cp_src, cp_dst
    torch.cuda.empty_cache()
    return {"hbm_read_probe_gbs": round(n / t_read / 1e9, 1),
            "hbm_copy_probe_gbs": round(2 * (1 << 30) / t_copy / 1e9, 1),
            "mfma_f16_probe_tflops": round(flops[0] / t_mfma / 1e12, 1),
            "spec_hbm_gbs": HBM_PEAK_GBS, "spec_mfma_f16_tflops": MFMA_F16_PEAK_TFLOPS,
            "what": "read: 4 GiB streamed once with 16-B loads; copy: 1 GiB device copy, read + write bytes; "
                    "mfma: 8 independent v_mfma_f32_32x32x16_f16 chains per wave, 2048 x 4 waves"}


def make_inputs(w, n, source: str):
    """Device inputs of a workload: N-1 cached tokens per sequence and the
    incoming token.  source 'numpy': the seeded per-sequence generator the
    tests and the oracle use; 'gpu': the same distributions drawn on the GPU
    (timing only)."""
    import torch

    from bit_kv_cache_writer_amd import workloads as wl

    B = w.batch
    if source == "numpy":
        ckv = torch.empty((B * (n - 1), 512), dtype=torch.int16, device="cuda")
        kr = torch.empty((B * (n - 1), 64), dtype=torch.int16, device="cuda")
        new_ckv = torch.empty((B, 512), dtype=torch.int16, device="cuda")
        new_kr = torch.empty((B, 64), dtype=torch.int16, device="cuda")
        for b in range(B):
            c, k = wl.seq_tokens(w, b)
            ckv[b * (n - 1):(b + 1) * (n - 1)] = torch.from_numpy(c[: n - 1].view(np.int16))
            kr[b * (n - 1):(b + 1) * (n - 1)] = torch.from_numpy(k[: n - 1].view(np.int16))
            new_ckv[b] = torch.from_numpy(c[n - 1].view(np.int16))
            new_kr[b] = torch.from_numpy(k[n - 1].view(np.int16))
        ql, qr = wl.queries(w)
        return ckv, kr, new_ckv, new_kr, torch.from_numpy(ql.view(np.int16)).cuda(), \
            torch.from_numpy(qr.view(np.int16)).cuda()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    outl = torch.ones(64, device="cuda")
    outl[list(w.outlier_channels)] = w.outlier_mult

    def rows(m, width, mult=None):
        out = torch.empty((m, width), dtype=torch.int16, device="cuda")
        for a in range(0, m, 1 << 20):
            e = min(m, a + (1 << 20))
            x = torch.randn((e - a, width), generator=gen, device="cuda", dtype=torch.float32)
            if mult is not None:
                x *= mult
            out[a:e] = x.to(torch.bfloat16).view(torch.int16)
        return out

    return (rows(B * (n - 1), 512), rows(B * (n - 1), 64, outl), rows(B, 512), rows(B, 64, outl),
            rows(B * w.heads, 512).view(B, w.heads, 512).contiguous(),
            rows(B * w.heads, 64).view(B, w.heads, 64).contiguous())


def measure(w, steps: int, warmup: int, layers: int = 0, source: str = "numpy", max_layers: int = 4096) -> dict:
    """Times `steps` steps over `layers` distinct layer caches (enough for
    >= 1 GB of packed pages unless given): per layer the writer appends the
    incoming token of every sequence (completing a page) and the decode attends
    over the N cached tokens; HIP events on the launch stream around every
    decode call."""
    import torch

    from bit_kv_cache_writer_amd import mla
    from bit_kv_cache_writer_amd import workloads as wl

    lay = mla.Layout(w.page_size, w.latent_bits, w.clip_q, w.sink, w.local)
    n = w.seqlen
    max_pages = w.pages_per_seq()
    bt, n_pool = wl.block_table(w, max_pages)
    page_bytes = mla.mla_lowbit_layout_query(lay)["page_bytes"]
    packed_layer = w.batch * max_pages * page_bytes
    layers = layers or min(max_layers, max(2, math.ceil(1.0e9 / packed_layer)))
    print(f"[bench] {w.name}: {layers} layers x {packed_layer / 1e6:.1f} MB packed ({source} inputs)",
          file=sys.stderr, flush=True)
    ckv, kr, new_ckv, new_kr, q_lat, q_rope = make_inputs(w, n, source)
    caches, fill_ms = [], []
    # the bulk fill: one mla_lowbit_write of N - 1 tokens per sequence, its
    # arguments already on the device, events around the call alone
    fill_cu = torch.arange(0, w.batch * (n - 1) + 1, n - 1, dtype=torch.int32, device="cuda")
    fill_before = torch.zeros(w.batch, dtype=torch.int32, device="cuda")
    fill_after = torch.full((w.batch,), n - 1, dtype=torch.int32, device="cuda")
    for _ in range(layers):
        cache = mla.DeviceCache(lay, w.batch, max_pages, bt, n_pool)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        mla.mla_lowbit_write(lay, ckv, kr, fill_cu, fill_before, w.batch, w.batch * (n - 1), n - 1,
                             cache.block_table, max_pages, n_pool, cache.pool, cache.sink, cache.ring, cache.tail)
        e1.record()
        cache.lengths.copy_(fill_after)
        cache.host_lengths = [n - 1] * w.batch
        caches.append(cache)
        if len(fill_ms) < 4:
            torch.cuda.synchronize()
            fill_ms.append(e0.elapsed_time(e1))
    del ckv, kr
    fill_bytes = w.batch * (n - 1) * 1152 + w.batch * (n - 1) * (512 * w.latent_bits // 8 + 16 + 32)
    stream = torch.cuda.current_stream()
    cu_new = torch.arange(w.batch + 1, dtype=torch.int32, device="cuda")
    before = torch.full((w.batch,), n - 1, dtype=torch.int32, device="cuda")
    seqlens = torch.full((w.batch,), n, dtype=torch.int32, device="cuda")
    ws_bytes = mla.mla_lowbit_decode_workspace(lay, w.batch, w.heads, n)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, w.heads, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.batch, w.heads), dtype=torch.float32, device="cuda")

    def layer_step(c, ev=None):
        mla.mla_lowbit_write(lay, new_ckv, new_kr, cu_new, before, w.batch, w.batch, 1, c.block_table,
                             max_pages, n_pool, c.pool, c.sink, c.ring, c.tail, stream)
        if ev is not None:
            ev[0].record(stream)
        mla.mla_lowbit_decode(lay, q_lat, q_rope, w.batch, w.heads, w.softmax_scale, c.pool, n_pool,
                              c.block_table, max_pages, seqlens, n, c.sink, c.ring, c.tail, out, lse,
                              ws, ws_bytes, stream)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(warmup):
        for c in caches:
            layer_step(c)
    torch.cuda.synchronize()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in caches] for _ in range(steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(steps):
        for li, c in enumerate(caches):
            layer_step(c, evs[s][li])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    dec_ms = np.array([a.elapsed_time(b) for row in evs for a, b in row])
    del caches
    torch.cuda.empty_cache()
    ms_per_step = total_ms / steps
    us_layer = ms_per_step * 1000.0 / layers
    dec_us = float(dec_ms.mean() * 1000.0)
    # the first fill also pays one-time costs (code object load): left out
    fill = float(np.median(fill_ms[1:] if len(fill_ms) > 1 else fill_ms))
    return {"layers": layers, "ms_per_step": ms_per_step, "us_layer": us_layer, "dec_us": dec_us,
            "dec_us_median": float(np.median(dec_ms) * 1000.0),
            "dec_us_p10": float(np.percentile(dec_ms, 10) * 1000.0),
            "dec_us_p90": float(np.percentile(dec_ms, 90) * 1000.0),
            "write_us": us_layer - dec_us, "fill_gbs": fill_bytes / (fill * 1e-3) / 1e9, "wall": wall,
            "workspace_bytes": ws_bytes}


def rates(w, m) -> dict:
    """Rates of a measured workload against the binding roofline: HBM time of
    the algorithmic bytes at 8 TB/s vs matrix-core time of the useful flops
    (2176 per cached token and head) at 2.5 PFLOP/s."""
    alg = algorithmic_decode_bytes(w, w.seqlen)
    byts = alg["total"] * w.batch
    flops = FLOPS_PER_TOKEN_HEAD * w.seqlen * w.heads * w.batch
    dec_s = m["dec_us"] * 1e-6
    gbs, tflops = byts / dec_s / 1e9, flops / dec_s / 1e12
    hbm_bound = byts / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_F16_PEAK_TFLOPS * 1e12)
    return {"decode_us": round(m["dec_us"], 3), "decode_us_median": round(m["dec_us_median"], 3),
            "decode_us_p10": round(m["dec_us_p10"], 3), "decode_us_p90": round(m["dec_us_p90"], 3),
            "algorithmic_bytes": byts, "flops": flops, "bound": "hbm" if hbm_bound else "mfma",
            "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "packed_cache_gbs": round(alg["cache"] * w.batch / dec_s / 1e9, 1),
            "mfma_tflops": round(tflops, 2), "mfma_frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
            "write_us": round(m["write_us"], 3), "new_tokens_per_step": w.batch,
            "writer_bulk_fill_gbs": round(m["fill_gbs"], 1), "layers": m["layers"]}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c4r4_h128")
    ap.add_argument("--layers", type=int, default=0, help="0: enough layers for >= 1 GB of packed cache")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-table", action="store_true", help="skip the per-workload table and the probes")
    ap.add_argument("--calibrate-copy", action="store_true", help="time a plain 1 GiB copy and exit")
    ap.add_argument("--sweep", action="store_true", help="context sweep 1K..1M at batch 1 and 8 (JSON lines)")
    ap.add_argument("--ragged", action="store_true", help="ragged-batch decode and chunked-prefill writer (JSON lines)")
    ap.add_argument("--transform", action="store_true",
                    help="cost of the latent transform fused into the writer vs a standalone GEMM (JSON lines)")
    ap.add_argument("--bf16-baseline", action="store_true",
                    help="low-bit decode against the plain BF16 paged cache (mla_bf16.h): context sweep 1K..1M at "
                         "batch 1 and 8, then the six workloads (JSON lines, Delta %% as QuantMLA Table 9)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2

    import torch

    from bit_kv_cache_writer_amd import mla
    from bit_kv_cache_writer_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        return calibrate_copy()
    if args.sweep:
        return sweep(max(1, min(args.steps, 5)))
    if args.ragged:
        return ragged(max(1, min(args.steps, 5)))
    if args.transform:
        return transform_cost(max(1, min(args.steps, 5)))
    if args.bf16_baseline:
        return bf16_compare(max(1, min(args.steps, 5)))
    mla.lib()
    w = wl.WORKLOADS[args.workload]

    m = measure(w, args.steps, args.warmup, args.layers, "numpy")
    head = rates(w, m)
    dec_us = m["dec_us"]
    hbm_roof = {"bound": "hbm", "achieved": head["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": head["hbm_frac"]}
    mfma_roof = {"bound": "mfma", "achieved": head["mfma_tflops"], "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": head["mfma_frac"]}
    hbm_bound = head["bound"] == "hbm"
    roof = dict(hbm_roof if hbm_bound else mfma_roof)
    roof.update({"traffic": measured_traffic(w.name),
                 "kernel": "mla_lowbit_decode call (its attention kernels + split merge), events per call",
                 "bytes_per_launch": head["algorithmic_bytes"], "flops_per_launch": head["flops"],
                 "other": mfma_roof if hbm_bound else hbm_roof})

    table, prb = None, None
    if not args.no_table:
        table = {}
        for name, wk in wl.WORKLOADS.items():
            if name == w.name:
                table[name] = head
                continue
            table[name] = rates(wk, measure(wk, max(1, min(args.steps, 5)), 1, 0, "gpu", max_layers=128))
        prb = probes()
        roof["measured_peak"] = {"hbm_read_gbs": prb["hbm_read_probe_gbs"],
                                 "mfma_f16_tflops": prb["mfma_f16_probe_tflops"]}
        roof["frac_of_measured_peak"] = round(
            (head["hbm_gbs"] / prb["hbm_read_probe_gbs"]) if hbm_bound else
            (head["mfma_tflops"] / prb["mfma_f16_probe_tflops"]), 4)

    cpu = None
    if not args.no_cpu:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, w.batch)

    line = {
        "metric": "MLA low-bit decode us/layer and packed-cache HBM GB/s (% of roofline)",
        "value": round(dec_us, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "batch": w.batch, "heads": w.heads,
                   "cached_tokens": w.seqlen, "page": w.page_size, "paths": w.paths, "sink": w.sink,
                   "local": w.local, "layers_per_step": m["layers"],
                   "step": "per layer: append 1 token per sequence (completes a page) + decode over N",
                   "value": "decode (attention + split merge) us per layer"},
        "decode_us": round(dec_us, 3),
        "decode_us_median": head["decode_us_median"],
        "write_us": round(m["write_us"], 3),
        "writer_new_tokens_per_step": w.batch,
        "writer_tokens_per_s": round(w.batch / (m["write_us"] * 1e-6), 1),
        "step_us_per_layer": round(m["us_layer"], 3),
        "packed_cache_gbs": head["packed_cache_gbs"],
        "packed_cache_frac_of_hbm": round(head["packed_cache_gbs"] / HBM_PEAK_GBS, 4),
        "writer_bulk_fill_gbs": round(m["fill_gbs"], 1),
        "writer_bulk_fill_frac_of_hbm": round(m["fill_gbs"] / HBM_PEAK_GBS, 4),
        "wall_s": round(m["wall"], 3),
        "roofline": roof,
        "cpu_baseline": cpu,
        "probes": prb,
        "configs": table,
        "context_h20": {"raq_mla_us_per_layer": 12.6, "flashmla_us_per_layer": 17.4,
                        "tpot_ms": [5.97, 6.56]},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
