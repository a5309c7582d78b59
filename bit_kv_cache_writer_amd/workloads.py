"""Seeded synthetic workloads for the low-bit MLA cache.

Random-number generation only: this module draws the inputs (latent c_KV,
positional key k_R, absorbed queries, block tables) and rounds them to bf16.
It holds none of the cache method's arithmetic, so both the GPU path and the
CPU reference can take their inputs from it.

Input recipe (shapes of the configurations the method is measured on; the
value structure follows the RAQ-MLA page, Figures 2 and 8: a diffuse latent
and a positional key with fixed-channel outlier bands):
  * c_KV  ~ N(0, 1)                                   [tokens][512]
  * k_R   ~ N(0, 1), a fixed set of channels scaled   [tokens][64]
  * q_lat ~ N(0, 1), q_rope ~ N(0, 1)                 [batch][heads][512|64]
  * every value rounded once from fp32 to bf16 (round to nearest even)
  * numpy PCG64; sequence b of a workload draws from SeedSequence([seed, b]),
    so any single sequence can be regenerated alone
  * block tables: a seeded random permutation over a page pool 1.25x larger
    than needed, so no contiguity is ever assumed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

C4_OUTLIERS = (7, 23, 39, 55)
C2_OUTLIERS = (6, 7, 22, 23, 38, 39, 54, 55)


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    seqlen: int
    page_size: int
    latent_bits: int
    clip_q: float
    sink: int
    local: int
    outlier_channels: tuple
    outlier_mult: float
    seed: int
    softmax_scale: float = 1.0 / math.sqrt(192.0)
    description: str = ""
    latent_dim: int = 512
    rope_dim: int = 64

    @property
    def paths(self) -> str:
        return f"C{self.latent_bits}R4"

    def pages_per_seq(self, extra_tokens: int = 0) -> int:
        return (self.seqlen + extra_tokens + self.page_size - 1) // self.page_size


WORKLOADS = {
    "tiny_c4r4": Workload(
        "tiny_c4r4", batch=1, heads=16, seqlen=256, page_size=64, latent_bits=4, clip_q=0.0,
        sink=4, local=32, outlier_channels=C4_OUTLIERS, outlier_mult=20.0, seed=1,
        description="C4R4 decode, batch 1, 16 heads, 256 cached tokens, page 64, sink 4, local 32"),
    "c4r4_h16_b8": Workload(
        "c4r4_h16_b8", batch=8, heads=16, seqlen=4096, page_size=128, latent_bits=4, clip_q=0.0,
        sink=4, local=128, outlier_channels=C4_OUTLIERS, outlier_mult=20.0, seed=2,
        description="C4R4 decode, batch 8 x 4096 tokens, 16 heads, page 128, sink 4 + local 128"),
    "c4r4_h16_b32": Workload(
        "c4r4_h16_b32", batch=32, heads=16, seqlen=4096, page_size=128, latent_bits=4, clip_q=0.0,
        sink=4, local=128, outlier_channels=C4_OUTLIERS, outlier_mult=20.0, seed=3,
        description="C4R4 decode, batch 32 x 4096 tokens, 16 heads, page 128, sink 4 + local 128"),
    "c2r4_h20": Workload(
        "c2r4_h20", batch=16, heads=20, seqlen=16384, page_size=128, latent_bits=2, clip_q=0.94,
        sink=4, local=128, outlier_channels=C2_OUTLIERS, outlier_mult=16.0, seed=4,
        description="C2R4 decode, batch 16 x 16384 tokens, 20 heads, page 128, 0.94 clip"),
    "c4r4_h128": Workload(
        "c4r4_h128", batch=64, heads=128, seqlen=32768, page_size=64, latent_bits=4, clip_q=0.0,
        sink=4, local=128, outlier_channels=C4_OUTLIERS, outlier_mult=20.0, seed=5,
        description="C4R4 decode, batch 64 x 32768 tokens, 128 heads, page 64"),
    "c2r4_h64_long": Workload(
        "c2r4_h64_long", batch=4, heads=64, seqlen=131072, page_size=64, latent_bits=2,
        clip_q=0.94, sink=4, local=128, outlier_channels=C2_OUTLIERS, outlier_mult=16.0, seed=6,
        description="C2R4 decode, batch 4 x 131072 tokens, 64 heads, page 64"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def seq_tokens(w: Workload, b: int, n: int | None = None, start: int = 0, latent_mult: float = 1.0):
    """Tokens [start, start+n) of sequence b: (c_kv, k_r) as bf16 bit arrays
    (the latent drawn N(0, latent_mult^2) when latent_mult != 1)."""
    n = w.seqlen if n is None else n
    rng = _rng(w.seed, b)
    if start:
        rng.standard_normal((start, w.latent_dim + w.rope_dim), dtype=np.float32)
    x = rng.standard_normal((n, w.latent_dim + w.rope_dim), dtype=np.float32)
    ckv = x[:, : w.latent_dim]
    if latent_mult != 1.0:
        ckv = ckv * np.float32(latent_mult)
    kr = x[:, w.latent_dim:].copy()
    if w.outlier_channels:
        kr[:, list(w.outlier_channels)] *= np.float32(w.outlier_mult)
    return f32_to_bf16_bits(ckv), f32_to_bf16_bits(kr)


def batch_tokens(w: Workload, n: int | None = None):
    """All sequences' tokens concatenated: ([B*n][512], [B*n][64]) bf16 bits."""
    n = w.seqlen if n is None else n
    ckv = np.empty((w.batch * n, w.latent_dim), dtype=np.uint16)
    kr = np.empty((w.batch * n, w.rope_dim), dtype=np.uint16)
    for b in range(w.batch):
        c, k = seq_tokens(w, b, n)
        ckv[b * n:(b + 1) * n] = c
        kr[b * n:(b + 1) * n] = k
    return ckv, kr


def queries(w: Workload, stream: int = 1_000_003):
    rng = _rng(w.seed, stream)
    ql = rng.standard_normal((w.batch, w.heads, w.latent_dim), dtype=np.float32)
    qr = rng.standard_normal((w.batch, w.heads, w.rope_dim), dtype=np.float32)
    return f32_to_bf16_bits(ql), f32_to_bf16_bits(qr)


def block_table(w: Workload, max_pages: int, stream: int = 2_000_003):
    """[batch][max_pages] int32 page ids, a permutation over a 1.25x pool."""
    need = w.batch * max_pages
    pool_pages = int(math.ceil(need * 1.25))
    perm = _rng(w.seed, stream).permutation(pool_pages)[:need].astype(np.int32)
    return perm.reshape(w.batch, max_pages), pool_pages


def cu_from_counts(counts) -> np.ndarray:
    counts = np.asarray(counts, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def random_orthogonal_bf16(seed: int, dim: int = 512) -> np.ndarray:
    """A seeded random orthogonal matrix (QR of a Gaussian one, signs fixed by
    R's diagonal), rounded to bf16 bits: a stand-in for a fitted latent
    transform, which needs training data."""
    g = _rng(seed, 3_000_017).standard_normal((dim, dim))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]
    return f32_to_bf16_bits(q.astype(np.float32))
