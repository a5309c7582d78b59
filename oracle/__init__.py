"""CPU reference of the dual-path low-bit MLA cache: writer and decode.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
(``bit_kv_cache_writer_amd``) never imports, links or calls it, and the two
share no code.

The arithmetic lives in ``mla_oracle.c`` (plain C, single thread, fp32
quantizer with every operation separately rounded, fp64 decode).  This module
only builds it with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "libmla_oracle.so")
_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (contraction off, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class OrcLayout(ctypes.Structure):
    _fields_ = [
        ("latent_dim", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("latent_bits", ctypes.c_int32),
        ("rope_bits", ctypes.c_int32),
        ("latent_group", ctypes.c_int32),
        ("latent_clip_q", ctypes.c_double),
        ("sink", ctypes.c_int32),
        ("local", ctypes.c_int32),
    ]


@dataclass(frozen=True)
class Layout:
    page_size: int
    latent_bits: int
    latent_clip_q: float
    sink: int
    local: int
    latent_dim: int = 512
    rope_dim: int = 64
    rope_bits: int = 4
    latent_group: int = 128

    def c(self) -> OrcLayout:
        return OrcLayout(self.latent_dim, self.rope_dim, self.page_size, self.latent_bits,
                         self.rope_bits, self.latent_group, self.latent_clip_q, self.sink,
                         self.local)


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("MLA_ORACLE_LIB")  # a planted-mistake build, tests only
        if path is None:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        L.oracle_page_bytes.restype = i64
        L.oracle_page_bytes.argtypes = [P]
        L.oracle_page_offsets.argtypes = [P, P]
        L.oracle_f16_round_down.restype = ctypes.c_uint16
        L.oracle_f16_round_down.argtypes = [f32]
        L.oracle_f16_round_up.restype = ctypes.c_uint16
        L.oracle_f16_round_up.argtypes = [f32]
        L.oracle_f16_round_down_n.argtypes = [P, i64, P]
        L.oracle_f16_round_up_n.argtypes = [P, i64, P]
        L.oracle_f16_value.restype = f64
        L.oracle_f16_value.argtypes = [ctypes.c_uint16]
        L.oracle_quantile_params.argtypes = [i32, f64, P, P, P]
        L.oracle_clip_value.restype = f32
        L.oracle_clip_value.argtypes = [P, i32, f64]
        L.oracle_quantize_group.argtypes = [P, i32, i32, i32, P, P, P]
        L.oracle_pack_row.argtypes = [P, i32, i32, P]
        L.oracle_unpack_row.argtypes = [P, i32, i32, P]
        L.oracle_write.restype = i32
        L.oracle_write.argtypes = [P, P, P, P, P, i32, P, i32, P, P, P, P]
        L.oracle_read_token.restype = i32
        L.oracle_read_token.argtypes = [P, P, P, P, P, P, i32, i32, i32, P]
        L.oracle_decode.argtypes = [P, P, P, i32, i32, f64, P, P, i32, P, P, P, P, P, P]
        L.oracle_decode_bf16.argtypes = [P, P, i32, i32, f64, P, i32, P, i32, P, P, P]
        L.oracle_transform.argtypes = [P, P, i64, i32, P]
        L.oracle_transform.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "arrays passed to the oracle must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def page_bytes(layout: Layout) -> int:
    return int(lib().oracle_page_bytes(ctypes.byref(layout.c())))


def page_offsets(layout: Layout) -> dict:
    out = np.zeros(6, dtype=np.int64)
    lib().oracle_page_offsets(ctypes.byref(layout.c()), _p(out))
    keys = ["latent_codes", "latent_meta", "rope_codes", "rope_meta", "page_bytes", "latent_row"]
    return {k: int(v) for k, v in zip(keys, out)}


def f16_round_down(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32).ravel())
    out = np.zeros(x.size, dtype=np.uint16)
    lib().oracle_f16_round_down_n(_p(x), x.size, _p(out))
    return out


def f16_round_up(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32).ravel())
    out = np.zeros(x.size, dtype=np.uint16)
    lib().oracle_f16_round_up_n(_p(x), x.size, _p(out))
    return out


def quantile_params(n: int, q: float):
    lo, hi, frac = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_float()
    lib().oracle_quantile_params(n, q, ctypes.byref(lo), ctypes.byref(hi), ctypes.byref(frac))
    return lo.value, hi.value, frac.value


def clip_value(x, q: float) -> float:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return float(lib().oracle_clip_value(_p(x), x.size, q))


def quantize_group(x, levels: int):
    """Returns (codes uint8[n], scale fp16 bits, min fp16 bits)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    codes = np.zeros(x.size, dtype=np.uint8)
    sh, mh = ctypes.c_uint16(), ctypes.c_uint16()
    lib().oracle_quantize_group(_p(x), x.size, 1, levels, ctypes.byref(sh), ctypes.byref(mh), _p(codes))
    return codes, sh.value, mh.value


def pack_row(codes, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    row = np.zeros(codes.size * bits // 8, dtype=np.uint8)
    lib().oracle_pack_row(_p(codes), codes.size, bits, _p(row))
    return row


def unpack_row(row, n: int, bits: int) -> np.ndarray:
    row = np.ascontiguousarray(np.asarray(row, dtype=np.uint8))
    codes = np.zeros(n, dtype=np.uint8)
    lib().oracle_unpack_row(_p(row), n, bits, _p(codes))
    return codes


def write(layout: Layout, c_kv, k_r, cu_new, seqlens_before, block_table, pool, sink_buf,
          ring_buf, tail_buf) -> None:
    """In-place append (see oracle_write).  bf16 arrays are uint16 views."""
    arrs = [c_kv, k_r, cu_new, seqlens_before, block_table, pool, sink_buf, ring_buf, tail_buf]
    for a in arrs:
        assert a.flags["C_CONTIGUOUS"]
    assert c_kv.dtype == np.uint16 and k_r.dtype == np.uint16
    assert cu_new.dtype == np.int32 and seqlens_before.dtype == np.int32
    assert block_table.dtype == np.int32 and pool.dtype == np.uint8
    batch = seqlens_before.size
    rc = lib().oracle_write(ctypes.byref(layout.c()), _p(c_kv), _p(k_r), _p(cu_new),
                            _p(seqlens_before), batch, _p(block_table), block_table.shape[1],
                            _p(pool), _p(sink_buf), _p(ring_buf), _p(tail_buf))
    if rc != 0:
        raise ValueError("oracle_write: position beyond the block table")


def transform(a_c, x) -> np.ndarray:
    """bf16(A_c x) per token row of x (see oracle_transform); uint16 views."""
    a_c = np.ascontiguousarray(a_c, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=np.uint16)
    dim = a_c.shape[0]
    assert a_c.shape == (dim, dim) and x.shape[-1] == dim
    y = np.zeros_like(x)
    lib().oracle_transform(_p(a_c), _p(x), x.size // dim, dim, _p(y))
    return y


def read_token(layout: Layout, pool, block_table, sink_buf, ring_buf, tail_buf, b: int,
               seqlen: int, j: int):
    out = np.zeros(layout.latent_dim + layout.rope_dim, dtype=np.float64)
    row = np.ascontiguousarray(block_table[b])
    kind = lib().oracle_read_token(ctypes.byref(layout.c()), _p(pool), _p(row), _p(sink_buf),
                                   _p(ring_buf), _p(tail_buf), b, seqlen, j, _p(out))
    return out, kind


def decode(layout: Layout, q_lat, q_rope, scale: float, pool, block_table, seqlens, sink_buf,
           ring_buf, tail_buf):
    """fp64 decode; returns (out [B][H][latent_dim], lse [B][H])."""
    B, H, D = q_lat.shape
    out = np.zeros((B, H, D), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    for a in (q_lat, q_rope, pool, block_table, seqlens, sink_buf, ring_buf, tail_buf):
        assert a.flags["C_CONTIGUOUS"]
    assert seqlens.dtype == np.int32 and block_table.dtype == np.int32
    lib().oracle_decode(ctypes.byref(layout.c()), _p(q_lat), _p(q_rope), B, H, scale, _p(pool),
                        _p(block_table), block_table.shape[1], _p(seqlens), _p(sink_buf),
                        _p(ring_buf), _p(tail_buf), _p(out), _p(lse))
    return out, lse


def append_bf16(pool, page_size: int, block_table, seqlens_before, c_kv, k_r, counts):
    """Plain BF16 paged cache (the baseline of QuantMLA Table 9 caption):
    sequence b's new rows go, in order, to positions seqlens_before[b] + i,
    position j at page block_table[b][j // P], slot j % P of pool
    [pages][P][576] as (c_KV, k_R) bf16 bits.  Writes pool in place."""
    n = 0
    for b, cnt in enumerate(counts):
        for i in range(cnt):
            j = int(seqlens_before[b]) + i
            pool[block_table[b][j // page_size], j % page_size, :512] = c_kv[n]
            pool[block_table[b][j // page_size], j % page_size, 512:] = k_r[n]
            n += 1
    return pool


def decode_bf16(q_lat, q_rope, scale: float, pool, page_size: int, block_table, seqlens):
    """fp64 decode over the plain BF16 paged cache; returns (out [B][H][512],
    lse [B][H])."""
    B, H, D = q_lat.shape
    assert D == 512 and q_rope.shape == (B, H, 64) and pool.shape[1:] == (page_size, 576)
    for a in (q_lat, q_rope, pool, block_table, seqlens):
        assert a.flags["C_CONTIGUOUS"]
    assert seqlens.dtype == np.int32 and block_table.dtype == np.int32
    out = np.zeros((B, H, D), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    lib().oracle_decode_bf16(_p(q_lat), _p(q_rope), B, H, scale, _p(pool), page_size,
                             _p(block_table), block_table.shape[1], _p(seqlens), _p(out), _p(lse))
    return out, lse
