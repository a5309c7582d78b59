"""ctypes binding of libmla_lowbit.so (declared in include/mla_lowbit.h).

Argument marshalling only: every step of the writer and the decode runs in the
HIP kernels of the library.  Tensors are torch tensors on the GPU (device
memory and streams are torch's); the functions keep the C names and order.
If the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_lowbit.so")

ERRORS = {
    0: "ok", -1: "MLA_LOWBIT_ERR_LAYOUT", -2: "MLA_LOWBIT_ERR_ARG", -3: "MLA_LOWBIT_ERR_UNSUPPORTED",
    -4: "MLA_LOWBIT_ERR_WORKSPACE", -5: "MLA_LOWBIT_ERR_HIP", -6: "MLA_LOWBIT_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 64 << 20  # MLA_LOWBIT_NOALLOC_SCRATCH_BYTES
EXPORTS = ("mla_lowbit_layout_query", "mla_lowbit_write", "mla_lowbit_write_transformed",
           "mla_lowbit_decode_workspace",
           "mla_lowbit_decode", "mla_lowbit_decode_noalloc", "mla_lowbit_strerror")
PROBE_EXPORTS = ("mla_lowbit_probe_read", "mla_lowbit_probe_mfma")  # include/mla_lowbit_probe.h
BF16_EXPORTS = ("mla_bf16_append", "mla_bf16_decode_workspace", "mla_bf16_decode")  # include/mla_bf16.h
PROBE_BLOCKS = 2048  # MLA_LOWBIT_PROBE_BLOCKS


class MlaError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {ERRORS.get(code, code)} ({strerror(code)})")
        self.code = code


class CLayout(ctypes.Structure):
    _fields_ = [
        ("version", ctypes.c_int32), ("latent_dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("latent_bits", ctypes.c_int32), ("rope_bits", ctypes.c_int32),
        ("latent_group", ctypes.c_int32), ("sink", ctypes.c_int32), ("local", ctypes.c_int32),
        ("reserved", ctypes.c_int32), ("latent_clip_q", ctypes.c_double),
    ]


class CSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "page_bytes", "latent_row_bytes", "latent_meta_offset", "rope_codes_offset", "rope_row_bytes",
        "rope_meta_offset", "bf16_row_bytes", "sink_bytes_per_seq", "ring_bytes_per_seq",
        "tail_bytes_per_seq")]


@dataclass(frozen=True)
class Layout:
    """Cache-layout descriptor (fields of mla_lowbit_layout)."""
    page_size: int
    latent_bits: int
    latent_clip_q: float
    sink: int
    local: int
    latent_dim: int = 512
    rope_dim: int = 64
    rope_bits: int = 4
    latent_group: int = 128
    version: int = 1

    def c(self) -> CLayout:
        return CLayout(self.version, self.latent_dim, self.rope_dim, self.page_size, self.latent_bits,
                       self.rope_bits, self.latent_group, self.sink, self.local, 0, self.latent_clip_q)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(LIB_PATH)
        P, i32 = ctypes.c_void_p, ctypes.c_int32
        L.mla_lowbit_layout_query.restype = ctypes.c_int
        L.mla_lowbit_layout_query.argtypes = [P, P]
        L.mla_lowbit_write.restype = ctypes.c_int
        L.mla_lowbit_write.argtypes = [P, P, P, P, P, i32, i32, i32, P, i32, i32, P, P, P, P, P]
        L.mla_lowbit_write_transformed.restype = ctypes.c_int
        L.mla_lowbit_write_transformed.argtypes = [P, P, P, P, P, P, i32, i32, i32, P, i32, i32, P, P, P, P, P]
        L.mla_lowbit_decode_workspace.restype = ctypes.c_int
        L.mla_lowbit_decode_workspace.argtypes = [P, i32, i32, i32, P]
        L.mla_lowbit_decode.restype = ctypes.c_int
        L.mla_lowbit_decode.argtypes = [P, P, P, i32, i32, ctypes.c_float, P, i32, P, i32, P, i32, P, P,
                                        P, P, P, P, ctypes.c_size_t, P]
        L.mla_lowbit_decode_noalloc.restype = ctypes.c_int
        L.mla_lowbit_decode_noalloc.argtypes = [P, P, P, i32, i32, ctypes.c_float, P, i32, P, i32, P, i32, P, P,
                                                P, P, P, P]
        L.mla_lowbit_probe_read.restype = ctypes.c_int
        L.mla_lowbit_probe_read.argtypes = [P, ctypes.c_size_t, P, P]
        L.mla_lowbit_probe_mfma.restype = ctypes.c_int
        L.mla_lowbit_probe_mfma.argtypes = [P, i32, ctypes.POINTER(ctypes.c_double), P]
        L.mla_bf16_append.restype = ctypes.c_int
        L.mla_bf16_append.argtypes = [P, P, P, P, i32, i32, i32, i32, P, i32, i32, P, P]
        L.mla_bf16_decode_workspace.restype = ctypes.c_int
        L.mla_bf16_decode_workspace.argtypes = [i32, i32, i32, i32, P]
        L.mla_bf16_decode.restype = ctypes.c_int
        L.mla_bf16_decode.argtypes = [P, P, i32, i32, ctypes.c_float, P, i32, i32, P, i32, P, i32, P, P, P,
                                      ctypes.c_size_t, P]
        L.mla_lowbit_strerror.restype = ctypes.c_char_p
        L.mla_lowbit_strerror.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().mla_lowbit_strerror(code).decode()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("mla_lowbit expects device tensors")
    if not t.is_contiguous():
        raise ValueError("mla_lowbit expects contiguous tensors")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise MlaError(rc, what)


def mla_lowbit_layout_query(layout: Layout) -> dict:
    s = CSizes()
    _check(lib().mla_lowbit_layout_query(ctypes.byref(layout.c()), ctypes.byref(s)),
           "mla_lowbit_layout_query")
    return {name: getattr(s, name) for name, _ in CSizes._fields_}


def mla_lowbit_write(layout: Layout, c_kv, k_r, cu_new, seqlens_before, batch: int, total_new: int,
                     max_new_per_seq: int, block_table, max_pages: int, num_pool_pages: int, page_pool,
                     sink_buf, ring_buf, rope_tail, stream=None) -> None:
    rc = lib().mla_lowbit_write(
        ctypes.byref(layout.c()), _ptr(c_kv), _ptr(k_r), _ptr(cu_new), _ptr(seqlens_before), batch,
        total_new, max_new_per_seq, _ptr(block_table), max_pages, num_pool_pages, _ptr(page_pool),
        _ptr(sink_buf), _ptr(ring_buf), _ptr(rope_tail), _stream(stream))
    _check(rc, "mla_lowbit_write")


def mla_lowbit_write_transformed(layout: Layout, a_c, c_kv, k_r, cu_new, seqlens_before, batch: int,
                                 total_new: int, max_new_per_seq: int, block_table, max_pages: int,
                                 num_pool_pages: int, page_pool, sink_buf, ring_buf, rope_tail,
                                 stream=None) -> None:
    rc = lib().mla_lowbit_write_transformed(
        ctypes.byref(layout.c()), _ptr(a_c), _ptr(c_kv), _ptr(k_r), _ptr(cu_new), _ptr(seqlens_before),
        batch, total_new, max_new_per_seq, _ptr(block_table), max_pages, num_pool_pages, _ptr(page_pool),
        _ptr(sink_buf), _ptr(ring_buf), _ptr(rope_tail), _stream(stream))
    _check(rc, "mla_lowbit_write_transformed")


def mla_lowbit_decode_workspace(layout: Layout, batch: int, heads: int, max_seqlen: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().mla_lowbit_decode_workspace(ctypes.byref(layout.c()), batch, heads, max_seqlen,
                                             ctypes.byref(n)), "mla_lowbit_decode_workspace")
    return n.value


def mla_lowbit_decode(layout: Layout, q_lat, q_rope, batch: int, heads: int, softmax_scale: float,
                      page_pool, num_pool_pages: int, block_table, max_pages: int, seqlens,
                      max_seqlen: int, sink_buf, ring_buf, rope_tail, out, lse, workspace,
                      workspace_bytes: int, stream=None) -> None:
    rc = lib().mla_lowbit_decode(
        ctypes.byref(layout.c()), _ptr(q_lat), _ptr(q_rope), batch, heads, softmax_scale,
        _ptr(page_pool), num_pool_pages, _ptr(block_table), max_pages, _ptr(seqlens), max_seqlen,
        _ptr(sink_buf), _ptr(ring_buf), _ptr(rope_tail), _ptr(out), _ptr(lse), _ptr(workspace),
        workspace_bytes, _stream(stream))
    _check(rc, "mla_lowbit_decode")


def mla_lowbit_decode_noalloc(layout: Layout, q_lat, q_rope, batch: int, heads: int, softmax_scale: float,
                              page_pool, num_pool_pages: int, block_table, max_pages: int, seqlens,
                              max_seqlen: int, sink_buf, ring_buf, rope_tail, out, lse, stream=None) -> None:
    rc = lib().mla_lowbit_decode_noalloc(
        ctypes.byref(layout.c()), _ptr(q_lat), _ptr(q_rope), batch, heads, softmax_scale,
        _ptr(page_pool), num_pool_pages, _ptr(block_table), max_pages, _ptr(seqlens), max_seqlen,
        _ptr(sink_buf), _ptr(ring_buf), _ptr(rope_tail), _ptr(out), _ptr(lse), _stream(stream))
    _check(rc, "mla_lowbit_decode_noalloc")


def mla_lowbit_probe_read(src, nbytes: int, sink, stream=None) -> None:
    _check(lib().mla_lowbit_probe_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)), "mla_lowbit_probe_read")


def mla_lowbit_probe_mfma(sink, iters: int, stream=None) -> float:
    """Launches the matrix-core probe; returns its flop count."""
    flops = ctypes.c_double()
    _check(lib().mla_lowbit_probe_mfma(_ptr(sink), iters, ctypes.byref(flops), _stream(stream)),
           "mla_lowbit_probe_mfma")
    return flops.value


def mla_bf16_append(c_kv, k_r, cu_new, seqlens_before, batch: int, total_new: int, max_new_per_seq: int,
                    page_size: int, block_table, max_pages: int, num_pool_pages: int, pool, stream=None) -> None:
    rc = lib().mla_bf16_append(_ptr(c_kv), _ptr(k_r), _ptr(cu_new), _ptr(seqlens_before), batch, total_new,
                               max_new_per_seq, page_size, _ptr(block_table), max_pages, num_pool_pages,
                               _ptr(pool), _stream(stream))
    _check(rc, "mla_bf16_append")


def mla_bf16_decode_workspace(page_size: int, batch: int, heads: int, max_seqlen: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().mla_bf16_decode_workspace(page_size, batch, heads, max_seqlen, ctypes.byref(n)),
           "mla_bf16_decode_workspace")
    return n.value


def mla_bf16_decode(q_lat, q_rope, batch: int, heads: int, softmax_scale: float, pool, num_pool_pages: int,
                    page_size: int, block_table, max_pages: int, seqlens, max_seqlen: int, out, lse, workspace,
                    workspace_bytes: int, stream=None) -> None:
    rc = lib().mla_bf16_decode(_ptr(q_lat), _ptr(q_rope), batch, heads, softmax_scale, _ptr(pool),
                               num_pool_pages, page_size, _ptr(block_table), max_pages, _ptr(seqlens),
                               max_seqlen, _ptr(out), _ptr(lse), _ptr(workspace), workspace_bytes,
                               _stream(stream))
    _check(rc, "mla_bf16_decode")


class Bf16Cache:
    """Device buffers of one layer's plain BF16 paged cache (torch-owned):
    pool [pages][P][576] bf16 bits, block table and lengths."""

    def __init__(self, page_size: int, batch: int, max_pages: int, block_table, num_pool_pages: int,
                 device="cuda"):
        import torch
        self.page_size, self.batch, self.max_pages = page_size, batch, max_pages
        self.num_pool_pages = num_pool_pages
        self.pool = torch.zeros((num_pool_pages, page_size, 576), dtype=torch.int16, device=device)
        self.block_table = torch.as_tensor(block_table, dtype=torch.int32).to(device).contiguous()
        self.lengths = torch.zeros(batch, dtype=torch.int32, device=device)
        self.host_lengths = [0] * batch

    def append(self, c_kv, k_r, counts, stream=None) -> None:
        import torch
        counts = [int(c) for c in counts]
        if len(counts) != self.batch or min(counts) < 0:
            raise ValueError("append needs one non-negative count per sequence")
        if max(a + c for a, c in zip(self.host_lengths, counts)) > self.max_pages * self.page_size:
            raise ValueError("append beyond the block table's capacity")
        cu = [0]
        for c in counts:
            cu.append(cu[-1] + c)
        dev = self.pool.device
        cu_t = torch.tensor(cu, dtype=torch.int32, device=dev)
        mla_bf16_append(c_kv, k_r, cu_t, self.lengths, self.batch, cu[-1], max(counts), self.page_size,
                        self.block_table, self.max_pages, self.num_pool_pages, self.pool, stream)
        self.lengths += torch.tensor(counts, dtype=torch.int32, device=dev)
        self.host_lengths = [a + c for a, c in zip(self.host_lengths, counts)]

    def workspace_bytes(self, heads: int) -> int:
        return mla_bf16_decode_workspace(self.page_size, self.batch, heads, max(self.host_lengths))

    def decode(self, q_lat, q_rope, softmax_scale: float, out=None, lse=None, workspace=None, stream=None):
        import torch
        B, H, _ = q_lat.shape
        dev = self.pool.device
        out = torch.empty((B, H, 512), dtype=torch.float32, device=dev) if out is None else out
        lse = torch.empty((B, H), dtype=torch.float32, device=dev) if lse is None else lse
        ws_bytes = self.workspace_bytes(H)
        if workspace is None:
            if getattr(self, "_ws", None) is None or self._ws.numel() < ws_bytes:
                self._ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
            workspace = self._ws
        mla_bf16_decode(q_lat, q_rope, B, H, softmax_scale, self.pool, self.num_pool_pages, self.page_size,
                        self.block_table, self.max_pages, self.lengths, max(self.host_lengths), out, lse,
                        workspace, workspace.numel(), stream)
        return out, lse


class DeviceCache:
    """Device buffers of one layer's cache for `batch` sequences (torch-owned).

    Holds the page pool, block table, BF16 sink / ring / tail buffers and the
    per-sequence lengths, and forwards to the C entry points.
    """

    def __init__(self, layout: Layout, batch: int, max_pages: int, block_table, num_pool_pages: int,
                 device="cuda"):
        import torch
        self.layout, self.batch, self.max_pages = layout, batch, max_pages
        self.sizes = mla_lowbit_layout_query(layout)
        self.num_pool_pages = num_pool_pages
        self.pool = torch.zeros(num_pool_pages * self.sizes["page_bytes"], dtype=torch.uint8, device=device)
        self.block_table = torch.as_tensor(block_table, dtype=torch.int32).to(device).contiguous()
        self.sink = torch.zeros((batch, max(layout.sink, 1), 576), dtype=torch.int16, device=device)
        self.ring = torch.zeros((batch, max(layout.local, 1), 576), dtype=torch.int16, device=device)
        self.tail = torch.zeros((batch, layout.page_size, 64), dtype=torch.int16, device=device)
        self.lengths = torch.zeros(batch, dtype=torch.int32, device=device)
        self.host_lengths = [0] * batch

    @property
    def capacity(self) -> int:
        return self.max_pages * self.layout.page_size

    def append(self, c_kv, k_r, counts, stream=None, a_c=None) -> None:
        """Append counts[b] new tokens per sequence (rows of c_kv / k_r in order);
        with a_c (bf16 [512][512]) the latent rows are transformed in the writer."""
        import torch
        counts = [int(c) for c in counts]
        if len(counts) != self.batch or min(counts) < 0:
            raise ValueError("append needs one non-negative count per sequence")
        if max(a + c for a, c in zip(self.host_lengths, counts)) > self.capacity:
            raise ValueError("append beyond the block table's capacity")
        cu = [0]
        for c in counts:
            cu.append(cu[-1] + c)
        dev = self.pool.device
        cu_t = torch.tensor(cu, dtype=torch.int32, device=dev)
        if a_c is None:
            mla_lowbit_write(self.layout, c_kv, k_r, cu_t, self.lengths, self.batch, cu[-1], max(counts),
                             self.block_table, self.max_pages, self.num_pool_pages, self.pool, self.sink,
                             self.ring, self.tail, stream)
        else:
            mla_lowbit_write_transformed(self.layout, a_c, c_kv, k_r, cu_t, self.lengths, self.batch, cu[-1],
                                         max(counts), self.block_table, self.max_pages, self.num_pool_pages,
                                         self.pool, self.sink, self.ring, self.tail, stream)
        self.lengths += torch.tensor(counts, dtype=torch.int32, device=dev)
        self.host_lengths = [a + c for a, c in zip(self.host_lengths, counts)]

    def workspace_bytes(self, heads: int) -> int:
        return mla_lowbit_decode_workspace(self.layout, self.batch, heads, max(self.host_lengths))

    def decode(self, q_lat, q_rope, softmax_scale: float, out=None, lse=None, workspace=None,
               stream=None):
        import torch
        B, H, _ = q_lat.shape
        dev = self.pool.device
        out = torch.empty((B, H, 512), dtype=torch.float32, device=dev) if out is None else out
        lse = torch.empty((B, H), dtype=torch.float32, device=dev) if lse is None else lse
        ws_bytes = self.workspace_bytes(H)
        if workspace is None:
            if getattr(self, "_ws", None) is None or self._ws.numel() < ws_bytes:
                self._ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
            workspace = self._ws
        mla_lowbit_decode(self.layout, q_lat, q_rope, B, H, softmax_scale, self.pool,
                          self.num_pool_pages, self.block_table, self.max_pages, self.lengths,
                          max(self.host_lengths), self.sink, self.ring, self.tail, out, lse, workspace,
                          workspace.numel(), stream)
        return out, lse


def pool_pages_for(batch: int, max_pages: int) -> int:
    return int(math.ceil(batch * max_pages * 1.25))
