"""TQ4 paged-KV attention for AMD Instinct MI355X (gfx950).

Python face of the C ABI in include/tq4.h (functions keep the C names).  It
marshals torch tensors into pointers and the current HIP stream; the work runs
in the library's HIP kernels.

Pool layout (one layer): k_words / v_words int32 bit patterns of uint32 words
[num_pages][n_kv][page_size][32]; k_norms / v_norms int16 bit patterns of fp16
[num_pages][n_kv][page_size].  The uniform INT8 arm's pools hold int8 codes
[num_pages][n_kv][page_size][256] and int16 bit patterns of fp16 scales
[num_pages][n_kv][page_size].
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from ._binding import (TQ4_BF16, TQ4_F16, TQ4_F32, Tq4Error, check, header_functions,
                       load_library, tq4_int8_pool, tq4_layer_pool)

__all__ = ["Tq4LayerPool", "Tq4Error", "tq4_abi_version", "tq4_codebook", "tq4_encode_pages", "tq4_attn_decode_variant", "prepare_decode_variant",
           "tq4_attn_decode_workspace_size", "tq4_attn_decode", "tq4_attn_prefill_workspace_size",
           "tq4_attn_prefill_chunk", "new_workspace", "header_functions", "load_library",
           "PreparedCall", "prepare_encode", "prepare_decode", "prepare_prefill",
           "tq4_attn_decode_append", "prepare_decode_append", "tq4_attn_decode_noalloc", "tq4_attn_verify_workspace_size",
           "tq4_attn_verify", "prepare_verify", "tq4_reconstruct_pages", "tq4_sdpa_decode_workspace_size",
           "tq4_sdpa_decode", "prepare_reconstruct", "prepare_sdpa_decode", "Int8LayerPool",
           "tq4_int8_encode_pages", "tq4_int8_attn_decode_workspace_size", "tq4_int8_attn_decode", "tq4_int8_attn_decode_append", "prepare_int8_decode_append",
           "prepare_int8_decode", "tq4_int8_attn_verify_workspace_size", "tq4_int8_attn_verify",
           "prepare_int8_verify", "tq4_int8_attn_prefill_workspace_size", "tq4_int8_attn_prefill_chunk",
           "prepare_int8_prefill"]

HEAD_DIM = 256
WORDS = 32


@dataclass
class Tq4LayerPool:
    k_words: torch.Tensor
    v_words: torch.Tensor
    k_norms: torch.Tensor
    v_norms: torch.Tensor

    @staticmethod
    def empty(num_pages: int, n_kv: int, page_size: int, device="cuda") -> "Tq4LayerPool":
        shp = (num_pages, n_kv, page_size)
        return Tq4LayerPool(torch.zeros(shp + (WORDS,), dtype=torch.int32, device=device),
                            torch.zeros(shp + (WORDS,), dtype=torch.int32, device=device),
                            torch.zeros(shp, dtype=torch.int16, device=device),
                            torch.zeros(shp, dtype=torch.int16, device=device))

    @property
    def num_pages(self) -> int:
        return self.k_words.shape[0]

    @property
    def n_kv(self) -> int:
        return self.k_words.shape[1]

    @property
    def page_size(self) -> int:
        return self.k_words.shape[2]

    def struct(self) -> tq4_layer_pool:
        for t in (self.k_words, self.v_words, self.k_norms, self.v_norms):
            if not t.is_contiguous():
                raise ValueError("pool tensors must be contiguous")
        return tq4_layer_pool(self.k_words.data_ptr(), self.v_words.data_ptr(),
                              self.k_norms.data_ptr(), self.v_norms.data_ptr(),
                              self.num_pages, self.page_size, self.n_kv, HEAD_DIM)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Context for allocating a call's missing outputs and workspace on the stream the call runs
    on: their fills are then ordered before the call's kernels, and the caching allocator reuses
    the memory only for work ordered after them on that stream."""
    return torch.cuda.stream(torch.cuda.current_stream() if stream is None else stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    return {torch.float32: TQ4_F32, torch.bfloat16: TQ4_BF16, torch.float16: TQ4_F16}.get(t.dtype, 99)


def tq4_abi_version() -> int:
    return load_library().tq4_abi_version()


def tq4_codebook():
    """(centroids[16], thresholds[15]) as Python floats (host)."""
    c = (ctypes.c_float * 16)()
    b = (ctypes.c_float * 15)()
    check(load_library().tq4_codebook(c, b))
    return list(c), list(b)


def tq4_encode_pages(pool: Tq4LayerPool, k, v, slots: torch.Tensor, stream=None) -> None:
    """Encode [n_tokens][n_kv][256] fp32/bf16 K and/or V into the records at slots (int32)."""
    src = k if k is not None else v
    if src is None:
        raise ValueError("need k or v")
    for t in (k, v):
        if t is not None and not t.is_contiguous():
            raise ValueError("sources must be contiguous")
    n_tokens = int(slots.shape[0])
    ps = pool.struct()
    check(load_library().tq4_encode_pages(ctypes.byref(ps), _ptr(k), _ptr(v), _dtype_code(src),
                                          _ptr(slots), n_tokens, _stream(stream)))


def tq4_attn_decode_workspace_size(batch: int, max_seq_len: int, n_q_heads: int, n_kv_heads: int,
                                   page_size: int) -> int:
    return int(load_library().tq4_attn_decode_workspace_size(batch, max_seq_len, n_q_heads,
                                                              n_kv_heads, page_size))


def tq4_attn_verify_workspace_size(batch: int, max_seq_len: int, n_queries: int, n_q_heads: int,
                                   n_kv_heads: int, page_size: int) -> int:
    return int(load_library().tq4_attn_verify_workspace_size(batch, max_seq_len, n_queries, n_q_heads,
                                                              n_kv_heads, page_size))


def tq4_attn_prefill_workspace_size(prior_len: int, chunk_len: int, n_q_heads: int, n_kv_heads: int,
                                    page_size: int) -> int:
    return int(load_library().tq4_attn_prefill_workspace_size(prior_len, chunk_len, n_q_heads,
                                                               n_kv_heads, page_size))


def new_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A workspace buffer of at least 256 bytes, allocated on the current stream (the calls do not
    read its contents on entry, so it is not cleared)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def tq4_attn_decode(pool: Tq4LayerPool, q: torch.Tensor, page_table: torch.Tensor,
                    seq_lens: torch.Tensor, max_seq_len: int, scale: float,
                    out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """q [batch][n_q][256] bf16; page_table int32 [batch][stride]; seq_lens int32 [batch]."""
    batch, n_q, _ = q.shape
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = new_workspace(tq4_attn_decode_workspace_size(batch, max_seq_len, n_q, pool.n_kv,
                                                                     pool.page_size), q.device)
    ps = pool.struct()
    check(load_library().tq4_attn_decode(
        ctypes.byref(ps), _ptr(q), _dtype_code(q), _ptr(page_table), int(page_table.shape[1]),
        _ptr(seq_lens), batch, int(max_seq_len), n_q, float(scale), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


DECODE_VARIANTS = {"fused": 0, "valu_rotated": 1, "valu_literal": 2}


def tq4_attn_decode_variant(pool: Tq4LayerPool, q: torch.Tensor, page_table: torch.Tensor,
                            seq_lens: torch.Tensor, max_seq_len: int, scale: float, variant: str,
                            out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                            stream=None) -> torch.Tensor:
    """tq4_attn_decode computed another way: "fused" (the fused kernel), "valu_rotated" (the same
    rotated-domain arithmetic without matrix cores) or "valu_literal" (per-key fp32 reconstruction
    and natural-domain attention).  Same workspace as tq4_attn_decode."""
    batch, n_q, _ = q.shape
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = new_workspace(tq4_attn_decode_workspace_size(batch, max_seq_len, n_q, pool.n_kv,
                                                                     pool.page_size), q.device)
    ps = pool.struct()
    check(load_library().tq4_attn_decode_variant(
        ctypes.byref(ps), _ptr(q), _dtype_code(q), _ptr(page_table), int(page_table.shape[1]),
        _ptr(seq_lens), batch, int(max_seq_len), n_q, float(scale), DECODE_VARIANTS[variant], _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def tq4_attn_decode_noalloc(pool: Tq4LayerPool, q: torch.Tensor, page_table: torch.Tensor,
                            seq_lens: torch.Tensor, max_seq_len: int, scale: float,
                            out: torch.Tensor, stream=None) -> torch.Tensor:
    """tq4_attn_decode without a workspace (the library's per-device scratch holds the split
    partials): nothing is allocated, so `out` must be given.  Calls that may overlap on one GPU
    race on the scratch."""
    batch, n_q, _ = q.shape
    ps = pool.struct()
    check(load_library().tq4_attn_decode_noalloc(
        ctypes.byref(ps), _ptr(q), _dtype_code(q), _ptr(page_table), int(page_table.shape[1]),
        _ptr(seq_lens), batch, int(max_seq_len), n_q, float(scale), _ptr(out), _stream(stream)))
    return out


def tq4_attn_decode_append(pool: Tq4LayerPool, k_new, v_new, new_slots: torch.Tensor, q: torch.Tensor,
                           page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, scale: float,
                           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                           stream=None) -> torch.Tensor:
    """Encode each request's new token (k_new / v_new [batch][n_kv][256] fp32 or bf16, written at
    new_slots[b], the slot of position seq_lens[b] - 1) and attend, in one call."""
    batch, n_q, _ = q.shape
    src = k_new if k_new is not None else v_new
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = new_workspace(tq4_attn_decode_workspace_size(batch, max_seq_len, n_q, pool.n_kv,
                                                                     pool.page_size), q.device)
    ps = pool.struct()
    check(load_library().tq4_attn_decode_append(
        ctypes.byref(ps), _ptr(k_new), _ptr(v_new), _dtype_code(src), _ptr(new_slots), _ptr(q), _dtype_code(q),
        _ptr(page_table), int(page_table.shape[1]), _ptr(seq_lens), batch, int(max_seq_len), n_q, float(scale),
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def tq4_attn_verify(pool: Tq4LayerPool, q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                    max_seq_len: int, scale: float, out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """q [batch][n_queries][n_q][256] bf16: the last n_queries cached positions of each request
    (seq_lens[b] counts them); query i attends positions 0 .. seq_lens[b] - n_queries + i."""
    batch, n_queries, n_q, _ = q.shape
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = new_workspace(tq4_attn_verify_workspace_size(batch, max_seq_len, n_queries, n_q, pool.n_kv,
                                                                     pool.page_size), q.device)
    ps = pool.struct()
    check(load_library().tq4_attn_verify(
        ctypes.byref(ps), _ptr(q), _dtype_code(q), n_queries, _ptr(page_table), int(page_table.shape[1]),
        _ptr(seq_lens), batch, int(max_seq_len), n_q, float(scale), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def tq4_reconstruct_pages(pool: Tq4LayerPool, page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                          k_out: torch.Tensor | None = None, v_out: torch.Tensor | None = None, stream=None):
    """bf16 K and V [batch][n_kv][max_seq_len][256] of every cached position (rows past a request's
    length are left as they were)."""
    batch = int(seq_lens.shape[0])
    shape = (batch, pool.n_kv, int(max_seq_len), HEAD_DIM)
    dev = pool.k_words.device
    with _on(stream):
        if k_out is None:
            k_out = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
        if v_out is None:
            v_out = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    ps = pool.struct()
    check(load_library().tq4_reconstruct_pages(
        ctypes.byref(ps), _ptr(page_table), int(page_table.shape[1]), _ptr(seq_lens), batch, int(max_seq_len),
        _dtype_code(k_out), _ptr(k_out), _ptr(v_out), _stream(stream)))
    return k_out, v_out


def tq4_sdpa_decode_workspace_size(batch: int, max_seq_len: int, n_q_heads: int, n_kv_heads: int) -> int:
    return int(load_library().tq4_sdpa_decode_workspace_size(batch, max_seq_len, n_q_heads, n_kv_heads))


def tq4_sdpa_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                    out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """q [batch][n_q][256] bf16 over dense k, v [batch][n_kv][max_seq_len][256] bf16."""
    batch, n_q, _ = q.shape
    n_kv, max_seq = int(k.shape[1]), int(k.shape[2])
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = new_workspace(tq4_sdpa_decode_workspace_size(batch, max_seq, n_q, n_kv), q.device)
    check(load_library().tq4_sdpa_decode(
        _ptr(q), _dtype_code(q), _ptr(k), _ptr(v), _dtype_code(k), _ptr(seq_lens), batch, max_seq, n_q, n_kv,
        float(scale), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def tq4_attn_prefill_chunk(pool: Tq4LayerPool, q: torch.Tensor, page_table: torch.Tensor,
                           prior_len: int, scale: float, out: torch.Tensor | None = None,
                           workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """q [chunk_len][n_q][256] bf16; page_table int32 covering prior_len + chunk_len positions."""
    chunk_len, n_q, _ = q.shape
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = new_workspace(tq4_attn_prefill_workspace_size(prior_len, chunk_len, n_q, pool.n_kv,
                                                                      pool.page_size), q.device)
    ps = pool.struct()
    check(load_library().tq4_attn_prefill_chunk(
        ctypes.byref(ps), _ptr(q), _dtype_code(q), _ptr(page_table), int(prior_len), chunk_len, n_q,
        float(scale), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


@dataclass
class Int8LayerPool:
    """One layer's pool of uniform INT8 records (codes and fp16 scales)."""
    k_codes: torch.Tensor
    v_codes: torch.Tensor
    k_scales: torch.Tensor
    v_scales: torch.Tensor

    @staticmethod
    def empty(num_pages: int, n_kv: int, page_size: int, device="cuda") -> "Int8LayerPool":
        shp = (num_pages, n_kv, page_size)
        return Int8LayerPool(torch.zeros(shp + (HEAD_DIM,), dtype=torch.int8, device=device),
                             torch.zeros(shp + (HEAD_DIM,), dtype=torch.int8, device=device),
                             torch.zeros(shp, dtype=torch.int16, device=device),
                             torch.zeros(shp, dtype=torch.int16, device=device))

    @property
    def num_pages(self) -> int:
        return self.k_codes.shape[0]

    @property
    def n_kv(self) -> int:
        return self.k_codes.shape[1]

    @property
    def page_size(self) -> int:
        return self.k_codes.shape[2]

    def struct(self) -> tq4_int8_pool:
        for t in (self.k_codes, self.v_codes, self.k_scales, self.v_scales):
            if not t.is_contiguous():
                raise ValueError("pool tensors must be contiguous")
        return tq4_int8_pool(self.k_codes.data_ptr(), self.v_codes.data_ptr(),
                             self.k_scales.data_ptr(), self.v_scales.data_ptr(),
                             self.num_pages, self.page_size, self.n_kv, HEAD_DIM)


def tq4_int8_encode_pages(pool: Int8LayerPool, k, v, slots: torch.Tensor, stream=None) -> None:
    """Encode [n_tokens][n_kv][256] fp32/bf16 K and/or V into INT8 records at slots (int32)."""
    src = k if k is not None else v
    if src is None:
        raise ValueError("need k or v")
    for t in (k, v):
        if t is not None and not t.is_contiguous():
            raise ValueError("sources must be contiguous")
    ps = pool.struct()
    check(load_library().tq4_int8_encode_pages(ctypes.byref(ps), _ptr(k), _ptr(v), _dtype_code(src),
                                               _ptr(slots), int(slots.shape[0]), _stream(stream)))


def tq4_int8_attn_decode_workspace_size(batch: int, max_seq_len: int, n_q_heads: int, n_kv_heads: int,
                                        page_size: int) -> int:
    return int(load_library().tq4_int8_attn_decode_workspace_size(batch, max_seq_len, n_q_heads,
                                                                   n_kv_heads, page_size))


def tq4_int8_attn_decode(pool: Int8LayerPool, q: torch.Tensor, page_table: torch.Tensor,
                         seq_lens: torch.Tensor, max_seq_len: int, scale: float,
                         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                         stream=None) -> torch.Tensor:
    """q [batch][n_q][256] bf16 over INT8 pages; page_table int32 [batch][stride]; seq_lens int32 [batch]."""
    batch, n_q, _ = q.shape
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = new_workspace(tq4_int8_attn_decode_workspace_size(batch, max_seq_len, n_q, pool.n_kv,
                                                                          pool.page_size), q.device)
    prepare_int8_decode(pool, q, page_table, seq_lens, max_seq_len, scale, out, workspace, stream)()
    return out


def tq4_int8_attn_decode_append(pool: Int8LayerPool, k_new, v_new, new_slots: torch.Tensor, q: torch.Tensor,
                                page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, scale: float,
                                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                                stream=None) -> torch.Tensor:
    """INT8 pages: encode each request's new token (k_new / v_new [batch][n_kv][256] fp32 or bf16,
    written at new_slots[b], the slot of position seq_lens[b] - 1) and attend, in one call."""
    batch, n_q, _ = q.shape
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = new_workspace(tq4_int8_attn_decode_workspace_size(batch, max_seq_len, n_q, pool.n_kv,
                                                                          pool.page_size), q.device)
    prepare_int8_decode_append(pool, k_new, v_new, new_slots, q, page_table, seq_lens, max_seq_len, scale, out,
                               workspace, stream)()
    return out


def tq4_int8_attn_verify_workspace_size(batch: int, max_seq_len: int, n_queries: int, n_q_heads: int,
                                        n_kv_heads: int, page_size: int) -> int:
    return int(load_library().tq4_int8_attn_verify_workspace_size(batch, max_seq_len, n_queries, n_q_heads,
                                                                   n_kv_heads, page_size))


def tq4_int8_attn_verify(pool: Int8LayerPool, q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                         max_seq_len: int, scale: float, out: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """q [batch][n_queries][n_q][256] bf16: the last n_queries positions of each request, causal."""
    batch, n_queries, n_q, _ = q.shape
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = new_workspace(tq4_int8_attn_verify_workspace_size(batch, max_seq_len, n_queries, n_q, pool.n_kv,
                                                                          pool.page_size), q.device)
    prepare_int8_verify(pool, q, page_table, seq_lens, max_seq_len, scale, out, workspace, stream)()
    return out


def tq4_int8_attn_prefill_workspace_size(prior_len: int, chunk_len: int, n_q_heads: int, n_kv_heads: int,
                                         page_size: int) -> int:
    return int(load_library().tq4_int8_attn_prefill_workspace_size(prior_len, chunk_len, n_q_heads,
                                                                    n_kv_heads, page_size))


def tq4_int8_attn_prefill_chunk(pool: Int8LayerPool, q: torch.Tensor, page_table: torch.Tensor, prior_len: int,
                                scale: float, out: torch.Tensor | None = None,
                                workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """q [chunk_len][n_q][256] bf16 over INT8 pages; page_table int32 covering prior_len + chunk_len positions."""
    chunk_len, n_q, _ = q.shape
    with _on(stream):
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            workspace = new_workspace(tq4_int8_attn_prefill_workspace_size(prior_len, chunk_len, n_q, pool.n_kv,
                                                                           pool.page_size), q.device)
    prepare_int8_prefill(pool, q, page_table, prior_len, scale, out, workspace, stream)()
    return out


class PreparedCall:
    """A library call with its ctypes arguments marshalled once.

    Calling it repeats the same C call (same pointers, same stream), which
    keeps Python overhead out of tight launch loops such as a decode step over
    many layers.  The tensors it was built from must stay alive."""

    def __init__(self, fn, args, keep):
        self._fn, self._args, self._keep = fn, args, keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != 0:
            check(st)


def prepare_encode(pool: Tq4LayerPool, k, v, slots: torch.Tensor, stream=None) -> PreparedCall:
    src = k if k is not None else v
    ps = pool.struct()
    args = (ctypes.byref(ps), _ptr(k), _ptr(v), _dtype_code(src), _ptr(slots), int(slots.shape[0]),
            _stream(stream))
    return PreparedCall(load_library().tq4_encode_pages, args, (ps, pool, k, v, slots))


def prepare_decode(pool: Tq4LayerPool, q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                   max_seq_len: int, scale: float, out: torch.Tensor, workspace: torch.Tensor,
                   stream=None) -> PreparedCall:
    batch, n_q, _ = q.shape
    ps = pool.struct()
    args = (ctypes.byref(ps), _ptr(q), _dtype_code(q), _ptr(page_table), int(page_table.shape[1]),
            _ptr(seq_lens), batch, int(max_seq_len), n_q, ctypes.c_float(scale), _ptr(out),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    return PreparedCall(load_library().tq4_attn_decode, args, (ps, pool, q, page_table, seq_lens, out, workspace))


def prepare_decode_variant(pool: Tq4LayerPool, q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                           max_seq_len: int, scale: float, variant: str, out: torch.Tensor, workspace: torch.Tensor,
                           stream=None) -> PreparedCall:
    batch, n_q, _ = q.shape
    ps = pool.struct()
    args = (ctypes.byref(ps), _ptr(q), _dtype_code(q), _ptr(page_table), int(page_table.shape[1]),
            _ptr(seq_lens), batch, int(max_seq_len), n_q, ctypes.c_float(scale), DECODE_VARIANTS[variant],
            _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    return PreparedCall(load_library().tq4_attn_decode_variant, args,
                        (ps, pool, q, page_table, seq_lens, out, workspace))


def prepare_verify(pool: Tq4LayerPool, q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                   max_seq_len: int, scale: float, out: torch.Tensor, workspace: torch.Tensor,
                   stream=None) -> PreparedCall:
    batch, n_queries, n_q, _ = q.shape
    ps = pool.struct()
    args = (ctypes.byref(ps), _ptr(q), _dtype_code(q), n_queries, _ptr(page_table), int(page_table.shape[1]),
            _ptr(seq_lens), batch, int(max_seq_len), n_q, ctypes.c_float(scale), _ptr(out),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    return PreparedCall(load_library().tq4_attn_verify, args, (ps, pool, q, page_table, seq_lens, out, workspace))


def prepare_reconstruct(pool: Tq4LayerPool, page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                        k_out: torch.Tensor, v_out: torch.Tensor, stream=None) -> PreparedCall:
    ps = pool.struct()
    args = (ctypes.byref(ps), _ptr(page_table), int(page_table.shape[1]), _ptr(seq_lens), int(seq_lens.shape[0]),
            int(max_seq_len), _dtype_code(k_out), _ptr(k_out), _ptr(v_out), _stream(stream))
    return PreparedCall(load_library().tq4_reconstruct_pages, args, (ps, pool, page_table, seq_lens, k_out, v_out))


def prepare_sdpa_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                        out: torch.Tensor, workspace: torch.Tensor, stream=None) -> PreparedCall:
    batch, n_q, _ = q.shape
    args = (_ptr(q), _dtype_code(q), _ptr(k), _ptr(v), _dtype_code(k), _ptr(seq_lens), batch, int(k.shape[2]), n_q,
            int(k.shape[1]), ctypes.c_float(scale), _ptr(out), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    return PreparedCall(load_library().tq4_sdpa_decode, args, (q, k, v, seq_lens, out, workspace))


def prepare_prefill(pool: Tq4LayerPool, q: torch.Tensor, page_table: torch.Tensor, prior_len: int,
                    scale: float, out: torch.Tensor, workspace: torch.Tensor, stream=None) -> PreparedCall:
    chunk_len, n_q, _ = q.shape
    ps = pool.struct()
    args = (ctypes.byref(ps), _ptr(q), _dtype_code(q), _ptr(page_table), int(prior_len), chunk_len, n_q,
            ctypes.c_float(scale), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(stream))
    return PreparedCall(load_library().tq4_attn_prefill_chunk, args, (ps, pool, q, page_table, out, workspace))


def prepare_decode_append(pool: Tq4LayerPool, k_new, v_new, new_slots: torch.Tensor, q: torch.Tensor,
                          page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, scale: float,
                          out: torch.Tensor, workspace: torch.Tensor, stream=None) -> PreparedCall:
    batch, n_q, _ = q.shape
    src = k_new if k_new is not None else v_new
    ps = pool.struct()
    args = (ctypes.byref(ps), _ptr(k_new), _ptr(v_new), _dtype_code(src), _ptr(new_slots), _ptr(q), _dtype_code(q),
            _ptr(page_table), int(page_table.shape[1]), _ptr(seq_lens), batch, int(max_seq_len), n_q,
            ctypes.c_float(scale), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(stream))
    return PreparedCall(load_library().tq4_attn_decode_append, args,
                        (ps, pool, k_new, v_new, new_slots, q, page_table, seq_lens, out, workspace))


def prepare_int8_decode(pool: Int8LayerPool, q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                        max_seq_len: int, scale: float, out: torch.Tensor, workspace: torch.Tensor,
                        stream=None) -> PreparedCall:
    batch, n_q, _ = q.shape
    ps = pool.struct()
    args = (ctypes.byref(ps), _ptr(q), _dtype_code(q), _ptr(page_table), int(page_table.shape[1]),
            _ptr(seq_lens), batch, int(max_seq_len), n_q, ctypes.c_float(scale), _ptr(out),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    return PreparedCall(load_library().tq4_int8_attn_decode, args,
                        (ps, pool, q, page_table, seq_lens, out, workspace))


def prepare_int8_decode_append(pool: Int8LayerPool, k_new, v_new, new_slots: torch.Tensor, q: torch.Tensor,
                               page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, scale: float,
                               out: torch.Tensor, workspace: torch.Tensor, stream=None) -> PreparedCall:
    batch, n_q, _ = q.shape
    src = k_new if k_new is not None else v_new
    ps = pool.struct()
    args = (ctypes.byref(ps), _ptr(k_new), _ptr(v_new), _dtype_code(src), _ptr(new_slots), _ptr(q), _dtype_code(q),
            _ptr(page_table), int(page_table.shape[1]), _ptr(seq_lens), batch, int(max_seq_len), n_q,
            ctypes.c_float(scale), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(stream))
    return PreparedCall(load_library().tq4_int8_attn_decode_append, args,
                        (ps, pool, k_new, v_new, new_slots, q, page_table, seq_lens, out, workspace))


def prepare_int8_verify(pool: Int8LayerPool, q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                        max_seq_len: int, scale: float, out: torch.Tensor, workspace: torch.Tensor,
                        stream=None) -> PreparedCall:
    batch, n_queries, n_q, _ = q.shape
    ps = pool.struct()
    args = (ctypes.byref(ps), _ptr(q), _dtype_code(q), n_queries, _ptr(page_table), int(page_table.shape[1]),
            _ptr(seq_lens), batch, int(max_seq_len), n_q, ctypes.c_float(scale), _ptr(out),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    return PreparedCall(load_library().tq4_int8_attn_verify, args,
                        (ps, pool, q, page_table, seq_lens, out, workspace))


def prepare_int8_prefill(pool: Int8LayerPool, q: torch.Tensor, page_table: torch.Tensor, prior_len: int,
                         scale: float, out: torch.Tensor, workspace: torch.Tensor, stream=None) -> PreparedCall:
    chunk_len, n_q, _ = q.shape
    ps = pool.struct()
    args = (ctypes.byref(ps), _ptr(q), _dtype_code(q), _ptr(page_table), int(prior_len), chunk_len, n_q,
            ctypes.c_float(scale), _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(stream))
    return PreparedCall(load_library().tq4_int8_attn_prefill_chunk, args, (ps, pool, q, page_table, out, workspace))
