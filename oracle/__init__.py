"""CPU oracle for the TQ4 paged KV codec and attention over it.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the GPU library and
its Python binding never do, and this package never imports them.

The arithmetic lives in ``tq4_oracle.c`` (plain scalar C, fp64 attention, the
encoder in fp32 as the readings there fix it); this module only builds that
file with gcc, loads it with ctypes and marshals numpy arrays.

Sources, by page and section:
  * "Fitting a 27B-Parameter LLM into 24 GiB of Laptop Memory"
    (simpleprog.com), section "KVExec: Fused Reconstruction with
    Layer-Scoped Lifetime" -- record format (32 U32 words of eight indices,
    one FP16 norm) and the decode steps (page IDs, centroid lookup, inverse
    Hadamard rotation, norm restore, scaled dot-product attention).
  * same page, section "The Memory Budget Equation" -- 4 KV heads of
    dimension 256, 16 full-attention layers, 16,640 B per position vs
    65,536 B in FP16, 3,640 MiB vs 14,336 MiB at 229,376 positions, and
    768 MiB of BF16 K/V for one layer at 192K positions.
  * same page, section "Reasoning at 200K: 29 of 30 AIME Problems" -- the
    uniform INT8 KV comparison arm (per-vector symmetric INT8 with an fp16
    scale, natural domain: the page fixes no format, this is the reading).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tq4_oracle.c")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libtq4oracle.so")

DIM = 256
WORDS = 32
LEVELS = 16

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no contraction)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off",
               "-fno-fast-math", "-fPIC", "-shared", SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    c_f32p, c_f64p = P(ctypes.c_float), P(ctypes.c_double)
    c_u32p, c_u16p, c_i32p = P(ctypes.c_uint32), P(ctypes.c_uint16), P(ctypes.c_int32)
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    lib.tq4o_lloyd_max16.argtypes = [c_f64p, c_f64p, c_f64p, ctypes.c_int]
    lib.tq4o_lloyd_max16.restype = ctypes.c_int
    lib.tq4o_codebook.argtypes = [c_f32p, c_f32p]
    lib.tq4o_f32_to_f16_array.argtypes = [c_f32p, c_u16p, i64]
    lib.tq4o_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.tq4o_f16_to_f64.restype = ctypes.c_double
    lib.tq4o_encode_many.argtypes = [c_f32p, i64, c_u32p, c_u16p]
    lib.tq4o_decode_many.argtypes = [c_u32p, c_u16p, i64, c_f64p]
    lib.tq4o_fwht_f32_many.argtypes = [c_f32p, i64]
    lib.tq4o_fwht_f64_many.argtypes = [c_f64p, i64]
    lib.tq4o_encode_to_pool.argtypes = [c_u32p, c_u16p, i32, i32, i32, c_f32p, c_i32p, i32]
    lib.tq4o_encode_to_pool.restype = ctypes.c_int
    lib.tq4o_attention.argtypes = [c_u32p, c_u16p, c_u32p, c_u16p, i32, i32, i32,
                                   c_f64p, i32, i32, c_i32p, i32, c_i32p, c_i32p,
                                   ctypes.c_double, i32, i32, c_f64p]
    lib.tq4o_attention.restype = ctypes.c_int
    lib.tq4o_f64_to_bf16_array.argtypes = [c_f64p, c_u16p, i64]
    lib.tq4o_reconstruct.argtypes = [c_u32p, c_u16p, c_u32p, c_u16p, i32, i32, i32, c_i32p, i32, c_i32p,
                                     i32, i32, c_u16p, c_u16p]
    lib.tq4o_reconstruct.restype = ctypes.c_int
    lib.tq4o_sdpa_dense.argtypes = [c_f64p, c_f64p, c_f64p, i32, i32, i32, i32, c_i32p, ctypes.c_double, c_f64p]
    lib.tq4o_sdpa_dense.restype = ctypes.c_int
    c_i8p = P(ctypes.c_int8)
    lib.tq4o_int8_encode_many.argtypes = [c_f32p, i64, c_i8p, c_u16p]
    lib.tq4o_int8_decode_many.argtypes = [c_i8p, c_u16p, i64, c_f64p]
    lib.tq4o_int8_encode_to_pool.argtypes = [c_i8p, c_u16p, i32, i32, i32, c_f32p, c_i32p, i32]
    lib.tq4o_int8_encode_to_pool.restype = ctypes.c_int
    lib.tq4o_int8_attention.argtypes = [c_i8p, c_u16p, c_i8p, c_u16p, i32, i32, i32,
                                        c_f64p, i32, i32, c_i32p, i32, c_i32p, c_i32p,
                                        ctypes.c_double, i32, i32, c_f64p]
    lib.tq4o_int8_attention.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# --------------------------------------------------------------------------
# Constants
# --------------------------------------------------------------------------

def lloyd_max16(max_iter: int = 1_000_000):
    """Lloyd-Max levels/boundaries for N(0,1), 16 levels, in fp64.

    Returns (levels[16], bounds[15], distortion, iterations)."""
    lib = _load()
    lev = np.zeros(LEVELS, np.float64)
    bnd = np.zeros(LEVELS - 1, np.float64)
    dist = ctypes.c_double(0.0)
    it = lib.tq4o_lloyd_max16(_ptr(lev, ctypes.c_double), _ptr(bnd, ctypes.c_double),
                              ctypes.byref(dist), max_iter)
    return lev, bnd, dist.value, it


def codebook():
    """(centroids fp32[16] ascending, thresholds fp32[15])."""
    lib = _load()
    c = np.zeros(LEVELS, np.float32)
    b = np.zeros(LEVELS - 1, np.float32)
    lib.tq4o_codebook(_ptr(c, ctypes.c_float), _ptr(b, ctypes.c_float))
    return c, b


# --------------------------------------------------------------------------
# Elementwise helpers
# --------------------------------------------------------------------------

def f32_to_f16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(x.shape, np.uint16)
    _load().tq4o_f32_to_f16_array(_ptr(x.reshape(-1), ctypes.c_float),
                                  _ptr(out.reshape(-1), ctypes.c_uint16), x.size)
    return out


def f16_bits_to_f64(h) -> np.ndarray:
    lib = _load()
    h = np.asarray(h, dtype=np.uint16)
    return np.array([lib.tq4o_f16_to_f64(int(v)) for v in h.reshape(-1)],
                    np.float64).reshape(h.shape)


def fwht_f32(x) -> np.ndarray:
    y = np.array(x, dtype=np.float32, copy=True, order="C").reshape(-1, DIM)
    _load().tq4o_fwht_f32_many(_ptr(y, ctypes.c_float), y.shape[0])
    return y.reshape(np.shape(x))


def fwht_f64(x) -> np.ndarray:
    y = np.array(x, dtype=np.float64, copy=True, order="C").reshape(-1, DIM)
    _load().tq4o_fwht_f64_many(_ptr(y, ctypes.c_double), y.shape[0])
    return y.reshape(np.shape(x))


# --------------------------------------------------------------------------
# Codec
# --------------------------------------------------------------------------

def encode(x):
    """Encode fp32 vectors [..., 256] -> (words uint32 [..., 32], norms uint16 [...])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape[-1] == DIM
    lead = x.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    words = np.zeros((n, WORDS), np.uint32)
    norms = np.zeros((n,), np.uint16)
    _load().tq4o_encode_many(_ptr(x.reshape(n, DIM), ctypes.c_float), n,
                             _ptr(words, ctypes.c_uint32), _ptr(norms, ctypes.c_uint16))
    return words.reshape(*lead, WORDS), norms.reshape(lead)


def decode(words, norms) -> np.ndarray:
    """Exact fp64 reconstruction of records (words [..., 32], norms [...])."""
    words = np.ascontiguousarray(words, dtype=np.uint32)
    norms = np.ascontiguousarray(norms, dtype=np.uint16)
    lead = norms.shape
    n = int(np.prod(lead)) if lead else 1
    out = np.zeros((n, DIM), np.float64)
    _load().tq4o_decode_many(_ptr(words.reshape(n, WORDS), ctypes.c_uint32),
                             _ptr(norms.reshape(n), ctypes.c_uint16), n,
                             _ptr(out, ctypes.c_double))
    return out.reshape(*lead, DIM)


def unpack(words) -> np.ndarray:
    """Indices [..., 256] of packed words [..., 32] (dim 8k+j in bits 4j.. of word k)."""
    w = np.asarray(words, dtype=np.uint32)
    shifts = (4 * np.arange(8, dtype=np.uint32))
    idx = (w[..., :, None] >> shifts) & np.uint32(0xF)
    return idx.reshape(*w.shape[:-1], DIM).astype(np.uint8)


def pack(idx) -> np.ndarray:
    idx = np.asarray(idx, dtype=np.uint32).reshape(*np.shape(idx)[:-1], WORDS, 8)
    shifts = (4 * np.arange(8, dtype=np.uint32))
    return np.bitwise_or.reduce(idx << shifts, axis=-1).astype(np.uint32)


# --------------------------------------------------------------------------
# Paged pools
# --------------------------------------------------------------------------

@dataclass
class Pool:
    """One layer's TQ4 page pool (host arrays).

    words: uint32 [num_pages][n_kv][P][32]; norms: fp16 bits [num_pages][n_kv][P]."""
    k_words: np.ndarray
    k_norms: np.ndarray
    v_words: np.ndarray
    v_norms: np.ndarray

    @property
    def num_pages(self):
        return self.k_words.shape[0]

    @property
    def n_kv(self):
        return self.k_words.shape[1]

    @property
    def page_size(self):
        return self.k_words.shape[2]

    @staticmethod
    def empty(num_pages: int, n_kv: int, page_size: int) -> "Pool":
        shp = (num_pages, n_kv, page_size)
        return Pool(np.zeros(shp + (WORDS,), np.uint32), np.zeros(shp, np.uint16),
                    np.zeros(shp + (WORDS,), np.uint32), np.zeros(shp, np.uint16))


def encode_to_pool(pool: Pool, k_src, v_src, slots) -> None:
    """Encode source K and V [n_tokens][n_kv][256] (fp32) into records at slots."""
    lib = _load()
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    for src, words, norms in ((k_src, pool.k_words, pool.k_norms),
                              (v_src, pool.v_words, pool.v_norms)):
        if src is None:
            continue
        src = np.ascontiguousarray(src, dtype=np.float32)
        assert src.shape == (slots.shape[0], pool.n_kv, DIM)
        rc = lib.tq4o_encode_to_pool(_ptr(words, ctypes.c_uint32), _ptr(norms, ctypes.c_uint16),
                                     pool.num_pages, pool.n_kv, pool.page_size,
                                     _ptr(src, ctypes.c_float), _ptr(slots, ctypes.c_int32),
                                     slots.shape[0])
        if rc != 0:
            raise ValueError("slot outside the pool")


def attention(pool: Pool, q, page_table, row_table, row_len, scale: float,
              heads: tuple | None = None) -> np.ndarray:
    """fp64 softmax attention over TQ4 pages.

    q: [n_rows][n_q][256] (values exactly representable in fp64, e.g. bf16 inputs);
    page_table: int32 [n_tables][stride]; row_table[r]: which table row query
    row r reads; row_len[r]: how many leading positions it attends.
    Returns fp64 [n_rows][n_q][256]; heads outside `heads` = (h0, h1) stay 0."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    n_rows, n_q, d = q.shape
    assert d == DIM and n_q % pool.n_kv == 0
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    if pt.ndim == 1:
        pt = pt[None, :]
    rt = np.ascontiguousarray(row_table, dtype=np.int32)
    rl = np.ascontiguousarray(row_len, dtype=np.int32)
    assert rt.shape == (n_rows,) and rl.shape == (n_rows,)
    h0, h1 = heads if heads is not None else (0, n_q)
    out = np.zeros((n_rows, n_q, DIM), np.float64)
    rc = _load().tq4o_attention(
        _ptr(pool.k_words, ctypes.c_uint32), _ptr(pool.k_norms, ctypes.c_uint16),
        _ptr(pool.v_words, ctypes.c_uint32), _ptr(pool.v_norms, ctypes.c_uint16),
        pool.num_pages, pool.n_kv, pool.page_size, _ptr(q, ctypes.c_double), n_q, n_rows,
        _ptr(pt, ctypes.c_int32), pt.shape[1], _ptr(rt, ctypes.c_int32), _ptr(rl, ctypes.c_int32),
        float(scale), h0, h1, _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"oracle attention failed ({rc})")
    return out


def attn_decode(pool: Pool, q, page_table, seq_lens, scale: float, heads=None) -> np.ndarray:
    """Single-query decode for each request b: q[b] attends positions 0..seq_lens[b]-1."""
    q = np.asarray(q)
    batch = q.shape[0]
    return attention(pool, q, page_table, np.arange(batch, dtype=np.int32),
                     np.asarray(seq_lens, np.int32), scale, heads)


def attn_verify(pool: Pool, q, page_table, seq_lens, scale: float, heads=None) -> np.ndarray:
    """Packed multi-query verification ("Fitting a 27B-Parameter LLM into 24 GiB of Laptop Memory",
    section "KVExec: Fused Reconstruction with Layer-Scoped Lifetime": a packed verifier is one of
    the multi-query paths).  q: [batch][k][n_q][256]; the k queries of request b are its last k
    cached positions, so query i sits at position L - k + i (L = seq_lens[b]) and attends positions
    0 .. L - k + i; a query with no such position gets zeros.  Returns [batch][k][n_q][256]."""
    q = np.asarray(q)
    batch, k = q.shape[0], q.shape[1]
    L = np.asarray(seq_lens, np.int64)
    rows = np.repeat(np.arange(batch, dtype=np.int32), k)
    lens = np.maximum(L[:, None] - k + np.arange(k)[None, :] + 1, 0).reshape(-1).astype(np.int32)
    out = attention(pool, q.reshape(batch * k, q.shape[2], DIM), page_table, rows, lens, scale, heads)
    return out.reshape(q.shape)


def attn_prefill_rows(pool: Pool, q_rows, rows, page_table_row, prior_len: int, scale: float,
                      heads=None) -> np.ndarray:
    """Chunk rows t (absolute position prior_len + t) attend positions 0..prior_len + t."""
    rows = np.asarray(rows, np.int32)
    return attention(pool, q_rows, np.asarray(page_table_row, np.int32)[None, :],
                     np.zeros(len(rows), np.int32), prior_len + rows + 1, scale, heads)


# --------------------------------------------------------------------------
# Unfused path (section "KVExec: Fused Reconstruction with Layer-Scoped
# Lifetime": reconstruction into contiguous query-dtype K/V, then SDPA)
# --------------------------------------------------------------------------

def f64_to_bf16_bits(x) -> np.ndarray:
    """Round fp64 values to bf16 (nearest, ties to even) in one step; uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.zeros(x.shape, np.uint16)
    _load().tq4o_f64_to_bf16_array(_ptr(x.reshape(-1), ctypes.c_double),
                                   _ptr(out.reshape(-1), ctypes.c_uint16), x.size)
    return out


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bits -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def reconstruct(pool: Pool, page_table, seq_lens, max_seq_len: int):
    """bf16 bits of K and V, [batch][n_kv][max_seq_len][256]: position p < seq_lens[b] (clamped) of
    request b is the exact decode of its record rounded to bf16; later positions stay 0."""
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    if pt.ndim == 1:
        pt = pt[None, :]
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    batch = lens.shape[0]
    k = np.zeros((batch, pool.n_kv, max_seq_len, DIM), np.uint16)
    v = np.zeros_like(k)
    rc = _load().tq4o_reconstruct(
        _ptr(pool.k_words, ctypes.c_uint32), _ptr(pool.k_norms, ctypes.c_uint16),
        _ptr(pool.v_words, ctypes.c_uint32), _ptr(pool.v_norms, ctypes.c_uint16),
        pool.num_pages, pool.n_kv, pool.page_size, _ptr(pt, ctypes.c_int32), pt.shape[1],
        _ptr(lens, ctypes.c_int32), batch, int(max_seq_len), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16))
    if rc != 0:
        raise ValueError("page ID outside the pool")
    return k, v


def sdpa_dense(q, k, v, seq_lens, scale: float) -> np.ndarray:
    """fp64 attention of q [batch][n_q][256] over dense k, v [batch][n_kv][S][256] (any real dtype,
    taken exactly), keys 0 .. seq_lens[b] - 1 (clamped to [0, S])."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    batch, n_q, _ = q.shape
    n_kv, S = k.shape[1], k.shape[2]
    out = np.zeros((batch, n_q, DIM), np.float64)
    rc = _load().tq4o_sdpa_dense(_ptr(q, ctypes.c_double), _ptr(k, ctypes.c_double), _ptr(v, ctypes.c_double),
                                 batch, n_q, n_kv, S, _ptr(lens, ctypes.c_int32), float(scale),
                                 _ptr(out, ctypes.c_double))
    if rc != 0:
        raise MemoryError("oracle sdpa_dense")
    return out


# --------------------------------------------------------------------------
# Uniform INT8 arm ("Fitting a 27B-Parameter LLM into 24 GiB of Laptop Memory",
# section "Reasoning at 200K: 29 of 30 AIME Problems": a uniform INT8 KV
# comparison).  Record: 256 signed codes in [-127, 127] and one fp16 scale,
# natural domain (no rotation); decode is codes * scale.
# --------------------------------------------------------------------------

def int8_encode(x):
    """Encode fp32 vectors [..., 256] -> (codes int8 [..., 256], scales fp16 bits [...])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape[-1] == DIM
    lead = x.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    codes = np.zeros((n, DIM), np.int8)
    scales = np.zeros((n,), np.uint16)
    _load().tq4o_int8_encode_many(_ptr(x.reshape(n, DIM), ctypes.c_float), n,
                                  _ptr(codes, ctypes.c_int8), _ptr(scales, ctypes.c_uint16))
    return codes.reshape(*lead, DIM), scales.reshape(lead)


def int8_decode(codes, scales) -> np.ndarray:
    """Exact fp64 values of INT8 records (codes [..., 256], scales [...])."""
    lead = np.shape(scales)
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    n = int(np.prod(lead)) if lead else 1
    out = np.zeros((n, DIM), np.float64)
    _load().tq4o_int8_decode_many(_ptr(codes.reshape(n, DIM), ctypes.c_int8),
                                  _ptr(scales.reshape(n), ctypes.c_uint16), n, _ptr(out, ctypes.c_double))
    return out.reshape(*lead, DIM)


@dataclass
class Int8Pool:
    """One layer's INT8 page pool (host arrays).

    codes: int8 [num_pages][n_kv][P][256]; scales: fp16 bits [num_pages][n_kv][P]."""
    k_codes: np.ndarray
    k_scales: np.ndarray
    v_codes: np.ndarray
    v_scales: np.ndarray

    @property
    def num_pages(self):
        return self.k_codes.shape[0]

    @property
    def n_kv(self):
        return self.k_codes.shape[1]

    @property
    def page_size(self):
        return self.k_codes.shape[2]

    @staticmethod
    def empty(num_pages: int, n_kv: int, page_size: int) -> "Int8Pool":
        shp = (num_pages, n_kv, page_size)
        return Int8Pool(np.zeros(shp + (DIM,), np.int8), np.zeros(shp, np.uint16),
                        np.zeros(shp + (DIM,), np.int8), np.zeros(shp, np.uint16))


def int8_encode_to_pool(pool: Int8Pool, k_src, v_src, slots) -> None:
    """Encode source K and V [n_tokens][n_kv][256] (fp32) into INT8 records at slots."""
    lib = _load()
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    for src, codes, scales in ((k_src, pool.k_codes, pool.k_scales), (v_src, pool.v_codes, pool.v_scales)):
        if src is None:
            continue
        src = np.ascontiguousarray(src, dtype=np.float32)
        assert src.shape == (slots.shape[0], pool.n_kv, DIM)
        rc = lib.tq4o_int8_encode_to_pool(_ptr(codes, ctypes.c_int8), _ptr(scales, ctypes.c_uint16),
                                          pool.num_pages, pool.n_kv, pool.page_size,
                                          _ptr(src, ctypes.c_float), _ptr(slots, ctypes.c_int32), slots.shape[0])
        if rc != 0:
            raise ValueError("slot outside the pool")


def int8_attention(pool: Int8Pool, q, page_table, row_table, row_len, scale: float, heads=None) -> np.ndarray:
    """fp64 softmax attention over INT8 pages (the same contract as `attention`): query row r reads
    table row row_table[r] and attends its first row_len[r] positions.  Returns [n_rows][n_q][256];
    heads outside `heads` = (h0, h1) stay 0."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    n_rows, n_q, d = q.shape
    assert d == DIM and n_q % pool.n_kv == 0
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    if pt.ndim == 1:
        pt = pt[None, :]
    rt = np.ascontiguousarray(row_table, dtype=np.int32)
    rl = np.ascontiguousarray(row_len, dtype=np.int32)
    assert rt.shape == (n_rows,) and rl.shape == (n_rows,)
    h0, h1 = heads if heads is not None else (0, n_q)
    out = np.zeros((n_rows, n_q, DIM), np.float64)
    rc = _load().tq4o_int8_attention(
        _ptr(pool.k_codes, ctypes.c_int8), _ptr(pool.k_scales, ctypes.c_uint16),
        _ptr(pool.v_codes, ctypes.c_int8), _ptr(pool.v_scales, ctypes.c_uint16),
        pool.num_pages, pool.n_kv, pool.page_size, _ptr(q, ctypes.c_double), n_q, n_rows,
        _ptr(pt, ctypes.c_int32), pt.shape[1], _ptr(rt, ctypes.c_int32), _ptr(rl, ctypes.c_int32),
        float(scale), h0, h1, _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"oracle INT8 attention failed ({rc})")
    return out


def int8_attn_decode(pool: Int8Pool, q, page_table, seq_lens, scale: float, heads=None) -> np.ndarray:
    """fp64 single-query decode attention over INT8 pages: q[b] attends positions 0..seq_lens[b]-1
    of its page-table row.  Returns [batch][n_q][256]; heads outside `heads` stay 0."""
    batch = np.shape(q)[0]
    return int8_attention(pool, q, page_table, np.arange(batch, dtype=np.int32),
                          np.asarray(seq_lens, np.int32), scale, heads)


def int8_attn_verify(pool: Int8Pool, q, page_table, seq_lens, scale: float, heads=None) -> np.ndarray:
    """The packed multi-query verifier's definition (as attn_verify) over INT8 pages: q is
    [batch][k][n_q][256]; query i of request b attends positions 0 .. L_b - k + i."""
    q = np.asarray(q)
    batch, k = q.shape[0], q.shape[1]
    L = np.asarray(seq_lens, np.int64)
    rows = np.repeat(np.arange(batch, dtype=np.int32), k)
    lens = np.maximum(L[:, None] - k + np.arange(k)[None, :] + 1, 0).reshape(-1).astype(np.int32)
    out = int8_attention(pool, q.reshape(batch * k, q.shape[2], DIM), page_table, rows, lens, scale, heads)
    return out.reshape(q.shape)


def int8_attn_prefill_rows(pool: Int8Pool, q_rows, rows, page_table_row, prior_len: int, scale: float,
                           heads=None) -> np.ndarray:
    """Chunk rows t (absolute position prior_len + t) attend positions 0..prior_len + t over INT8 pages."""
    rows = np.asarray(rows, np.int32)
    return int8_attention(pool, q_rows, np.asarray(page_table_row, np.int32)[None, :],
                          np.zeros(len(rows), np.int32), prior_len + rows + 1, scale, heads)


def int8_bytes_per_position(n_layers: int = 16, n_kv: int = 4) -> int:
    """INT8 bytes one cached position occupies across all full-attention layers (K and V)."""
    return n_layers * n_kv * 2 * (DIM + 2)


# --------------------------------------------------------------------------
# Closed-form sizes (section "The Memory Budget Equation")
# --------------------------------------------------------------------------

def bytes_per_vector() -> int:
    """32 U32 words + one FP16 norm."""
    return WORDS * 4 + 2


def bytes_per_position(n_layers: int = 16, n_kv: int = 4) -> int:
    """TQ4 bytes one cached position occupies across all full-attention layers (K and V)."""
    return n_layers * n_kv * 2 * bytes_per_vector()


def fp16_bytes_per_position(n_layers: int = 16, n_kv: int = 4, dim: int = DIM) -> int:
    return n_layers * n_kv * 2 * dim * 2
