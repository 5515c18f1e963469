"""The C ABI on the CPU: the library loads, exports every function include/tq4.h
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes

import numpy as np
import pytest

from compressed_kv_attention_kvexec_amd import _binding as B

FAKE = 0x10000000  # never dereferenced: every case below fails host validation first


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def _pool(num_pages=8, page_size=64, n_kv=4, head_dim=256, ptr=FAKE):
    return B.tq4_layer_pool(ptr, ptr + 0x100000, ptr + 0x200000, ptr + 0x300000,
                            num_pages, page_size, n_kv, head_dim)


def test_exports_every_declared_function(lib):
    names = B.header_functions()
    assert {"tq4_encode_pages", "tq4_attn_decode", "tq4_attn_prefill_chunk"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    assert lib.tq4_abi_version() == 1
    for st in range(9):
        assert lib.tq4_status_string(st)


def test_codebook_matches_oracle_bitwise(lib, oracle_mod):
    c = (ctypes.c_float * 16)()
    b = (ctypes.c_float * 15)()
    assert lib.tq4_codebook(c, b) == 0
    oc, ob = oracle_mod.codebook()
    np.testing.assert_array_equal(np.array(c, np.float32).view(np.uint32), oc.view(np.uint32))
    np.testing.assert_array_equal(np.array(b, np.float32).view(np.uint32), ob.view(np.uint32))
    assert lib.tq4_codebook(None, b) == 1


def _decode(lib, pool=None, q=FAKE, q_dtype=B.TQ4_BF16, table=FAKE, stride=64, seq=FAKE, batch=1,
            max_seq=4000, n_q=24, out=FAKE, ws=FAKE, ws_bytes=1 << 30, scale=0.0625):
    pool = _pool() if pool is None else pool
    return lib.tq4_attn_decode(ctypes.byref(pool), q, q_dtype, table, stride, seq, batch, max_seq,
                               n_q, scale, out, ws, ws_bytes, None)


BAD_SCALES = [0.0, -0.0625, float("nan"), float("inf"), -float("inf")]


def test_softmax_scale_must_be_finite_and_positive(lib):
    """A scale <= 0 or non-finite would turn masked scores (-inf) into NaN or +inf inside the
    kernels, so every attention entry point rejects it on the host with TQ4_ERR_VALUE."""
    pool, ipool = _pool(), _i8pool()
    for sc in BAD_SCALES:
        assert _decode(lib, scale=sc) == 8, sc
        assert lib.tq4_attn_verify(ctypes.byref(pool), FAKE, B.TQ4_BF16, 4, FAKE, 64, FAKE, 1, 4000, 24,
                                   sc, FAKE, FAKE, 1 << 30, None) == 8
        assert lib.tq4_attn_decode_append(ctypes.byref(pool), FAKE, FAKE, B.TQ4_F32, FAKE, FAKE, B.TQ4_BF16,
                                          FAKE, 64, FAKE, 1, 4000, 24, sc, FAKE, FAKE, 1 << 30, None) == 8
        assert lib.tq4_attn_prefill_chunk(ctypes.byref(pool), FAKE, B.TQ4_BF16, FAKE, 100, 28, 24, sc,
                                          FAKE, FAKE, 1 << 30, None) == 8
        assert lib.tq4_sdpa_decode(FAKE, B.TQ4_BF16, FAKE, FAKE, B.TQ4_BF16, FAKE, 1, 4000, 24, 4, sc,
                                   FAKE, FAKE, 1 << 30, None) == 8
        assert lib.tq4_int8_attn_decode(ctypes.byref(ipool), FAKE, B.TQ4_BF16, FAKE, 64, FAKE, 1, 4000, 24,
                                        sc, FAKE, FAKE, 1 << 30, None) == 8
        assert lib.tq4_int8_attn_verify(ctypes.byref(ipool), FAKE, B.TQ4_BF16, 4, FAKE, 64, FAKE, 1, 4000, 24,
                                        sc, FAKE, FAKE, 1 << 30, None) == 8
        assert lib.tq4_int8_attn_prefill_chunk(ctypes.byref(ipool), FAKE, B.TQ4_BF16, FAKE, 100, 28, 24, sc,
                                               FAKE, FAKE, 1 << 30, None) == 8
    assert "scale" in lib.tq4_status_string(8).decode()


def test_decode_validation(lib):
    assert lib.tq4_attn_decode(None, FAKE, 1, FAKE, 4, FAKE, 1, 200, 24, 0.0625, FAKE, FAKE, 1 << 30, None) == 1
    assert _decode(lib, pool=_pool(head_dim=128)) == 2
    assert _decode(lib, pool=_pool(page_size=48)) == 2
    assert _decode(lib, pool=_pool(page_size=2048)) == 2
    assert _decode(lib, pool=_pool(num_pages=0)) == 2
    assert _decode(lib, pool=_pool(ptr=0)) == 1
    assert _decode(lib, q=None) == 1
    assert _decode(lib, table=None) == 1
    assert _decode(lib, seq=None) == 1
    assert _decode(lib, out=None) == 1
    assert _decode(lib, q_dtype=B.TQ4_F32) == 3
    assert _decode(lib, n_q=22) == 2           # not a multiple of 4 KV heads
    assert _decode(lib, n_q=68) == 2           # group of 17 > 16
    assert _decode(lib, batch=0) == 2
    assert _decode(lib, max_seq=0) == 2
    assert _decode(lib, max_seq=4097) == 2     # beyond stride * page_size = 4096
    assert _decode(lib, q=FAKE + 2) == 4
    assert _decode(lib, out=FAKE + 8) == 4
    assert _decode(lib, pool=_pool(ptr=FAKE + 4)) == 4
    assert _decode(lib, ws=None) == 5
    need = lib.tq4_attn_decode_workspace_size(1, 4000, 24, 4, 64)
    assert need > 0
    assert lib.tq4_attn_decode_workspace_size(1, 200, 24, 4, 64) == 0  # one split, no scratch
    assert _decode(lib, ws_bytes=need - 1) == 5
    assert _decode(lib, ws=FAKE + 128) == 4


def test_decode_workspace_size_is_bounded(lib):
    ws = lib.tq4_attn_decode_workspace_size
    assert ws(0, 100, 24, 4, 256) == 0
    assert ws(1, 100, 24, 5, 256) == 0
    assert ws(1, 100, 24, 4, 100) == 0
    # past the split cap the scratch no longer grows with the sequence
    assert ws(1, 212992, 24, 4, 256) == ws(1, 2_000_000, 24, 4, 256)
    assert ws(1, 212992, 24, 4, 256) < 4 << 20
    assert ws(2, 131072, 24, 4, 256) >= ws(1, 131072, 24, 4, 256)


def _verify(lib, n_queries=4, n_q=24, ws=FAKE, ws_bytes=1 << 30, pool=None, q=FAKE):
    pool = _pool() if pool is None else pool
    return lib.tq4_attn_verify(ctypes.byref(pool), q, B.TQ4_BF16, n_queries, FAKE, 64, FAKE, 1, 4000, n_q,
                               0.0625, FAKE, ws, ws_bytes, None)


def test_verify_validation(lib):
    assert _verify(lib, n_queries=0) == 2
    assert _verify(lib, n_queries=9) == 2        # 9 x 6 = 54 query rows > 48
    assert _verify(lib, n_queries=4, n_q=64) == 2  # 4 x 16 = 64 rows
    assert _verify(lib, n_q=22) == 2
    assert _verify(lib, q=None) == 1
    assert _verify(lib, q=FAKE + 2) == 4
    assert _verify(lib, ws=None) == 5
    vs = lib.tq4_attn_verify_workspace_size
    assert vs(1, 4000, 0, 24, 4, 64) == 0
    assert vs(1, 4000, 9, 24, 4, 64) == 0
    assert vs(1, 4000, 8, 24, 4, 64) > 0         # 48 rows: the largest packing
    # one query is decode
    for args in [(1, 4000, 24, 4, 64), (3, 212992, 24, 4, 256), (1, 200, 24, 4, 64), (2, 5000, 64, 4, 32)]:
        b, L, nq, nkv, P = args
        assert vs(b, L, 1, nq, nkv, P) == lib.tq4_attn_decode_workspace_size(*args)
    need = vs(1, 4000, 4, 24, 4, 64)
    assert need > lib.tq4_attn_decode_workspace_size(1, 4000, 24, 4, 64)
    assert _verify(lib, ws_bytes=need - 1) == 5


def test_unfused_validation(lib):
    pool = _pool()
    rec = lambda **kw: lib.tq4_reconstruct_pages(
        ctypes.byref(kw.get("pool", pool)), kw.get("table", FAKE), 64, kw.get("seq", FAKE), kw.get("batch", 1),
        kw.get("max_seq", 4000), kw.get("dtype", B.TQ4_BF16), kw.get("k", FAKE), kw.get("v", FAKE), None)
    assert rec(pool=_pool(head_dim=64)) == 2
    assert rec(table=None) == 1
    assert rec(k=None) == 1
    assert rec(dtype=B.TQ4_F32) == 3
    assert rec(batch=0) == 2
    assert rec(batch=70000) == 2
    assert rec(max_seq=4097) == 2
    assert rec(k=FAKE + 8) == 4
    sd = lambda **kw: lib.tq4_sdpa_decode(
        kw.get("q", FAKE), B.TQ4_BF16, FAKE, kw.get("v", FAKE), kw.get("kvd", B.TQ4_BF16), FAKE, 1,
        kw.get("max_seq", 4000), kw.get("n_q", 24), 4, 0.0625, FAKE, kw.get("ws", FAKE), kw.get("ws_bytes", 1 << 30),
        None)
    assert sd(q=None) == 1
    assert sd(kvd=B.TQ4_F32) == 3
    assert sd(n_q=22) == 2
    assert sd(n_q=68) == 2
    assert sd(v=FAKE + 2) == 4
    assert sd(ws=None) == 5
    need = lib.tq4_sdpa_decode_workspace_size(1, 4000, 24, 4)
    assert need > 0 and lib.tq4_sdpa_decode_workspace_size(1, 100, 24, 4) == 0
    assert sd(ws_bytes=need - 1) == 5
    assert lib.tq4_sdpa_decode_workspace_size(0, 100, 24, 4) == 0


def test_encode_validation(lib):
    pool = _pool()
    enc = lib.tq4_encode_pages
    assert enc(None, FAKE, FAKE, 0, FAKE, 3, None) == 1
    assert enc(ctypes.byref(pool), None, None, 0, FAKE, 3, None) == 1
    assert enc(ctypes.byref(pool), FAKE, FAKE, B.TQ4_F16, FAKE, 3, None) == 3
    assert enc(ctypes.byref(pool), FAKE, FAKE, 0, FAKE, -1, None) == 2
    assert enc(ctypes.byref(pool), FAKE, FAKE, 0, None, 3, None) == 1
    assert enc(ctypes.byref(pool), FAKE + 4, FAKE, 0, FAKE, 3, None) == 4
    bad = _pool(head_dim=64)
    assert enc(ctypes.byref(bad), FAKE, FAKE, 0, FAKE, 3, None) == 2
    assert enc(ctypes.byref(pool), FAKE, FAKE, 0, FAKE, 0, None) == 0  # nothing to do


def test_prefill_validation(lib):
    pool = _pool()
    pf = lib.tq4_attn_prefill_chunk
    args = dict(q=FAKE, dt=B.TQ4_BF16, table=FAKE, prior=100, chunk=16, n_q=24, out=FAKE, ws=FAKE,
                wsb=1 << 30)

    def call(**kw):
        a = dict(args, **kw)
        return pf(ctypes.byref(kw.get("pool", pool)), a["q"], a["dt"], a["table"], a["prior"],
                  a["chunk"], a["n_q"], 0.0625, a["out"], a["ws"], a["wsb"], None)

    assert call(q=None) == 1
    assert call(dt=B.TQ4_F32) == 3
    assert call(chunk=0) == 2
    assert call(prior=-1) == 2
    assert call(n_q=25) == 2
    assert call(q=FAKE + 2) == 4
    assert call(ws=None) == 5
    assert call(pool=_pool(page_size=40)) == 2
    assert lib.tq4_attn_prefill_workspace_size(100, 0, 24, 4, 256) == 0
    assert lib.tq4_attn_prefill_workspace_size(100, 16, 24, 4, 256) > 0


def _i8pool(num_pages=8, page_size=64, n_kv=4, head_dim=256, ptr=FAKE):
    return B.tq4_int8_pool(ptr, ptr + 0x100000, ptr + 0x200000, ptr + 0x300000,
                           num_pages, page_size, n_kv, head_dim)


def _i8decode(lib, pool=None, q=FAKE, q_dtype=B.TQ4_BF16, table=FAKE, stride=64, seq=FAKE, batch=1,
              max_seq=4000, n_q=24, out=FAKE, ws=FAKE, ws_bytes=1 << 30):
    pool = _i8pool() if pool is None else pool
    return lib.tq4_int8_attn_decode(ctypes.byref(pool), q, q_dtype, table, stride, seq, batch, max_seq,
                                    n_q, 0.0625, out, ws, ws_bytes, None)


def test_int8_decode_validation(lib):
    assert lib.tq4_int8_attn_decode(None, FAKE, 1, FAKE, 4, FAKE, 1, 200, 24, 0.0625, FAKE, FAKE, 1 << 30,
                                    None) == 1
    assert _i8decode(lib, pool=_i8pool(head_dim=128)) == 2
    assert _i8decode(lib, pool=_i8pool(page_size=48)) == 2
    assert _i8decode(lib, pool=_i8pool(num_pages=0)) == 2
    assert _i8decode(lib, pool=_i8pool(ptr=0)) == 1
    assert _i8decode(lib, pool=_i8pool(ptr=FAKE + 8)) == 4   # codes need 16-byte alignment
    assert _i8decode(lib, q=None) == 1
    assert _i8decode(lib, seq=None) == 1
    assert _i8decode(lib, q_dtype=B.TQ4_F32) == 3
    assert _i8decode(lib, n_q=22) == 2
    assert _i8decode(lib, n_q=68) == 2
    assert _i8decode(lib, max_seq=4097) == 2
    assert _i8decode(lib, q=FAKE + 2) == 4
    assert _i8decode(lib, ws=None) == 5
    need = lib.tq4_int8_attn_decode_workspace_size(1, 4000, 24, 4, 64)
    assert need == lib.tq4_attn_decode_workspace_size(1, 4000, 24, 4, 64) > 0
    assert _i8decode(lib, ws_bytes=need - 1) == 5
    assert _i8decode(lib, ws=FAKE + 128) == 4


def _append(lib, fn, pool, k=FAKE, v=FAKE, src=B.TQ4_F32, slots=FAKE, q=FAKE, table=FAKE, seq=FAKE, batch=1,
            max_seq=4000, ws_bytes=1 << 30):
    return fn(ctypes.byref(pool), k, v, src, slots, q, B.TQ4_BF16, table, 64, seq, batch, max_seq, 24, 0.0625,
              FAKE, FAKE, ws_bytes, None)


@pytest.mark.parametrize("which", ["tq4", "int8"])
def test_decode_append_validation(lib, which):
    fn = lib.tq4_attn_decode_append if which == "tq4" else lib.tq4_int8_attn_decode_append
    pool = _pool() if which == "tq4" else _i8pool()
    assert _append(lib, fn, pool, k=None, v=None) == 1       # nothing to append
    assert _append(lib, fn, pool, slots=None) == 1
    assert _append(lib, fn, pool, q=None) == 1
    assert _append(lib, fn, pool, src=B.TQ4_F16) == 3          # sources: fp32 or bf16
    assert _append(lib, fn, pool, k=FAKE + 4) == 4
    assert _append(lib, fn, pool, v=FAKE + 8) == 4
    assert _append(lib, fn, pool, slots=FAKE + 2) == 4
    assert _append(lib, fn, pool, batch=0) == 2
    assert _append(lib, fn, pool, max_seq=4097) == 2
    assert _append(lib, fn, pool, ws_bytes=0) == 5
    assert fn(None, FAKE, FAKE, B.TQ4_F32, FAKE, FAKE, B.TQ4_BF16, FAKE, 64, FAKE, 1, 4000, 24, 0.0625, FAKE,
              FAKE, 1 << 30, None) == 1


def test_int8_encode_validation(lib):
    enc = lib.tq4_int8_encode_pages
    p = _i8pool()
    assert enc(None, FAKE, FAKE, B.TQ4_F32, FAKE, 4, None) == 1
    assert enc(ctypes.byref(p), None, None, B.TQ4_F32, FAKE, 4, None) == 1
    assert enc(ctypes.byref(p), FAKE, FAKE, B.TQ4_F16, FAKE, 4, None) == 3
    assert enc(ctypes.byref(p), FAKE, FAKE, B.TQ4_F32, FAKE, -1, None) == 2
    assert enc(ctypes.byref(p), FAKE, FAKE, B.TQ4_F32, None, 4, None) == 1
    assert enc(ctypes.byref(p), FAKE + 4, FAKE, B.TQ4_F32, FAKE, 4, None) == 4
    assert enc(ctypes.byref(p), FAKE, FAKE, B.TQ4_F32, FAKE + 2, 4, None) == 4
    assert enc(ctypes.byref(_i8pool(page_size=40)), FAKE, FAKE, B.TQ4_F32, FAKE, 4, None) == 2
    assert enc(ctypes.byref(p), FAKE, FAKE, B.TQ4_F32, FAKE, 0, None) == 0  # nothing to do


def test_grid_limits_rejected_on_the_host(lib):
    # batch and KV heads are grid dimensions (<= 65535)
    assert _decode(lib, batch=65536, max_seq=100) == 2
    assert _decode(lib, pool=_pool(num_pages=1, page_size=32, n_kv=65536), n_q=65536, max_seq=32, stride=1) == 2
    assert _i8decode(lib, batch=65536, max_seq=100) == 2
    assert lib.tq4_attn_decode_workspace_size(65536, 4000, 24, 4, 64) == 0
    assert lib.tq4_attn_verify_workspace_size(65536, 4000, 2, 24, 4, 64) == 0
    # prefill: 128 query rows per grid row, at most 65535 rows of workgroups
    assert lib.tq4_attn_prefill_workspace_size(0, 65535 * 128 // 6 + 100, 24, 4, 64) == 0
    assert lib.tq4_attn_prefill_workspace_size(0, 65535 * 128 // 6 - 100, 24, 4, 64) > 0


def test_missing_library_fails_loudly(tmp_path):
    """The binding has no fallback: a missing shared library raises instead of computing
    anything elsewhere, and the package imports no oracle code."""
    import subprocess
    import sys
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from compressed_kv_attention_kvexec_amd import _binding as B\n"
        "try:\n"
        "    B.load_library(%r)\n"
        "except RuntimeError as e:\n"
        "    print('raised', 'missing' in str(e))\n"
        "import compressed_kv_attention_kvexec_amd\n"
        "print('oracle' in sys.modules)\n"
    ) % (str(__import__("pathlib").Path(__file__).resolve().parents[1]), str(tmp_path / "libtq4.so"))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120).stdout.split()
    assert out == ["raised", "True", "False"], out


def test_int8_prefill_validation(lib):
    pf = lib.tq4_int8_attn_prefill_chunk
    p = _i8pool()
    need = lib.tq4_int8_attn_prefill_workspace_size(1000, 100, 24, 4, 64)
    assert need == lib.tq4_attn_prefill_workspace_size(1000, 100, 24, 4, 64) > 0
    args = lambda **kw: dict(dict(pool=ctypes.byref(p), q=FAKE, dt=B.TQ4_BF16, table=FAKE, prior=1000, chunk=100,
                                  n_q=24, out=FAKE, ws=FAKE, ws_bytes=need), **kw)
    call = lambda a: pf(a["pool"], a["q"], a["dt"], a["table"], a["prior"], a["chunk"], a["n_q"], 0.0625, a["out"],
                        a["ws"], a["ws_bytes"], None)
    assert call(args(pool=None)) == 1
    assert call(args(q=None)) == 1
    assert call(args(dt=B.TQ4_F32)) == 3
    assert call(args(chunk=0)) == 2
    assert call(args(prior=-1)) == 2
    assert call(args(n_q=22)) == 2
    assert call(args(ws=None)) == 5
    assert call(args(ws_bytes=need - 1)) == 5
    assert call(args(ws=FAKE + 64)) == 4
    assert call(args(q=FAKE + 2)) == 4


def test_noalloc_decode_validation(lib):
    """tq4_attn_decode_noalloc checks its arguments like tq4_attn_decode, and rejects plans larger
    than its 4 MiB device scratch on the host, before any HIP call."""
    pool = _pool()
    call = lambda **kw: lib.tq4_attn_decode_noalloc(
        ctypes.byref(kw.get("pool", pool)), kw.get("q", FAKE), B.TQ4_BF16, FAKE, kw.get("stride", 64), FAKE,
        kw.get("batch", 1), kw.get("max_seq", 4000), kw.get("n_q", 24), kw.get("scale", 0.0625), kw.get("out", FAKE),
        None)
    assert call(q=None) == 1
    assert call(out=None) == 1
    assert call(n_q=22) == 2
    assert call(scale=0.0) == 8
    assert call(q=FAKE + 2) == 4
    # a group of 16 and one long request: the plan needs more than the 4 MiB scratch
    big = _pool(num_pages=4096, page_size=256, n_kv=4)
    assert lib.tq4_attn_decode_workspace_size(1, 1_000_000, 64, 4, 256) > 4 << 20
    assert call(pool=big, stride=4096, max_seq=1_000_000, n_q=64) == 5


def test_decode_variant_validation(lib):
    """tq4_attn_decode_variant: the decode checks, then the variant (unknown: TQ4_ERR_VALUE) and
    the group sizes the vector-ALU kernels are built for (1, 2, 4, 6, 8), all on the host."""
    pool = _pool()
    call = lambda **kw: lib.tq4_attn_decode_variant(
        ctypes.byref(pool), kw.get("q", FAKE), B.TQ4_BF16, FAKE, 64, FAKE, 1, 4000, kw.get("n_q", 24),
        0.0625, kw.get("variant", B.TQ4_DECODE_VALU_ROTATED), kw.get("out", FAKE), None, 0, None)
    assert call(q=None) == 1
    assert call(variant=3) == 8
    assert call(variant=-1) == 8
    assert call(n_q=48, variant=B.TQ4_DECODE_VALU_LITERAL) == 2  # group 12
    assert call(n_q=64, variant=B.TQ4_DECODE_VALU_ROTATED) == 2  # group 16
    # a valid call would need a workspace for this plan: the workspace check comes last
    assert lib.tq4_attn_decode_workspace_size(1, 4000, 24, 4, 64) > 0
    assert call() == 5
    assert call(variant=B.TQ4_DECODE_FUSED) == 5
