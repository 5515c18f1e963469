"""tq4_attn_decode_noalloc: decode with the library's per-device scratch instead of a workspace
(for callers that cannot allocate).  Through the C ABI it must return exactly what
tq4_attn_decode returns (same kernels, same plan) and meet the oracle bar, on consecutive calls
that reuse the scratch, the second one smaller."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from _pools import bf16_queries, oracle_pool, parity, to_device

pytestmark = pytest.mark.gpu


def _noalloc(dpool, q, table, seq, max_seq, out):
    from compressed_kv_attention_kvexec_amd import _binding as B
    import torch
    lib = B.load_library()
    ps = dpool.struct()
    st = lib.tq4_attn_decode_noalloc(ctypes.byref(ps), ctypes.c_void_p(q.data_ptr()), B.TQ4_BF16,
                                     ctypes.c_void_p(table.data_ptr()), int(table.shape[1]),
                                     ctypes.c_void_p(seq.data_ptr()), int(q.shape[0]), int(max_seq), int(q.shape[1]),
                                     synth.SCALE, ctypes.c_void_p(out.data_ptr()),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, B.STATUS_NAMES.get(st, st)


def _case(w, layer=0):
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    pool, table = oracle_pool(w, layer=layer)
    q_t, q64 = bf16_queries(w, layer, w.batch)
    dpool = to_device(pool)
    q, tab = q_t.cuda(), torch.from_numpy(table).cuda()
    seq = torch.tensor(w.seq_lens, dtype=torch.int32).cuda()
    max_seq = max(w.seq_lens)
    out = torch.full_like(q, float("nan"))
    _noalloc(dpool, q, tab, seq, max_seq, out)
    ref = tq4.tq4_attn_decode(dpool, q, tab, seq, max_seq, synth.SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    parity(out.cpu(), oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE), w.name)
    return out


def test_noalloc_equals_decode_on_consecutive_calls():
    """Two calls in a row (the second smaller) reuse the scratch; a third call repeats the first
    and returns the same bits."""
    import torch
    big = synth.Workload(170, "noalloc_big", "decode", 1, 64, 400, seq_lens=(9000, 4100, 12000))
    small = synth.Workload(171, "noalloc_small", "decode", 1, 64, 60, seq_lens=(2500,))
    a = _case(big)
    _case(small)
    assert torch.equal(_case(big), a)


def test_noalloc_full_size_sampled_head():
    """212,992 cached positions in the launch configuration of the 16-layer decode step; the pool
    holds one KV head's records and the oracle checks that head."""
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    w = synth.WORKLOADS["decode_212k_16l"]
    g, layer = 2, 4
    table = synth.placement(w, layer)
    slots = synth.used_slots(w, table)
    pool = oracle.Pool.empty(w.pool_pages, w.n_kv, w.page_size)
    one = oracle.Pool.empty(w.pool_pages, 1, w.page_size)
    k = np.ascontiguousarray(synth.kv_source(w, layer, len(slots), synth.T_K)[:, g:g + 1])
    v = np.ascontiguousarray(synth.kv_source(w, layer, len(slots), synth.T_V)[:, g:g + 1])
    oracle.encode_to_pool(one, k, v, slots)
    for dst, src in ((pool.k_words, one.k_words), (pool.k_norms, one.k_norms),
                     (pool.v_words, one.v_words), (pool.v_norms, one.v_norms)):
        dst[:, g] = src[:, 0]
    q_t, q64 = bf16_queries(w, layer, w.batch)
    dpool = to_device(pool)
    q, tab = q_t.cuda(), torch.from_numpy(table).cuda()
    seq = torch.tensor(w.seq_lens, dtype=torch.int32).cuda()
    out = torch.empty_like(q)
    _noalloc(dpool, q, tab, seq, w.seq_lens[0], out)
    ref = tq4.tq4_attn_decode(dpool, q, tab, seq, w.seq_lens[0], synth.SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    G = w.n_q // w.n_kv
    want = oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE, heads=(g * G, (g + 1) * G))
    parity(out.cpu()[:, g * G:(g + 1) * G], want[:, g * G:(g + 1) * G], "noalloc 212k")
