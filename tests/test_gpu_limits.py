"""GPU parity at the documented limits: the largest pages (512 and 1,024 positions), many KV heads
(8 and 16, groups of 2 and 1), and a batch of 300 short requests (one split each, lengths 1 ..
300).  Encoding is bit-exact; attention meets max |err| <= 2e-2, rel-L2 <= 5e-3."""
import numpy as np
import pytest

import oracle
import synth
from _pools import (bf16_queries, from_device, int8_to_device, oracle_int8_pool, oracle_pool, parity,
                    to_device)

pytestmark = pytest.mark.gpu


def _t(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("page", [512, 1024])
def test_large_pages_encode_decode_verify(page):
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    lens = (5000, 1023, 1025)
    w = synth.Workload(170, "bigpage", "decode", 1, page, sum(-(-L // page) for L in lens) + 2, seq_lens=lens)
    pool, table = oracle_pool(w)
    # encode on the GPU into an empty pool: bit-exact records
    slots = synth.used_slots(w, table)
    dpool = tq4.Tq4LayerPool.empty(w.pool_pages, w.n_kv, page)
    tq4.tq4_encode_pages(dpool, _t(synth.kv_source(w, 0, len(slots), synth.T_K)),
                         _t(synth.kv_source(w, 0, len(slots), synth.T_V)), _t(slots))
    torch.cuda.synchronize()
    got_pool = from_device(dpool)
    for a, b in ((got_pool.k_words, pool.k_words), (got_pool.k_norms, pool.k_norms),
                 (got_pool.v_words, pool.v_words), (got_pool.v_norms, pool.v_norms)):
        np.testing.assert_array_equal(a, b)
    q_t, q64 = bf16_queries(w, 0, w.batch)
    out = tq4.tq4_attn_decode(dpool, q_t.cuda(), _t(table), _t(np.array(lens, np.int32)), max(lens), synth.SCALE)
    torch.cuda.synchronize()
    parity(out.cpu(), oracle.attn_decode(pool, q64, table, lens, synth.SCALE), f"decode page {page}")
    qv, qv64 = bf16_queries(w, 1, w.batch * 4)
    qv = qv.reshape(w.batch, 4, w.n_q, 256).contiguous()
    qv64 = qv64.reshape(w.batch, 4, w.n_q, 256)
    outv = tq4.tq4_attn_verify(dpool, qv.cuda(), _t(table), _t(np.array(lens, np.int32)), max(lens), synth.SCALE)
    torch.cuda.synchronize()
    parity(outv.cpu(), oracle.attn_verify(pool, qv64, table, lens, synth.SCALE), f"verify page {page}")


@pytest.mark.parametrize("page", [512, 1024])
def test_large_pages_prefill(page):
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    prior, chunk = 3000, 100
    w = synth.Workload(171, "bigpage_pf", "prefill", 1, page, -(-(prior + chunk) // page) + 3, prior_len=prior,
                       chunk_len=chunk)
    pool, table = oracle_pool(w)
    q_t, q64 = bf16_queries(w, 0, chunk)
    ws = tq4.new_workspace(tq4.tq4_attn_prefill_workspace_size(prior, chunk, w.n_q, w.n_kv, page))
    out = tq4.tq4_attn_prefill_chunk(to_device(pool), q_t.cuda(), _t(table[0]), prior, synth.SCALE, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.attn_prefill_rows(pool, q64, np.arange(chunk), table[0], prior, synth.SCALE)
    parity(out.cpu(), ref, f"prefill page {page}")


@pytest.mark.parametrize("page", [512, 1024])
def test_large_pages_int8_and_unfused(page):
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    lens = (4000, 1)
    w = synth.Workload(172, "bigpage_i8", "decode", 1, page, sum(-(-L // page) for L in lens) + 2, seq_lens=lens)
    pool8, table = oracle_int8_pool(w)
    q_t, q64 = bf16_queries(w, 0, w.batch)
    out = tq4.tq4_int8_attn_decode(int8_to_device(pool8), q_t.cuda(), _t(table), _t(np.array(lens, np.int32)),
                                   max(lens), synth.SCALE)
    torch.cuda.synchronize()
    parity(out.cpu(), oracle.int8_attn_decode(pool8, q64, table, lens, synth.SCALE), f"int8 page {page}")
    pool, _ = oracle_pool(w, table=table)
    k, v = tq4.tq4_reconstruct_pages(to_device(pool), _t(table), _t(np.array(lens, np.int32)), max(lens))
    torch.cuda.synchronize()
    kb, vb = oracle.reconstruct(pool, table, lens, max(lens))
    got_k = k.view(torch.int16).cpu().numpy().view(np.uint16)
    # most values bit-identical to the oracle's one-step rounding (the rest differ by one bf16 unit)
    for b, L in enumerate(lens):
        same = np.mean(got_k[b, :, :L] == kb[b, :, :L])
        assert same > 0.99, same


@pytest.mark.parametrize("n_q,n_kv", [(16, 8), (16, 16)])
def test_many_kv_heads(n_q, n_kv):
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    lens = (3000, 300)
    w = synth.Workload(173, "manykv", "decode", 1, 64, sum(-(-L // 64) for L in lens) + 2, seq_lens=lens,
                       n_q=n_q, n_kv=n_kv)
    pool, table = oracle_pool(w)
    q_t, q64 = bf16_queries(w, 0, w.batch)
    out = tq4.tq4_attn_decode(to_device(pool), q_t.cuda(), _t(table), _t(np.array(lens, np.int32)), 3000, synth.SCALE)
    torch.cuda.synchronize()
    parity(out.cpu(), oracle.attn_decode(pool, q64, table, lens, synth.SCALE), f"n_kv={n_kv}")
    pool8, _ = oracle_int8_pool(w, table=table)
    out8 = tq4.tq4_int8_attn_decode(int8_to_device(pool8), q_t.cuda(), _t(table), _t(np.array(lens, np.int32)),
                                    3000, synth.SCALE)
    torch.cuda.synchronize()
    parity(out8.cpu(), oracle.int8_attn_decode(pool8, q64, table, lens, synth.SCALE), f"int8 n_kv={n_kv}")


def test_batch_of_300_short_requests():
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    lens = tuple(range(1, 301))
    w = synth.Workload(174, "b300", "decode", 1, 32, sum(-(-L // 32) for L in lens) + 2, seq_lens=lens)
    pool, table = oracle_pool(w)
    q_t, q64 = bf16_queries(w, 0, w.batch)
    seq = _t(np.array(lens, np.int32))
    out = tq4.tq4_attn_decode(to_device(pool), q_t.cuda(), _t(table), seq, 300, synth.SCALE)
    torch.cuda.synchronize()
    parity(out.cpu(), oracle.attn_decode(pool, q64, table, lens, synth.SCALE), "batch 300")
    pool8, _ = oracle_int8_pool(w, table=table)
    out8 = tq4.tq4_int8_attn_decode(int8_to_device(pool8), q_t.cuda(), _t(table), seq, 300, synth.SCALE)
    torch.cuda.synchronize()
    parity(out8.cpu(), oracle.int8_attn_decode(pool8, q64, table, lens, synth.SCALE), "int8 batch 300")
