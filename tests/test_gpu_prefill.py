"""GPU prefill parity: tq4_attn_prefill_chunk against the fp64 oracle (causal inside the
chunk, all keys read back from TQ4 pages), within max |err| <= 2e-2 and rel-L2 <= 5e-3."""
import numpy as np
import pytest

import oracle
import synth
from _pools import bf16_queries, oracle_pool, parity, to_device

pytestmark = pytest.mark.gpu


def _prefill(dpool, q_t, table_row, prior):
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    out = tq4.tq4_attn_prefill_chunk(dpool, q_t.cuda(), torch.from_numpy(np.ascontiguousarray(table_row, np.int32)).cuda(),
                                     prior, synth.SCALE)
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("prior,chunk,page,n_q,n_kv", [
    (100, 28, 64, 24, 4),      # ragged pages, chunk inside one page
    (0, 1, 64, 24, 4),         # a single token and nothing cached
    (0, 77, 32, 6, 1),         # no prior context, causal only
    (3000, 300, 256, 24, 4),   # several row blocks and key splits
    (1000, 130, 128, 64, 4),   # group of 16
])
def test_prefill_matches_oracle_all_rows(prior, chunk, page, n_q, n_kv):
    L = prior + chunk
    w = synth.Workload(97, "pf", "prefill", 1, page, L // page + 5, prior_len=prior, chunk_len=chunk,
                       n_q=n_q, n_kv=n_kv)
    pool, table = oracle_pool(w)
    q_t, q64 = bf16_queries(w, 0, chunk)
    rows = np.arange(chunk)
    ref = oracle.attn_prefill_rows(pool, q64, rows, table[0], prior, synth.SCALE)
    got = _prefill(to_device(pool), q_t, table[0], prior)
    parity(got, ref, f"prefill prior={prior} chunk={chunk}")


def test_prefill_row_equals_decode_at_that_length():
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    prior, chunk = 700, 40
    w = synth.Workload(98, "pfd", "prefill", 1, 64, 20, prior_len=prior, chunk_len=chunk)
    pool, table = oracle_pool(w)
    q_t, _ = bf16_queries(w, 0, chunk)
    dpool = to_device(pool)
    got = _prefill(dpool, q_t, table[0], prior)
    for t in (0, 17, 39):
        dec = tq4.tq4_attn_decode(dpool, q_t[t:t + 1].cuda(), torch.from_numpy(table).cuda(),
                                  torch.tensor([prior + t + 1], dtype=torch.int32).cuda(), prior + t + 1,
                                  synth.SCALE)
        torch.cuda.synchronize()
        assert (dec.cpu()[0].double() - got[t].double()).abs().max().item() < 4e-3


def test_prefill_full_size_sampled_rows():
    """The 2,048-token chunk over 194,560 cached positions in its full launch; the pool holds
    one KV head's records, the oracle checks sampled rows of that head."""
    w = synth.WORKLOADS["prefill_2k_over_194k"]
    g = 3
    table = synth.placement(w, 0)
    slots = synth.used_slots(w, table)
    pool = oracle.Pool.empty(w.pool_pages, w.n_kv, w.page_size)
    one = oracle.Pool.empty(w.pool_pages, 1, w.page_size)
    k = np.ascontiguousarray(synth.kv_source(w, 0, len(slots), synth.T_K)[:, g:g + 1])
    v = np.ascontiguousarray(synth.kv_source(w, 0, len(slots), synth.T_V)[:, g:g + 1])
    oracle.encode_to_pool(one, k, v, slots)
    for dst, src in ((pool.k_words, one.k_words), (pool.k_norms, one.k_norms),
                     (pool.v_words, one.v_words), (pool.v_norms, one.v_norms)):
        dst[:, g] = src[:, 0]
    q_t, q64 = bf16_queries(w, 0, w.chunk_len)
    got = _prefill(to_device(pool), q_t, table[0], w.prior_len)
    G = w.n_q // w.n_kv
    rows = np.array([0, 1, 1023, 2047])
    ref = oracle.attn_prefill_rows(pool, q64[rows], rows, table[0], w.prior_len, synth.SCALE,
                                   heads=(g * G, (g + 1) * G))
    parity(got[rows, g * G:(g + 1) * G], ref[:, g * G:(g + 1) * G], "prefill full size")


@pytest.mark.parametrize("prior,chunk", [(100, 28), (640, 33)])
def test_prefill_ignores_garbage_past_the_chunk(prior, chunk):
    """Records past prior + chunk in the last page hold random bits (NaN norms among them)."""
    w = synth.Workload(152, "pfgarbage", "prefill", 1, 64, (prior + chunk) // 64 + 5, prior_len=prior,
                       chunk_len=chunk)
    pool, table = oracle_pool(w, fill=np.random.default_rng(8))
    q_t, q64 = bf16_queries(w, 0, chunk)
    ref = oracle.attn_prefill_rows(pool, q64, np.arange(chunk), table[0], prior, synth.SCALE)
    got = _prefill(to_device(pool), q_t, table[0], prior)
    parity(got, ref, f"prefill garbage prior={prior} chunk={chunk}")
