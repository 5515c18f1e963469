"""GPU parity of the packed multi-query verifier: tq4_attn_verify against the fp64 oracle
(query i of k attends the first L - k + i + 1 positions) within max |err| <= 2e-2 and
rel-L2 <= 5e-3, over every packing of query rows into MFMA column blocks, plus its
identities with decode."""
import numpy as np
import pytest

import oracle
import synth
from _pools import bf16_queries, oracle_pool, parity, to_device

pytestmark = pytest.mark.gpu


def _queries(w, k, layer=0, scale=1.0):
    q_t, q64 = bf16_queries(w, layer, w.batch * k, scale)
    return (q_t.reshape(w.batch, k, w.n_q, 256).contiguous(), q64.reshape(w.batch, k, w.n_q, 256))


def _verify(dpool, q_t, table, seq_lens, max_seq, scale=synth.SCALE, workspace=None):
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    out = tq4.tq4_attn_verify(dpool, q_t.cuda(), torch.from_numpy(np.ascontiguousarray(table, np.int32)).cuda(),
                              torch.tensor(seq_lens, dtype=torch.int32).cuda(), max_seq, scale,
                              workspace=workspace)
    torch.cuda.synchronize()
    return out.cpu()


# k x G rows: 12 and 16 fit one 16-column block, 18 and 24 two, 48 three
@pytest.mark.parametrize("k,n_q,n_kv", [(2, 24, 4), (4, 16, 4), (3, 24, 4), (4, 24, 4), (8, 24, 4),
                                        (3, 64, 4), (8, 4, 4)])
def test_verify_matches_oracle(k, n_q, n_kv):
    w = synth.Workload(110, "verify", "decode", 1, 64, 120, seq_lens=(3000, 700, 5),
                       n_q=n_q, n_kv=n_kv)
    pool, table = oracle_pool(w)
    q_t, q64 = _queries(w, k)
    ref = oracle.attn_verify(pool, q64, table, w.seq_lens, synth.SCALE)
    got = _verify(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens))
    parity(got, ref, f"k={k} G={n_q // n_kv}")


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_verify_single_split_and_short_requests(k):
    """Lengths below one split's range (the split kernel writes the output itself), lengths
    shorter than k (leading queries see nothing and return zeros) and length 0."""
    w = synth.Workload(111, "vshort", "decode", 1, 32, 16, seq_lens=(200, 7, 3, 1, 0))
    pool, table = oracle_pool(w)
    q_t, q64 = _queries(w, k)
    ref = oracle.attn_verify(pool, q64, table, w.seq_lens, synth.SCALE)
    got = _verify(to_device(pool), q_t, table, w.seq_lens, 200)
    parity(got, ref, f"short k={k}")
    for b, L in enumerate(w.seq_lens):
        for i in range(k):
            if L - k + i + 1 <= 0:
                assert np.all(got[b, i].float().numpy() == 0.0)


def test_verify_peaked_softmax():
    w = synth.Workload(112, "vpeak", "decode", 1, 64, 60, seq_lens=(2500, 1200))
    pool, table = oracle_pool(w)
    q_t, q64 = _queries(w, 4, scale=8.0)
    ref = oracle.attn_verify(pool, q64, table, w.seq_lens, synth.SCALE)
    got = _verify(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens))
    parity(got, ref, "peaked")


def test_verify_one_query_is_decode_bit_for_bit():
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    w = synth.Workload(113, "v1", "decode", 1, 64, 160, seq_lens=(5000, 333, 64))
    pool, table = oracle_pool(w)
    q_t, _ = _queries(w, 1)
    dpool = to_device(pool)
    got = _verify(dpool, q_t, table, w.seq_lens, 5000)
    dec = tq4.tq4_attn_decode(dpool, q_t[:, 0].contiguous().cuda(), torch.from_numpy(table).cuda(),
                              torch.tensor(w.seq_lens, dtype=torch.int32).cuda(), 5000, synth.SCALE)
    torch.cuda.synchronize()
    assert torch.equal(got[:, 0], dec.cpu())


@pytest.mark.parametrize("k", [3, 8])
def test_verify_rows_match_decode_at_their_length(k):
    """Query i equals a decode call at length L - k + i + 1 within rounding (the two calls may
    split the keys differently)."""
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    w = synth.Workload(114, "vrow", "decode", 1, 64, 100, seq_lens=(6000,))
    pool, table = oracle_pool(w)
    q_t, _ = _queries(w, k)
    dpool = to_device(pool)
    got = _verify(dpool, q_t, table, w.seq_lens, 6000)
    L = w.seq_lens[0]
    for i in range(k):
        dec = tq4.tq4_attn_decode(dpool, q_t[:, i].contiguous().cuda(), torch.from_numpy(table).cuda(),
                                  torch.tensor([L - k + i + 1], dtype=torch.int32).cuda(), 6000, synth.SCALE)
        torch.cuda.synchronize()
        assert (dec.cpu()[0].double() - got[0, i].double()).abs().max().item() < 4e-3


def test_verify_deterministic_and_workspace_reuse():
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    w = synth.Workload(115, "vdet", "decode", 1, 64, 220, seq_lens=(9000, 4100))
    pool, table = oracle_pool(w)
    dpool = to_device(pool)
    ws = tq4.new_workspace(tq4.tq4_attn_verify_workspace_size(2, 9000, 8, 24, 4, 64))
    q8, q64 = _queries(w, 8)
    a = _verify(dpool, q8, table, w.seq_lens, 9000, workspace=ws)
    q3, q3_64 = _queries(w, 3, layer=1)
    b = _verify(dpool, q3, table, w.seq_lens, 9000, workspace=ws)
    c = _verify(dpool, q8, table, w.seq_lens, 9000, workspace=ws)
    assert torch.equal(a, c)
    parity(b, oracle.attn_verify(pool, q3_64, table, w.seq_lens, synth.SCALE), "reuse k=3")


@pytest.mark.parametrize("k", [4, 8])
def test_verify_full_212k_sampled_head(k):
    """212,992 cached positions in the full launch; the pool holds one KV head's records and the
    oracle checks that head's rows."""
    name, g, layer = "decode_212k_16l", 1, 5
    w = synth.WORKLOADS[name]
    table = synth.placement(w, layer)
    slots = synth.used_slots(w, table)
    pool = oracle.Pool.empty(w.pool_pages, w.n_kv, w.page_size)
    one = oracle.Pool.empty(w.pool_pages, 1, w.page_size)
    kk = np.ascontiguousarray(synth.kv_source(w, layer, len(slots), synth.T_K)[:, g:g + 1])
    vv = np.ascontiguousarray(synth.kv_source(w, layer, len(slots), synth.T_V)[:, g:g + 1])
    oracle.encode_to_pool(one, kk, vv, slots)
    for dst, src in ((pool.k_words, one.k_words), (pool.k_norms, one.k_norms),
                     (pool.v_words, one.v_words), (pool.v_norms, one.v_norms)):
        dst[:, g] = src[:, 0]
    q_t, q64 = _queries(w, k, layer)
    G = w.n_q // w.n_kv
    ref = oracle.attn_verify(pool, q64, table, w.seq_lens, synth.SCALE, heads=(g * G, (g + 1) * G))
    got = _verify(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens))
    parity(got[:, :, g * G:(g + 1) * G], ref[:, :, g * G:(g + 1) * G], f"212k verify k={k}")


def test_verify_ignores_garbage_past_the_lengths():
    w = synth.Workload(151, "vgarbage", "decode", 1, 64, 60, seq_lens=(1000, 37, 64 * 5 + 1))
    pool, table = oracle_pool(w, fill=np.random.default_rng(7))
    q_t, q64 = _queries(w, 4)
    ref = oracle.attn_verify(pool, q64, table, w.seq_lens, synth.SCALE)
    got = _verify(to_device(pool), q_t, table, w.seq_lens, 1000)
    parity(got, ref, "verify garbage tail")
