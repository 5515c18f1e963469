"""Seeded sweep of random shapes through every attention entry point, each checked against the
oracle (max |err| <= 2e-2, rel-L2 <= 5e-3): page sizes 32..512, groups 1..16, batches 1..5 with
ragged lengths 1..4,000 (and empty requests), verifier k = 1..8 within the 48-row limit, prefill
chunks 1..160 over 0..1,500 cached positions, and the INT8 and unfused paths; the fused appends
(TQ4 and INT8) equal encode followed by decode bit for bit on the same shapes."""
import numpy as np
import pytest

import oracle
import synth
from _pools import bf16_queries, int8_to_device, oracle_int8_pool, oracle_pool, parity, to_device

pytestmark = pytest.mark.gpu

PAGES = (32, 64, 128, 256, 512)
GROUPS = ((24, 4), (16, 16), (8, 4), (12, 4), (64, 4), (6, 1), (32, 2))
PREFILL_GROUPS = ((24, 4), (8, 4), (12, 4), (6, 1), (32, 2))  # the oracle decodes every key per row


def _decode_case(rng, i):
    page = int(rng.choice(PAGES))
    n_q, n_kv = GROUPS[int(rng.integers(len(GROUPS)))]
    batch = int(rng.integers(1, 6))
    lens = tuple(int(x) for x in rng.integers(0, 4001, batch))
    if batch > 1 and i % 4 == 3:
        lens = lens[:-1] + (0,)  # an empty request among others
    if max(lens) == 0:
        lens = (1,) + lens[1:]
    pages = sum(-(-L // page) for L in lens) + int(rng.integers(0, 4))
    w = synth.Workload(200 + i, f"sweep{i}", "decode", 1, page, max(pages, 1), seq_lens=lens, n_q=n_q, n_kv=n_kv)
    return w


@pytest.mark.parametrize("i", range(12))
def test_sweep_decode_verify_int8(i):
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    rng = np.random.default_rng(1000 + i)
    w = _decode_case(rng, i)
    pool, table = oracle_pool(w)
    dpool = to_device(pool)
    tab = torch.from_numpy(np.ascontiguousarray(table, np.int32)).cuda()
    seq = torch.tensor(w.seq_lens, dtype=torch.int32).cuda()
    max_seq = max(w.seq_lens)
    what = f"case {i}: page {w.page_size}, n_q {w.n_q}, n_kv {w.n_kv}, lens {w.seq_lens}"
    # decode
    q_t, q64 = bf16_queries(w, 0, w.batch)
    out = tq4.tq4_attn_decode(dpool, q_t.cuda(), tab, seq, max_seq, synth.SCALE)
    torch.cuda.synchronize()
    parity(out.cpu(), oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE), "decode " + what)
    # verifier with a random k inside the row limit
    G = w.n_q // w.n_kv
    k = int(rng.integers(1, max(1, min(8, 48 // G)) + 1))
    qv, qv64 = bf16_queries(w, 1, w.batch * k)
    qv = qv.reshape(w.batch, k, w.n_q, 256).contiguous()
    qv64 = qv64.reshape(w.batch, k, w.n_q, 256)
    outv = tq4.tq4_attn_verify(dpool, qv.cuda(), tab, seq, max_seq, synth.SCALE)
    torch.cuda.synchronize()
    parity(outv.cpu(), oracle.attn_verify(pool, qv64, table, w.seq_lens, synth.SCALE), f"verify k={k} " + what)
    # INT8 arm on the same placement
    pool8, _ = oracle_int8_pool(w, table=table)
    out8 = tq4.tq4_int8_attn_decode(int8_to_device(pool8), q_t.cuda(), tab, seq, max_seq, synth.SCALE)
    torch.cuda.synchronize()
    parity(out8.cpu(), oracle.int8_attn_decode(pool8, q64, table, w.seq_lens, synth.SCALE), "int8 " + what)
    outv8 = tq4.tq4_int8_attn_verify(int8_to_device(pool8), qv.cuda(), tab, seq, max_seq, synth.SCALE)
    torch.cuda.synchronize()
    parity(outv8.cpu(), oracle.int8_attn_verify(pool8, qv64, table, w.seq_lens, synth.SCALE),
           f"int8 verify k={k} " + what)
    # fused appends (new token at position L - 1 of every non-empty request) against encode followed
    # by decode, bit for bit, on copies of both pools
    new = torch.from_numpy(rng.standard_normal((2, w.batch, w.n_kv, 256)).astype(np.float32)).cuda()
    last = torch.tensor([int(table[b, (L - 1) // w.page_size]) * w.page_size + (L - 1) % w.page_size if L > 0 else -1
                         for b, L in enumerate(w.seq_lens)], dtype=torch.int32).cuda()
    fused, ref = to_device(pool), to_device(pool)
    got = tq4.tq4_attn_decode_append(fused, new[0], new[1], last, q_t.cuda(), tab, seq, max_seq, synth.SCALE)
    tq4.tq4_encode_pages(ref, new[0], new[1], last)
    want = tq4.tq4_attn_decode(ref, q_t.cuda(), tab, seq, max_seq, synth.SCALE)
    torch.cuda.synchronize()
    assert torch.equal(got, want), "append " + what
    fused8, ref8 = int8_to_device(pool8), int8_to_device(pool8)
    got8 = tq4.tq4_int8_attn_decode_append(fused8, new[0], new[1], last, q_t.cuda(), tab, seq, max_seq, synth.SCALE)
    tq4.tq4_int8_encode_pages(ref8, new[0], new[1], last)
    want8 = tq4.tq4_int8_attn_decode(ref8, q_t.cuda(), tab, seq, max_seq, synth.SCALE)
    torch.cuda.synchronize()
    assert torch.equal(got8, want8), "int8 append " + what
    for a, b in ((fused.k_words, ref.k_words), (fused.v_norms, ref.v_norms), (fused8.k_codes, ref8.k_codes),
                 (fused8.v_scales, ref8.v_scales)):
        assert torch.equal(a, b), "append records " + what
    # unfused chain against attention over the pages
    kd, vd = tq4.tq4_reconstruct_pages(dpool, tab, seq, max_seq)
    outs = tq4.tq4_sdpa_decode(q_t.cuda(), kd, vd, seq, synth.SCALE)
    torch.cuda.synchronize()
    parity(outs.cpu(), oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE), "unfused " + what)


@pytest.mark.parametrize("i", range(8))
def test_sweep_prefill(i):
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    rng = np.random.default_rng(2000 + i)
    page = int(rng.choice(PAGES))
    n_q, n_kv = PREFILL_GROUPS[int(rng.integers(len(PREFILL_GROUPS)))]
    prior = int(rng.integers(0, 1501))
    chunk = int(rng.integers(1, 161))
    w = synth.Workload(300 + i, f"pfsweep{i}", "prefill", 1, page, -(-(prior + chunk) // page) + 2,
                       prior_len=prior, chunk_len=chunk, n_q=n_q, n_kv=n_kv)
    pool, table = oracle_pool(w)
    q_t, q64 = bf16_queries(w, 0, chunk)
    out = tq4.tq4_attn_prefill_chunk(to_device(pool), q_t.cuda(), torch.from_numpy(table[0]).cuda(), prior,
                                     synth.SCALE)
    torch.cuda.synchronize()
    ref = oracle.attn_prefill_rows(pool, q64, np.arange(chunk), table[0], prior, synth.SCALE)
    what = f"case {i}: page {page}, n_q {n_q}, n_kv {n_kv}, prior {prior}, chunk {chunk}"
    parity(out.cpu(), ref, "prefill " + what)
    pool8, _ = oracle_int8_pool(w, table=table)
    out8 = tq4.tq4_int8_attn_prefill_chunk(int8_to_device(pool8), q_t.cuda(), torch.from_numpy(table[0]).cuda(),
                                           prior, synth.SCALE)
    torch.cuda.synchronize()
    parity(out8.cpu(), oracle.int8_attn_prefill_rows(pool8, q64, np.arange(chunk), table[0], prior, synth.SCALE),
           "int8 prefill " + what)
