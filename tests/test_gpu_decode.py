"""GPU decode parity: tq4_attn_decode against the fp64 oracle on the same
oracle-built pools (max |err| <= 2e-2 and relative L2 <= 5e-3 per call), plus
invariances that hold for any correct implementation."""
import numpy as np
import pytest

import oracle
import synth
from _pools import bf16_queries, oracle_pool, parity, to_device

pytestmark = pytest.mark.gpu


def _run(dpool, q_t, table, seq_lens, max_seq, scale=synth.SCALE):
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    out = tq4.tq4_attn_decode(dpool, q_t.cuda(), torch.from_numpy(np.ascontiguousarray(table, np.int32)).cuda(),
                              torch.tensor(seq_lens, dtype=torch.int32).cuda(), max_seq, scale)
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("name", ["decode_1k_p64", "decode_32k"])
def test_decode_matches_oracle_full(name):
    w = synth.WORKLOADS[name]
    pool, table = oracle_pool(w)
    q_t, q64 = bf16_queries(w, 0, w.batch)
    ref = oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE)
    got = _run(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens))
    parity(got, ref, name)


def test_decode_ragged_batch_shared_first_page():
    w = synth.Workload(91, "ragged", "decode", 1, 64, 48, seq_lens=(1, 33, 1000, 64, 257),
                       shared_prefix_pages=1)
    pool, table = oracle_pool(w)
    q_t, q64 = bf16_queries(w, 0, w.batch)
    ref = oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE)
    got = _run(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens))
    parity(got, ref, "ragged")
    # a request of length 1 returns its single value vector
    one = oracle.decode(pool.v_words[table[0, 0], :, 0], pool.v_norms[table[0, 0], :, 0])
    np.testing.assert_allclose(got[0].double().numpy(), np.repeat(one, 6, axis=0), atol=2e-2)


@pytest.mark.parametrize("n_q,n_kv,page", [(4, 4, 256), (8, 4, 32), (64, 4, 128), (6, 1, 64)])
def test_decode_group_sizes_and_page_sizes(n_q, n_kv, page):
    w = synth.Workload(92, "groups", "decode", 1, page, 3000 // page + 8, seq_lens=(2999, 130),
                       n_kv=n_kv, n_q=n_q)
    pool, table = oracle_pool(w)
    q_t, q64 = bf16_queries(w, 0, w.batch)
    ref = oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE)
    got = _run(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens))
    parity(got, ref, f"G={n_q // n_kv} P={page}")


def test_decode_peaked_softmax():
    """Queries scaled x8 make the softmax sharp, so score precision matters."""
    w = synth.Workload(93, "peaked", "decode", 1, 64, 40, seq_lens=(2000, 500))
    pool, table = oracle_pool(w)
    q_t, q64 = bf16_queries(w, 0, w.batch, scale=8.0)
    ref = oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE)
    got = _run(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens))
    parity(got, ref, "peaked")


def test_decode_zero_length_and_clamping():
    w = synth.Workload(94, "zero", "decode", 1, 64, 40, seq_lens=(640, 640))
    pool, table = oracle_pool(w)
    q_t, q64 = bf16_queries(w, 0, 3)
    table3 = np.vstack([table, table[:1]])
    got = _run(to_device(pool), q_t, table3, [0, 640, 10_000], 640)
    assert np.all(got[0].float().numpy() == 0.0)
    ref = oracle.attn_decode(pool, q64[1:], table3[1:], [640, 640], synth.SCALE)
    parity(got[1:], ref, "clamped")


def test_decode_invariances():
    """Deterministic; physical page placement does not change any bit; the split plan
    (set by max_seq_len) changes results only within rounding."""
    import torch
    w = synth.Workload(95, "inv", "decode", 1, 64, 160, seq_lens=(5000, 3333))
    pool, table = oracle_pool(w)
    q_t, _ = bf16_queries(w, 0, w.batch)
    dpool = to_device(pool)
    a = _run(dpool, q_t, table, w.seq_lens, 5000)
    b = _run(dpool, q_t, table, w.seq_lens, 5000)
    assert torch.equal(a, b)
    perm = np.random.default_rng(95).permutation(160)
    inv = np.argsort(perm)
    moved = oracle.Pool(pool.k_words[inv].copy(), pool.k_norms[inv].copy(),
                        pool.v_words[inv].copy(), pool.v_norms[inv].copy())
    c = _run(to_device(moved), q_t, perm[table], w.seq_lens, 5000)
    assert torch.equal(a, c)
    table_wide = np.hstack([table, np.zeros((2, 200), np.int32)])
    d = _run(dpool, q_t, table_wide, w.seq_lens, table_wide.shape[1] * 64)
    diff = (a.double() - d.double()).abs().max().item()
    assert diff < 4e-3


def test_decode_shared_prefix_equals_private_copy():
    w = synth.Workload(96, "alias", "decode", 1, 64, 64, seq_lens=(1500, 1100), shared_prefix_pages=8)
    pool, table = oracle_pool(w)
    q_t, _ = bf16_queries(w, 0, w.batch)
    got = _run(to_device(pool), q_t, table, w.seq_lens, 1500)
    # give request 1 private copies of the shared pages
    free = sorted(set(range(64)) - set(table[0, :24].tolist()) - set(table[1, :18].tolist()))[:8]
    priv = oracle.Pool(pool.k_words.copy(), pool.k_norms.copy(), pool.v_words.copy(), pool.v_norms.copy())
    t2 = table.copy()
    for i, pg in enumerate(free):
        src = table[1, i]
        for arr in (priv.k_words, priv.k_norms, priv.v_words, priv.v_norms):
            arr[pg] = arr[src]
        t2[1, i] = pg
    got2 = _run(to_device(priv), q_t, t2, w.seq_lens, 1500)
    import torch
    assert torch.equal(got, got2)


def _sampled_full_size(name, g, layer=0):
    """One KV head of a full-size workload: the pool holds only that head's records,
    so the oracle encodes and attends one head's keys while the GPU runs the full launch."""
    w = synth.WORKLOADS[name]
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
    G = w.n_q // w.n_kv
    ref = oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE, heads=(g * G, (g + 1) * G))
    got = _run(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens))
    return got[:, g * G:(g + 1) * G], ref[:, g * G:(g + 1) * G]


def test_decode_full_212k_sampled_head():
    got, ref = _sampled_full_size("decode_212k_16l", g=2, layer=3)
    parity(got, ref, "212k head 2")


def test_decode_full_two_requests_shared_prefix_sampled_head():
    got, ref = _sampled_full_size("decode_2req_shared", g=1, layer=0)
    parity(got, ref, "2req head 1")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_append_equals_encode_then_decode(dtype):
    """The fused append call writes the same records as tq4_encode_pages and returns the same bits
    as tq4_attn_decode on the updated pool; a second call reuses the workspace."""
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    from _pools import from_device
    w = synth.Workload(99, "append", "decode", 1, 64, 80, seq_lens=(1, 63, 64, 65, 2000, 777))
    pool, table = oracle_pool(w)
    q_t, _ = bf16_queries(w, 0, w.batch)
    rng = np.random.default_rng(99)
    new = rng.standard_normal((2, w.batch, w.n_kv, 256)).astype(np.float32)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    k_new, v_new = (torch.from_numpy(new[i]).to(tdt).cuda().contiguous() for i in range(2))
    last = np.array([table[b, (L - 1) // 64] * 64 + (L - 1) % 64 for b, L in enumerate(w.seq_lens)], np.int32)
    slots = torch.from_numpy(last).cuda()
    tab = torch.from_numpy(table).cuda()
    seq = torch.tensor(w.seq_lens, dtype=torch.int32).cuda()
    # reference: separate encode then decode on a copy
    ref_pool = to_device(pool)
    tq4.tq4_encode_pages(ref_pool, k_new, v_new, slots)
    ref = tq4.tq4_attn_decode(ref_pool, q_t.cuda(), tab, seq, max(w.seq_lens), synth.SCALE)
    fused_pool = to_device(pool)
    ws = tq4.new_workspace(tq4.tq4_attn_decode_workspace_size(w.batch, max(w.seq_lens), w.n_q, w.n_kv, 64))
    for _ in range(2):
        got = tq4.tq4_attn_decode_append(fused_pool, k_new, v_new, slots, q_t.cuda(), tab, seq,
                                         max(w.seq_lens), synth.SCALE, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
    a, b = from_device(fused_pool), from_device(ref_pool)
    for x, y in ((a.k_words, b.k_words), (a.k_norms, b.k_norms), (a.v_words, b.v_words), (a.v_norms, b.v_norms)):
        np.testing.assert_array_equal(x, y)
    # and the new records are the oracle's
    chk = oracle.Pool(pool.k_words.copy(), pool.k_norms.copy(), pool.v_words.copy(), pool.v_norms.copy())
    oracle.encode_to_pool(chk, np.asarray(k_new.float().cpu()), np.asarray(v_new.float().cpu()), last)
    np.testing.assert_array_equal(a.k_words, chk.k_words)
    np.testing.assert_array_equal(a.v_norms, chk.v_norms)


def test_decode_workspace_reuse_across_pools():
    """One workspace serves consecutive calls on different pools and lengths (as the layers of a
    decode step do); every call matches the oracle."""
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    ws = tq4.new_workspace(tq4.tq4_attn_decode_workspace_size(2, 9000, 24, 4, 64))
    for layer, lens in enumerate([(9000, 4100), (300, 8999), (4096, 1)]):
        w = synth.Workload(100, "reuse", "decode", 1, 64, 300, seq_lens=lens)
        pool, table = oracle_pool(w, layer=layer)
        q_t, q64 = bf16_queries(w, layer, w.batch)
        got = tq4.tq4_attn_decode(to_device(pool), q_t.cuda(), torch.from_numpy(table).cuda(),
                                  torch.tensor(lens, dtype=torch.int32).cuda(), max(lens), synth.SCALE,
                                  workspace=ws)
        torch.cuda.synchronize()
        parity(got.cpu(), oracle.attn_decode(pool, q64, table, lens, synth.SCALE), f"reuse {lens}")


def test_decode_ignores_garbage_past_the_lengths():
    """Records past the lengths (inside the last tile and beyond) hold random bits, NaN and
    infinite norms among them; they must not reach the output."""
    w = synth.Workload(150, "garbage", "decode", 1, 64, 60, seq_lens=(1000, 37, 64 * 5 + 1))
    pool, table = oracle_pool(w, fill=np.random.default_rng(6))
    assert np.isnan(oracle.f16_bits_to_f64(pool.v_norms)).any()
    q_t, q64 = bf16_queries(w, 0, w.batch)
    ref = oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE)
    got = _run(to_device(pool), q_t, table, w.seq_lens, 1000)
    parity(got, ref, "garbage tail")


def test_side_stream_without_buffers():
    """Calls on a side stream with no output or workspace passed allocate them on that stream, so
    their fills are ordered before the kernels (decode, prefill and reconstruction, whose bf16
    outputs are zero-filled), while the current stream is kept busy."""
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    w = synth.Workload(101, "side", "decode", 1, 64, 120, seq_lens=(3000, 700))
    pool, table = oracle_pool(w)
    q_t, q64 = bf16_queries(w, 0, w.batch)
    dpool = to_device(pool)
    tab = torch.from_numpy(table).cuda()
    seq = torch.tensor(w.seq_lens, dtype=torch.int32).cuda()
    side = torch.cuda.Stream()
    busy = torch.ones(64 << 20, device="cuda")
    qd = q_t.cuda()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(4):
        busy.mul_(1.0)  # keeps the current stream occupied while the side stream works
    out = tq4.tq4_attn_decode(dpool, qd, tab, seq, 3000, synth.SCALE, stream=side)
    k, v = tq4.tq4_reconstruct_pages(dpool, tab, seq, 3000, stream=side)
    pq_t, pq64 = bf16_queries(w, 1, 40)
    pf = tq4.tq4_attn_prefill_chunk(dpool, pq_t.cuda(), tab[0].contiguous(), 2960, synth.SCALE, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    parity(out.cpu(), oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE), "side stream decode")
    ref_k, _ = oracle.reconstruct(pool, table, w.seq_lens, 3000)
    got_k = k.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.all(got_k[1, :, 700:] == 0)  # rows past the length keep the zero fill
    assert (got_k[0] == ref_k[0]).mean() > 0.99
    ref_pf = oracle.attn_prefill_rows(pool, pq64, np.arange(40), table[0], 2960, synth.SCALE)
    parity(pf.cpu(), ref_pf, "side stream prefill")
