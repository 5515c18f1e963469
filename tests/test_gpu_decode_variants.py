"""GPU parity of the decode variants without matrix cores (tq4_attn_decode_variant):
"valu_rotated" (the fused kernel's rotated-domain arithmetic on the vector ALUs) and
"valu_literal" (each key and value rebuilt in fp32 -- centroid lookup, inverse Hadamard rotation,
norm restore -- then natural-domain attention, the order of "Fitting a 27B-Parameter LLM into
24 GiB of Laptop Memory", section "KVExec: Fused Reconstruction with Layer-Scoped Lifetime").

Both are held to the attention bar against the fp64 oracle (max |err| <= 2e-2, rel-L2 <= 5e-3),
on the same seeded oracle-built pools as the fused kernel's tests."""
import numpy as np
import pytest

import oracle
import synth
from _pools import bf16_queries, oracle_pool, parity, to_device

pytestmark = pytest.mark.gpu

VARIANTS = ["valu_rotated", "valu_literal"]


def _run(dpool, q_t, table, seq_lens, max_seq, variant, scale=synth.SCALE):
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    out = tq4.tq4_attn_decode_variant(dpool, q_t.cuda(),
                                      torch.from_numpy(np.ascontiguousarray(table, np.int32)).cuda(),
                                      torch.tensor(seq_lens, dtype=torch.int32).cuda(), max_seq, scale, variant)
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("name", ["decode_1k_p64", "decode_32k"])
def test_variant_matches_oracle(variant, name):
    w = synth.WORKLOADS[name]
    pool, table = oracle_pool(w)
    q_t, q64 = bf16_queries(w, 0, w.batch)
    ref = oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE)
    got = _run(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens), variant)
    parity(got, ref, f"{variant} {name}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_variant_ragged_zero_and_clamped(variant):
    """Lengths 0, 1, a partial tile, a page plus one, and one past max_seq_len (clamped); page IDs
    shared by two requests."""
    w = synth.Workload(191, "ragged", "decode", 1, 64, 48, seq_lens=(1, 33, 1000, 64, 257),
                       shared_prefix_pages=1)
    pool, table = oracle_pool(w)
    q_t, q64 = bf16_queries(w, 0, w.batch + 1)
    table6 = np.vstack([table, table[2:3]])
    lens = list(w.seq_lens) + [0]
    got = _run(to_device(pool), q_t, table6, lens, 1000, variant)
    ref = oracle.attn_decode(pool, q64[:5], table, w.seq_lens, synth.SCALE)
    parity(got[:5], ref, f"{variant} ragged")
    assert np.all(got[5].float().numpy() == 0.0)
    clamped = _run(to_device(pool), q_t[2:3], table[2:3], [5000], 1000, variant)
    parity(clamped, ref[2:3], f"{variant} clamped")


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("n_q,n_kv,page", [(4, 4, 256), (8, 4, 32), (8, 1, 128), (12, 2, 64)])
def test_variant_group_and_page_sizes(variant, n_q, n_kv, page):
    w = synth.Workload(192, "groups", "decode", 1, page, 3000 // page + 8, seq_lens=(2999, 130),
                       n_kv=n_kv, n_q=n_q)
    pool, table = oracle_pool(w)
    q_t, q64 = bf16_queries(w, 0, w.batch)
    ref = oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE)
    got = _run(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens), variant)
    parity(got, ref, f"{variant} G={n_q // n_kv} P={page}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_variant_single_split_and_peaked(variant):
    """One workgroup per (request, KV head) writes the output itself; queries x8 sharpen the
    softmax so score precision matters."""
    w = synth.Workload(193, "peaked", "decode", 1, 64, 40, seq_lens=(200, 2000))
    pool, table = oracle_pool(w)
    q_t, q64 = bf16_queries(w, 0, w.batch, scale=8.0)
    ref = oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE)
    got1 = _run(to_device(pool), q_t[:1], table[:1], [200], 200, variant)
    parity(got1, ref[:1], f"{variant} single split")
    got = _run(to_device(pool), q_t, table, w.seq_lens, 2000, variant)
    parity(got, ref, f"{variant} peaked")


@pytest.mark.parametrize("variant", VARIANTS)
def test_variant_mixed_norms(variant):
    """Key norms over 10^4 and value norms over 10^6 from one position to the next."""
    w = synth.Workload(194, "mixed", "decode", 1, 64, 96, seq_lens=(4000, 900))
    n = len(synth.used_slots(w, synth.placement(w, 0)))
    kf = synth.log_uniform_f32(synth.seed_of(w.wid, 0, synth.T_KSCALE), n, 1e-2, 1e2)
    vf = synth.log_uniform_f32(synth.seed_of(w.wid, 0, synth.T_VSCALE), n, 1e-3, 1e3)
    pool, table = oracle_pool(w, kscale=kf, vscale=vf)
    q_t, q64 = bf16_queries(w, 0, w.batch, 1.0 / 16)
    ref = oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE)
    got = _run(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens), variant)
    parity(got, ref, f"{variant} mixed", value_scale=1e3)


@pytest.mark.parametrize("variant", VARIANTS)
def test_variant_full_212k_sampled_head(variant):
    """The full 212,992-position launch; the pool holds only KV head 1's records, which the oracle
    attends."""
    w = synth.WORKLOADS["decode_212k_16l"]
    g, layer = 1, 5
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
    got = _run(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens), variant)
    parity(got[:, g * G:(g + 1) * G], ref[:, g * G:(g + 1) * G], f"{variant} 212k head {g}")


def test_variants_agree_with_fused():
    """The three ways of computing decode agree within twice the attention bar."""
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    w = synth.WORKLOADS["decode_32k"]
    pool, table = oracle_pool(w)
    dpool = to_device(pool)
    q_t, _ = bf16_queries(w, 0, w.batch)
    fused = tq4.tq4_attn_decode(dpool, q_t.cuda(), torch.from_numpy(table.astype(np.int32)).cuda(),
                                torch.tensor(w.seq_lens, dtype=torch.int32).cuda(), max(w.seq_lens),
                                synth.SCALE).cpu().double().numpy()
    for variant in VARIANTS:
        got = _run(dpool, q_t, table, w.seq_lens, max(w.seq_lens), variant).double().numpy()
        assert float(np.max(np.abs(got - fused))) <= 4e-2, variant


def test_variant_validation():
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    from compressed_kv_attention_kvexec_amd import Tq4Error
    w = synth.Workload(195, "val", "decode", 1, 64, 8, seq_lens=(100,), n_q=48, n_kv=4)
    pool, table = oracle_pool(w)
    q_t, _ = bf16_queries(w, 0, 1)
    with pytest.raises(Tq4Error, match="TQ4_ERR_SHAPE"):  # group 12 is not built for the VALU kernels
        _run(to_device(pool), q_t, table, [100], 100, "valu_rotated")
    dpool = to_device(pool)
    lib = tq4.load_library()
    ps = dpool.struct()
    import ctypes
    qd = q_t.cuda()
    out = torch.empty_like(qd)
    tab = torch.from_numpy(table.astype(np.int32)).cuda()
    lens = torch.tensor([100], dtype=torch.int32).cuda()
    st = lib.tq4_attn_decode_variant(ctypes.byref(ps), qd.data_ptr(), 1, tab.data_ptr(), table.shape[1],
                                     lens.data_ptr(), 1, 100, 48, 0.0625, 7, out.data_ptr(), None, 0, None)
    assert st == 8  # TQ4_ERR_VALUE: unknown variant
