"""GPU parity over the range of the fp16 norm field.

A TQ4 record keeps one fp16 norm per vector and attention restores it ("Fitting a 27B-Parameter
LLM into 24 GiB of Laptop Memory", section "KVExec: Fused Reconstruction with Layer-Scoped
Lifetime"); nothing there limits its range, and the oracle handles any norm exactly.  These tests
run decode, the packed verifier and chunked prefill on pools whose sources are scaled so that
norms span about 2^-6 .. 2^14 (uniform scales from 1e-3 to 1e3), and on mixed pools whose key and
value norms vary by 10^4 to 10^6 from one position to the next.

Bar: the spec bar (max |err| <= 2e-2, rel-L2 <= 5e-3) in units of the value scale s: the
outputs and their bf16 rounding scale with s, so the absolute bound is 2e-2 s (s = the largest
value factor for a mixed pool); the relative bound is unchanged.  Key scales above 10 come with
queries scaled by the inverse factor, so the logits stay of order one (the norms are what is
tested, not logits of several hundred)."""
import numpy as np
import pytest

import oracle
import synth
from _pools import bf16_queries, oracle_pool, parity, to_device

pytestmark = pytest.mark.gpu

# (key factor, value factor, query factor); norms are about 16 x the factor
UNIFORM = [(1e-3, 1e-3, 1.0), (1e-1, 1e-1, 1.0), (10.0, 10.0, 1.0), (100.0, 100.0, 1e-2),
           (1000.0, 1000.0, 1e-3), (1.0, 1e-3, 1.0), (1.0, 1000.0, 1.0), (100.0, 1000.0, 0.1)]


def _mixed(w, layer, n, vlo=1e-2, vhi=1e2):
    """Per-position factors: keys log-uniform in [1e-2, 1e2], values in [vlo, vhi]."""
    return (synth.log_uniform_f32(synth.seed_of(w.wid, layer, synth.T_KSCALE), n, 1e-2, 1e2),
            synth.log_uniform_f32(synth.seed_of(w.wid, layer, synth.T_VSCALE), n, vlo, vhi))


def _decode(dpool, q_t, table, seq_lens, max_seq):
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    out = tq4.tq4_attn_decode(dpool, q_t.cuda(), torch.from_numpy(np.ascontiguousarray(table, np.int32)).cuda(),
                              torch.tensor(seq_lens, dtype=torch.int32).cuda(), max_seq, synth.SCALE)
    torch.cuda.synchronize()
    return out.cpu()


def _verify(dpool, q_t, table, seq_lens, max_seq):
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    out = tq4.tq4_attn_verify(dpool, q_t.cuda(), torch.from_numpy(np.ascontiguousarray(table, np.int32)).cuda(),
                              torch.tensor(seq_lens, dtype=torch.int32).cuda(), max_seq, synth.SCALE)
    torch.cuda.synchronize()
    return out.cpu()


def _prefill(dpool, q_t, table_row, prior):
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    out = tq4.tq4_attn_prefill_chunk(dpool, q_t.cuda(), torch.from_numpy(np.ascontiguousarray(table_row, np.int32)).cuda(),
                                     prior, synth.SCALE)
    torch.cuda.synchronize()
    return out.cpu()


def _vq(w, k, layer=0, scale=1.0):
    q_t, q64 = bf16_queries(w, layer, w.batch * k, scale)
    return q_t.reshape(w.batch, k, w.n_q, 256).contiguous(), q64.reshape(w.batch, k, w.n_q, 256)


@pytest.mark.parametrize("ks,vs,qs", UNIFORM)
def test_decode_uniform_scales(ks, vs, qs):
    w = synth.Workload(160, "nr_dec", "decode", 1, 64, 120, seq_lens=(3000, 700, 5))
    pool, table = oracle_pool(w, kscale=ks, vscale=vs)
    q_t, q64 = bf16_queries(w, 0, w.batch, qs)
    ref = oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE)
    got = _decode(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens))
    parity(got, ref, f"decode k x{ks} v x{vs}", value_scale=vs)


@pytest.mark.parametrize("vlo,vhi", [(1e-2, 1e2), (1e-3, 1e3)])
def test_decode_mixed_norms(vlo, vhi):
    w = synth.Workload(161, "nr_mix", "decode", 1, 64, 120, seq_lens=(3000, 700, 5))
    n = len(synth.used_slots(w, synth.placement(w, 0)))
    kf, vf = _mixed(w, 0, n, vlo, vhi)
    pool, table = oracle_pool(w, kscale=kf, vscale=vf)
    q_t, q64 = bf16_queries(w, 0, w.batch, 1.0 / 16)
    ref = oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE)
    got = _decode(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens))
    parity(got, ref, f"decode mixed v in [{vlo}, {vhi}]", value_scale=vhi)


def test_decode_single_split_large_and_small_norms():
    """One workgroup per request (the split kernel writes the output itself)."""
    w = synth.Workload(162, "nr_one", "decode", 1, 32, 16, seq_lens=(200, 31, 1))
    n = len(synth.used_slots(w, synth.placement(w, 0)))
    kf, vf = _mixed(w, 0, n, 1e-3, 1e3)
    pool, table = oracle_pool(w, kscale=kf, vscale=vf)
    q_t, q64 = bf16_queries(w, 0, w.batch, 1.0 / 16)
    ref = oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE)
    got = _decode(to_device(pool), q_t, table, w.seq_lens, 200)
    parity(got, ref, "single split mixed", value_scale=1e3)


@pytest.mark.parametrize("k", [4, 8])
@pytest.mark.parametrize("mode", ["v1000", "mixed"])
def test_verify_norm_range(k, mode):
    w = synth.Workload(163, "nr_ver", "decode", 1, 64, 120, seq_lens=(3000, 700, 5))
    n = len(synth.used_slots(w, synth.placement(w, 0)))
    if mode == "v1000":
        kf, vf, vs = 1.0, 1000.0, 1000.0
        qs = 1.0
    else:
        kf, vf = _mixed(w, 0, n, 1e-3, 1e3)
        vs, qs = 1e3, 1.0 / 16
    pool, table = oracle_pool(w, kscale=kf, vscale=vf)
    q_t, q64 = _vq(w, k, scale=qs)
    ref = oracle.attn_verify(pool, q64, table, w.seq_lens, synth.SCALE)
    got = _verify(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens))
    parity(got, ref, f"verify k={k} {mode}", value_scale=vs)


@pytest.mark.parametrize("mode", ["v1000", "v0.001", "mixed"])
def test_prefill_norm_range(mode):
    prior, chunk = 3000, 300
    w = synth.Workload(164, "nr_pf", "prefill", 1, 256, (prior + chunk) // 256 + 5, prior_len=prior,
                       chunk_len=chunk)
    n = prior + chunk
    if mode == "mixed":
        kf, vf = _mixed(w, 0, n, 1e-3, 1e3)
        vs, qs = 1e3, 1.0 / 16
    else:
        kf, vf = 1.0, float(mode[1:])
        vs, qs = vf, 1.0
    pool, table = oracle_pool(w, kscale=kf, vscale=vf)
    q_t, q64 = bf16_queries(w, 0, chunk, qs)
    ref = oracle.attn_prefill_rows(pool, q64, np.arange(chunk), table[0], prior, synth.SCALE)
    got = _prefill(to_device(pool), q_t, table[0], prior)
    parity(got, ref, f"prefill {mode}", value_scale=vs)


def _one_head_mixed(w, g, layer):
    """A full-size pool holding only KV head g's records, from mixed-norm sources (keys in
    [1e-2, 1e2], values in [1e-3, 1e3] times N(0,1))."""
    table = synth.placement(w, layer)
    slots = synth.used_slots(w, table)
    kf, vf = _mixed(w, layer, len(slots), 1e-3, 1e3)
    pool = oracle.Pool.empty(w.pool_pages, w.n_kv, w.page_size)
    one = oracle.Pool.empty(w.pool_pages, 1, w.page_size)
    kk = np.ascontiguousarray(synth.kv_source(w, layer, len(slots), synth.T_K)[:, g:g + 1] * kf[:, None, None])
    vv = np.ascontiguousarray(synth.kv_source(w, layer, len(slots), synth.T_V)[:, g:g + 1] * vf[:, None, None])
    oracle.encode_to_pool(one, kk, vv, slots)
    for dst, src in ((pool.k_words, one.k_words), (pool.k_norms, one.k_norms),
                     (pool.v_words, one.v_words), (pool.v_norms, one.v_norms)):
        dst[:, g] = src[:, 0]
    return pool, table


def test_decode_full_212k_mixed_norms_sampled_head():
    w = synth.WORKLOADS["decode_212k_16l"]
    g, layer = 0, 7
    pool, table = _one_head_mixed(w, g, layer)
    G = w.n_q // w.n_kv
    q_t, q64 = bf16_queries(w, layer, w.batch, 1.0 / 16)
    ref = oracle.attn_decode(pool, q64, table, w.seq_lens, synth.SCALE, heads=(g * G, (g + 1) * G))
    got = _decode(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens))
    parity(got[:, g * G:(g + 1) * G], ref[:, g * G:(g + 1) * G], "212k mixed", value_scale=1e3)


def test_verify_full_212k_mixed_norms_sampled_head():
    w = synth.WORKLOADS["decode_212k_16l"]
    g, layer, k = 3, 8, 8
    pool, table = _one_head_mixed(w, g, layer)
    G = w.n_q // w.n_kv
    q_t, q64 = _vq(w, k, layer, 1.0 / 16)
    ref = oracle.attn_verify(pool, q64, table, w.seq_lens, synth.SCALE, heads=(g * G, (g + 1) * G))
    got = _verify(to_device(pool), q_t, table, w.seq_lens, max(w.seq_lens))
    parity(got[:, :, g * G:(g + 1) * G], ref[:, :, g * G:(g + 1) * G], "212k verify mixed", value_scale=1e3)


def test_prefill_full_size_mixed_norms_sampled_rows():
    w = synth.WORKLOADS["prefill_2k_over_194k"]
    g = 1
    pool, table = _one_head_mixed(w, g, 0)
    q_t, q64 = bf16_queries(w, 0, w.chunk_len, 1.0 / 16)
    got = _prefill(to_device(pool), q_t, table[0], w.prior_len)
    G = w.n_q // w.n_kv
    rows = np.array([0, 5, 1024, 2047])
    ref = oracle.attn_prefill_rows(pool, q64[rows], rows, table[0], w.prior_len, synth.SCALE,
                                   heads=(g * G, (g + 1) * G))
    parity(got[rows, g * G:(g + 1) * G], ref[:, g * G:(g + 1) * G], "prefill full mixed", value_scale=1e3)
