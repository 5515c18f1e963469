"""GPU parity where wavefronts own more than 64 tiles (the page-ID prefetch is refilled chunk by
chunk): a batch of 64 requests (one split per request and KV head, 67 tiles per decode wavefront,
133 per verifier wavefront) and one request of 1,500,000 positions (92 tiles per wavefront).  The
page tables alias a few distinct pages many times over, which is legal (shared pages) and keeps the
oracle's encoding small; the oracle checks sampled requests or one KV head."""
import numpy as np
import pytest

import oracle
import synth
from _pools import int8_to_device, parity, to_device

pytestmark = pytest.mark.gpu

P = 256


def _aliased(rng, n_distinct, n_kv, batch, stride):
    """Records for n_distinct pages and page tables [batch][stride] drawn from them."""
    slots = np.arange(n_distinct * P, dtype=np.int32)
    k = rng.standard_normal((len(slots), n_kv, 256)).astype(np.float32)
    v = rng.standard_normal((len(slots), n_kv, 256)).astype(np.float32)
    table = rng.integers(0, n_distinct, (batch, stride)).astype(np.int32)
    return slots, k, v, table


def _q(rng, rows, n_q):
    import torch
    qt = torch.from_numpy(rng.standard_normal((rows, n_q, 256)).astype(np.float32)).to(torch.bfloat16)
    return qt, qt.to(torch.float64).numpy()


def _batch64(seed):
    rng = np.random.default_rng(seed)
    batch, n_kv, n_q = 64, 4, 24
    lens = [16400 + 10 * b for b in range(batch)]
    stride = -(-max(lens) // P)
    slots, k, v, table = _aliased(rng, 24, n_kv, batch, stride)
    return rng, lens, slots, k, v, table, n_q


SAMPLED = (0, 31, 63)


def test_decode_batch64_many_tiles_per_wave():
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    rng, lens, slots, k, v, table, n_q = _batch64(160)
    pool = oracle.Pool.empty(24, 4, P)
    oracle.encode_to_pool(pool, k, v, slots)
    q_t, q64 = _q(rng, len(lens), n_q)
    out = tq4.tq4_attn_decode(to_device(pool), q_t.cuda(), torch.from_numpy(table).cuda(),
                              torch.tensor(lens, dtype=torch.int32).cuda(), max(lens), synth.SCALE)
    torch.cuda.synchronize()
    rows = np.array(SAMPLED, np.int32)
    ref = oracle.attention(pool, q64[rows], table, rows, np.array(lens, np.int32)[rows], synth.SCALE)
    parity(out.cpu()[list(SAMPLED)], ref, "decode batch 64")


def test_verify_batch64_many_tiles_per_wave():
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    rng, lens, slots, k, v, table, n_q = _batch64(161)
    pool = oracle.Pool.empty(24, 4, P)
    oracle.encode_to_pool(pool, k, v, slots)
    kq = 4
    q_t, q64 = _q(rng, len(lens) * kq, n_q)
    q_t = q_t.reshape(len(lens), kq, n_q, 256).contiguous()
    q64 = q64.reshape(len(lens), kq, n_q, 256)
    out = tq4.tq4_attn_verify(to_device(pool), q_t.cuda(), torch.from_numpy(table).cuda(),
                              torch.tensor(lens, dtype=torch.int32).cuda(), max(lens), synth.SCALE)
    torch.cuda.synchronize()
    got = out.cpu()
    for b in SAMPLED:
        rows = np.full(kq, b, np.int32)
        row_len = np.array([lens[b] - kq + i + 1 for i in range(kq)], np.int32)
        ref = oracle.attention(pool, q64[b], table, rows, row_len, synth.SCALE)
        parity(got[b], ref, f"verify batch 64 request {b}")


def test_int8_decode_batch64_many_tiles_per_wave():
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    rng, lens, slots, k, v, table, n_q = _batch64(162)
    pool = oracle.Int8Pool.empty(24, 4, P)
    oracle.int8_encode_to_pool(pool, k, v, slots)
    q_t, q64 = _q(rng, len(lens), n_q)
    out = tq4.tq4_int8_attn_decode(int8_to_device(pool), q_t.cuda(), torch.from_numpy(table).cuda(),
                                   torch.tensor(lens, dtype=torch.int32).cuda(), max(lens), synth.SCALE)
    torch.cuda.synchronize()
    rows = np.array(SAMPLED, np.int32)
    sub = table[rows]
    ref = oracle.int8_attn_decode(pool, q64[rows], sub, np.array(lens, np.int32)[rows], synth.SCALE)
    parity(out.cpu()[list(SAMPLED)], ref, "int8 batch 64")


def _long(seed):
    rng = np.random.default_rng(seed)
    L, n_kv, n_q = 1_500_000, 4, 24
    slots, k, v, table = _aliased(rng, 16, n_kv, 1, -(-L // P))
    return rng, L, slots, k, v, table, n_q


def test_decode_1_5M_positions_one_head():
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    rng, L, slots, k, v, table, n_q = _long(163)
    pool = oracle.Pool.empty(16, 4, P)
    oracle.encode_to_pool(pool, k, v, slots)
    q_t, q64 = _q(rng, 1, n_q)
    out = tq4.tq4_attn_decode(to_device(pool), q_t.cuda(), torch.from_numpy(table).cuda(),
                              torch.tensor([L], dtype=torch.int32).cuda(), L, synth.SCALE)
    torch.cuda.synchronize()
    ref = oracle.attn_decode(pool, q64, table, [L], synth.SCALE, heads=(6, 12))
    parity(out.cpu()[:, 6:12], ref[:, 6:12], "decode 1.5M")


def test_int8_decode_1_5M_positions_one_head():
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    rng, L, slots, k, v, table, n_q = _long(164)
    pool = oracle.Int8Pool.empty(16, 4, P)
    oracle.int8_encode_to_pool(pool, k, v, slots)
    q_t, q64 = _q(rng, 1, n_q)
    out = tq4.tq4_int8_attn_decode(int8_to_device(pool), q_t.cuda(), torch.from_numpy(table).cuda(),
                                   torch.tensor([L], dtype=torch.int32).cuda(), L, synth.SCALE)
    torch.cuda.synchronize()
    ref = oracle.int8_attn_decode(pool, q64, table, [L], synth.SCALE, heads=(18, 24))
    parity(out.cpu()[:, 18:24], ref[:, 18:24], "int8 1.5M")
