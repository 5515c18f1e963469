"""Page tables from the library's allocator drive the GPU path: two requests with a shared prefix,
then a third that reuses pages the first gave back at the boundary; encode and decode attention
over those tables match the oracle, and the survivor's results do not change."""
import numpy as np
import pytest

import oracle
import synth
from _pools import parity, to_device

pytestmark = pytest.mark.gpu

P, PAGES, N_KV, N_Q = 64, 40, 4, 24


def _slots(table, positions):
    positions = np.asarray(positions)
    return (np.asarray(table)[positions // P] * P + positions % P).astype(np.int32)


def test_allocator_tables_drive_encode_and_decode():
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    from compressed_kv_attention_kvexec_amd.pages import PageAllocator
    rng = np.random.default_rng(130)
    alloc = PageAllocator(PAGES, P)
    a = alloc.admit(700, 200)
    assert alloc.extend(a, 900)
    b = alloc.admit(600, 100, prefix_pages=alloc.table(a)[:5])  # the first 320 positions are shared
    assert alloc.extend(b, 700)
    src_a = rng.standard_normal((2, 900, N_KV, 256)).astype(np.float32)
    src_b = rng.standard_normal((2, 700, N_KV, 256)).astype(np.float32)
    src_b[:, :320] = src_a[:, :320]
    ref_pool = oracle.Pool.empty(PAGES, N_KV, P)
    dpool = to_device(ref_pool)

    def encode(table, src, first, last):
        slots = _slots(table, np.arange(first, last))
        oracle.encode_to_pool(ref_pool, np.ascontiguousarray(src[0, first:last]),
                              np.ascontiguousarray(src[1, first:last]), slots)
        tq4.tq4_encode_pages(dpool, torch.from_numpy(np.ascontiguousarray(src[0, first:last])).cuda(),
                             torch.from_numpy(np.ascontiguousarray(src[1, first:last])).cuda(),
                             torch.from_numpy(slots).cuda())

    def attend(rids, lens, q64):
        stride = max(len(alloc.table(r)) for r in rids)
        table = np.zeros((len(rids), stride), np.int32)
        for i, r in enumerate(rids):
            t = alloc.table(r)
            table[i, :len(t)] = t
        q_t = torch.from_numpy(q64).to(torch.bfloat16)
        got = tq4.tq4_attn_decode(dpool, q_t.cuda(), torch.from_numpy(table).cuda(),
                                  torch.tensor(lens, dtype=torch.int32).cuda(), max(lens), synth.SCALE)
        torch.cuda.synchronize()
        ref = oracle.attn_decode(ref_pool, q64, table, lens, synth.SCALE)
        parity(got.cpu(), ref, f"allocator tables {lens}")
        return got.cpu()

    encode(alloc.table(a), src_a, 0, 900)
    encode(alloc.table(b), src_b, 320, 700)
    q = synth.bf16_round(rng.standard_normal((2, N_Q, 256)))
    out_ab = attend([a, b], [900, 700], q)

    table_a = alloc.table(a)
    alloc.finish(a)
    assert alloc.table(a)[:5] == alloc.table(b)[:5]  # still held before the boundary
    alloc.boundary()
    assert all(alloc.refcount(p) == 1 for p in alloc.table(b)[:5])
    a_private = set(table_a[5:])
    c = alloc.admit(1400, 100)
    assert alloc.extend(c, 1500)  # 24 pages: past the never-used ones into a's returned pages
    assert set(alloc.table(c)) & a_private
    src_c = rng.standard_normal((2, 1500, N_KV, 256)).astype(np.float32)
    encode(alloc.table(c), src_c, 0, 1500)
    q2 = np.stack([q[1], synth.bf16_round(rng.standard_normal((N_Q, 256)))])
    out_bc = attend([b, c], [700, 1500], q2)
    # b's pages were never reassigned: the same result up to the split plan's rounding
    assert (out_bc[0].double() - out_ab[1].double()).abs().max().item() < 4e-3
    alloc.close()
