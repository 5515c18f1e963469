"""GPU encode parity: tq4_encode_pages must reproduce the oracle's records bit for bit."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _gpu_encode(workload, k, v, slots, dtype="f32"):
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    pool = tq4.Tq4LayerPool.empty(workload.pool_pages, workload.n_kv, workload.page_size)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    kt = None if k is None else torch.from_numpy(k).to(tdt).cuda().contiguous()
    vt = None if v is None else torch.from_numpy(v).to(tdt).cuda().contiguous()
    tq4.tq4_encode_pages(pool, kt, vt, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    from _pools import from_device
    return from_device(pool)


def _assert_pools_equal(a, b):
    np.testing.assert_array_equal(a.k_norms, b.k_norms)
    np.testing.assert_array_equal(a.v_norms, b.v_norms)
    np.testing.assert_array_equal(a.k_words, b.k_words)
    np.testing.assert_array_equal(a.v_words, b.v_words)


@pytest.mark.parametrize("name", ["decode_1k_p64", "decode_32k"])
def test_encode_bit_exact_workload(name):
    w = synth.WORKLOADS[name]
    table = synth.placement(w)
    slots = synth.used_slots(w, table)
    k = synth.kv_source(w, 0, len(slots), synth.T_K)
    v = synth.kv_source(w, 0, len(slots), synth.T_V)
    ref = oracle.Pool.empty(w.pool_pages, w.n_kv, w.page_size)
    oracle.encode_to_pool(ref, k, v, slots)
    got = _gpu_encode(w, k, v, slots)
    _assert_pools_equal(got, ref)


def test_encode_bf16_source_and_k_only():
    w = synth.WORKLOADS["decode_1k_p64"]
    slots = synth.used_slots(w, synth.placement(w))[:300]
    k = synth.bf16_round(synth.kv_source(w, 5, len(slots), synth.T_K) * 7.0)
    ref = oracle.Pool.empty(w.pool_pages, w.n_kv, w.page_size)
    oracle.encode_to_pool(ref, k, None, slots)
    got = _gpu_encode(w, k, None, slots, dtype="bf16")
    _assert_pools_equal(got, ref)


def test_encode_edge_vectors_and_bad_slots():
    """Zero, spike, constant, huge, tiny, overflowing and mixed-scale vectors; out-of-pool slots are
    skipped."""
    w = synth.Workload(90, "edge", "decode", 1, 64, 4, seq_lens=(256,), n_kv=2)
    rng = np.random.default_rng(90)
    n = 40
    k = rng.standard_normal((n, 2, 256)).astype(np.float32)
    k[0] = 0.0
    k[1] = 0.0
    k[1, :, 0] = 3.0
    k[2] = 1.0
    k[3] *= np.float32(1e17)
    k[4] *= np.float32(1e-20)
    k[5, 0, :128] *= np.float32(1e4)
    k[6, 1, ::2] = 0.0
    # the largest finite norms and squares that overflow (infinite norm), squares that underflow,
    # an infinite element, and a wavefront whose vectors mix finite and infinite norms
    unit = k / np.linalg.norm(k.astype(np.float64), axis=-1, keepdims=True)
    k[9] = (unit[9] * 1.5e19).astype(np.float32)
    k[10] *= np.float32(1e-30)
    k[11, 0, 5] = np.inf
    k[12, 1] *= np.float32(2e18)
    k[13] = (unit[13] * 2.5e19).astype(np.float32)
    v = -k[::-1].copy()
    slots = rng.permutation(4 * 64)[:n].astype(np.int32)
    ref = oracle.Pool.empty(4, 2, 64)
    oracle.encode_to_pool(ref, k, v, slots)
    bad = slots.copy()
    bad[7], bad[8] = -1, 4 * 64
    ref_bad = oracle.Pool.empty(4, 2, 64)
    keep = np.ones(n, bool)
    keep[[7, 8]] = False
    oracle.encode_to_pool(ref_bad, k[keep], v[keep], slots[keep])
    _assert_pools_equal(_gpu_encode(w, k, v, slots), ref)
    _assert_pools_equal(_gpu_encode(w, k, v, bad), ref_bad)


def test_encode_bit_exact_large_sample():
    """300k vectors of the 16-layer workload's first layer, as the pool build encodes them."""
    w = synth.WORKLOADS["decode_212k_16l"]
    table = synth.placement(w)
    slots = synth.used_slots(w, table)[:37_500]
    k = synth.kv_source(w, 0, len(slots), synth.T_K)
    v = synth.kv_source(w, 0, len(slots), synth.T_V)
    ref = oracle.Pool.empty(w.pool_pages, w.n_kv, w.page_size)
    oracle.encode_to_pool(ref, k, v, slots)
    _assert_pools_equal(_gpu_encode(w, k, v, slots), ref)


@pytest.mark.parametrize("n_kv,page", [(1, 32), (3, 96), (5, 160), (6, 64), (8, 1024)])
def test_encode_head_counts_and_page_sizes(n_kv, page):
    """Head counts and page sizes that are not powers of two: the slot -> (page, offset) and
    vector -> (token, head) divisions."""
    pages = 2048 // page + 3
    w = synth.Workload(91, "shapes", "decode", 1, page, pages, seq_lens=(64,), n_kv=n_kv)
    rng = np.random.default_rng(91 + n_kv)
    n = 257
    k = rng.standard_normal((n, n_kv, 256)).astype(np.float32)
    v = rng.standard_normal((n, n_kv, 256)).astype(np.float32) * np.float32(3.0)
    slots = rng.permutation(pages * page)[:n].astype(np.int32)
    slots[0] = pages * page - 1  # the pool's last slot
    ref = oracle.Pool.empty(pages, n_kv, page)
    oracle.encode_to_pool(ref, k, v, slots)
    _assert_pools_equal(_gpu_encode(w, k, v, slots), ref)
