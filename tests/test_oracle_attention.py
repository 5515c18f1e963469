"""Pins for the oracle's attention half: closed forms, a 50-digit brute force on
tiny inputs, GQA head mapping, and page-placement invariance."""
from fractions import Fraction

import mpmath
import numpy as np
import scipy.linalg

import synth


def _rand_pool(oracle_mod, num_pages, n_kv, P, n_tokens, seed):
    rng = np.random.default_rng(seed)
    pool = oracle_mod.Pool.empty(num_pages, n_kv, P)
    k = rng.standard_normal((n_tokens, n_kv, 256)).astype(np.float32)
    v = rng.standard_normal((n_tokens, n_kv, 256)).astype(np.float32)
    table = rng.permutation(num_pages)[: -(-n_tokens // P)].astype(np.int32)
    slots = (table[np.arange(n_tokens) // P] * P + np.arange(n_tokens) % P).astype(np.int32)
    oracle_mod.encode_to_pool(pool, k, v, slots)
    return pool, table


def _bf16_q(rows, n_q, seed, scale=1.0):
    return synth.bf16_round(np.random.default_rng(seed).standard_normal((rows, n_q, 256)) * scale)


def _records(pool, table, n_tokens, g, which):
    P = pool.page_size
    words = pool.k_words if which == "k" else pool.v_words
    norms = pool.k_norms if which == "k" else pool.v_norms
    pages, offs = table[np.arange(n_tokens) // P], np.arange(n_tokens) % P
    return words[pages, g, offs], norms[pages, g, offs]


def test_single_position_returns_its_value(oracle_mod):
    pool, table = _rand_pool(oracle_mod, 4, 2, 64, 1, 11)
    q = _bf16_q(1, 6, 12)
    out = oracle_mod.attn_decode(pool, q, table[None], [1], 1 / 16)
    for g in range(2):
        w, n = _records(pool, table, 1, g, "v")
        vh = oracle_mod.decode(w, n)[0]
        for h in range(3 * g, 3 * g + 3):
            np.testing.assert_array_equal(out[0, h], vh)


def test_two_positions_closed_form(oracle_mod):
    pool, table = _rand_pool(oracle_mod, 4, 1, 64, 2, 13)
    q = _bf16_q(1, 2, 14)
    out = oracle_mod.attn_decode(pool, q, table[None], [2], 1 / 16)
    kw, kn = _records(pool, table, 2, 0, "k")
    vw, vn = _records(pool, table, 2, 0, "v")
    kh, vh = oracle_mod.decode(kw, kn), oracle_mod.decode(vw, vn)
    for h in range(2):
        s0, s1 = (kh @ q[0, h].astype(np.float64)) / 16
        w0 = 1 / (1 + np.exp(s1 - s0))
        ref = w0 * vh[0] + (1 - w0) * vh[1]
        np.testing.assert_allclose(out[0, h], ref, rtol=1e-13, atol=1e-13)


def test_zero_query_and_identical_keys_give_mean_of_values(oracle_mod):
    n = 150
    pool, table = _rand_pool(oracle_mod, 8, 1, 64, n, 15)
    vw, vn = _records(pool, table, n, 0, "v")
    mean_v = oracle_mod.decode(vw, vn).mean(axis=0)
    out = oracle_mod.attn_decode(pool, np.zeros((1, 1, 256)), table[None], [n], 1 / 16)
    np.testing.assert_allclose(out[0, 0], mean_v, rtol=1e-12, atol=1e-12)
    # identical keys: copy one K record over every position
    P = pool.page_size
    pages, offs = table[np.arange(n) // P], np.arange(n) % P
    pool.k_words[pages, 0, offs] = pool.k_words[pages[0], 0, offs[0]]
    pool.k_norms[pages, 0, offs] = pool.k_norms[pages[0], 0, offs[0]]
    out = oracle_mod.attn_decode(pool, _bf16_q(1, 1, 16), table[None], [n], 1 / 16)
    np.testing.assert_allclose(out[0, 0], mean_v, rtol=1e-12, atol=1e-12)


def _mpf(fr):
    return mpmath.mpf(fr.numerator) / fr.denominator


def _exact_records(oracle_mod, pool, table, L, g):
    """Decoded K and V of positions 0..L-1 of KV head g in exact rationals (dense Hadamard)."""
    c, _ = oracle_mod.codebook()
    cF = [Fraction(float(v)) for v in c]
    H = scipy.linalg.hadamard(256)
    dec = {}
    for which in ("k", "v"):
        w, n = _records(pool, table, L, g, which)
        idx = oracle_mod.unpack(w)
        vecs = []
        for j in range(L):
            nj = Fraction(float(np.uint16(n[j]).view(np.float16)))
            ys = np.array([cF[i] for i in idx[j]], dtype=object)
            vecs.append([nj * sum(int(H[d, t]) * ys[t] for t in range(256)) / 16 for d in range(256)])
        dec[which] = vecs
    return dec


def _mp_attention(q_row, dec, n_keys, dims):
    """50-digit softmax attention of one query row over the first n_keys decoded positions."""
    qh = [Fraction(float(v)) for v in q_row]
    s = [_mpf(sum(a * b for a, b in zip(qh, dec["k"][j]))) / 16 for j in range(n_keys)]
    mx = max(s)
    e = [mpmath.exp(x - mx) for x in s]
    tot = sum(e)
    return [sum(e[j] * _mpf(dec["v"][j][d]) for j in range(n_keys)) / tot for d in dims]


def test_brute_force_50_digits(oracle_mod):
    """Dense Hadamard decode in exact rationals and softmax in 50-digit arithmetic."""
    mpmath.mp.dps = 50
    dims = (0, 5, 128, 255)
    for L, seed in [(1, 21), (3, 22), (8, 23)]:
        pool, table = _rand_pool(oracle_mod, 3, 2, 64, L, seed)
        q = _bf16_q(1, 4, seed + 100, scale=4.0)      # peaked softmax
        out = oracle_mod.attn_decode(pool, q, table[None], [L], 1 / 16)
        for g in range(2):
            dec = _exact_records(oracle_mod, pool, table, L, g)
            for h in (2 * g, 2 * g + 1):
                ref = _mp_attention(q[0, h], dec, L, dims)
                for d, r in zip(dims, ref):
                    assert abs(float(r) - out[0, h, d]) <= 1e-12 * max(1.0, abs(float(r)))


def test_verify_brute_force_50_digits(oracle_mod):
    """Packed verification of k = 3 queries over L = 5 positions: query i sees L - k + i + 1 keys
    (3, 4, 5), checked against the 50-digit brute force; with L = 2 < k the first query sees
    nothing (zeros) and the second sees one key (its value vector)."""
    mpmath.mp.dps = 50
    dims = (1, 64, 200)
    L, k = 5, 3
    pool, table = _rand_pool(oracle_mod, 3, 1, 64, L, 61)
    q = _bf16_q(k, 2, 62, scale=4.0).reshape(1, k, 2, 256)
    out = oracle_mod.attn_verify(pool, q, table[None], [L], 1 / 16)
    dec = _exact_records(oracle_mod, pool, table, L, 0)
    for i in range(k):
        for h in range(2):
            ref = _mp_attention(q[0, i, h], dec, L - k + i + 1, dims)
            for d, r in zip(dims, ref):
                assert abs(float(r) - out[0, i, h, d]) <= 1e-12 * max(1.0, abs(float(r)))
    short = oracle_mod.attn_verify(pool, q, table[None], [2], 1 / 16)
    assert np.all(short[0, 0] == 0.0)
    for h in range(2):
        for d in dims:
            assert abs(float(_mpf(dec["v"][0][d])) - short[0, 1, h, d]) <= 1e-12


def test_gqa_heads_read_their_group(oracle_mod):
    """With 12 query heads over 4 KV heads, head h reads KV head h // 3."""
    n = 70
    pool, table = _rand_pool(oracle_mod, 4, 4, 64, n, 31)
    q = _bf16_q(1, 12, 32)
    out = oracle_mod.attn_decode(pool, q, table[None], [n], 1 / 16)
    for h in range(12):
        g = h // 3
        single = oracle_mod.Pool(pool.k_words[:, g:g + 1].copy(), pool.k_norms[:, g:g + 1].copy(),
                                 pool.v_words[:, g:g + 1].copy(), pool.v_norms[:, g:g + 1].copy())
        ref = oracle_mod.attn_decode(single, q[:, h:h + 1], table[None], [n], 1 / 16)
        np.testing.assert_array_equal(out[0, h], ref[0, 0])


def test_physical_page_permutation_invariance(oracle_mod):
    n = 300
    pool, table = _rand_pool(oracle_mod, 8, 2, 64, n, 41)
    q = _bf16_q(2, 4, 42)
    tables = np.stack([table, table])
    out = oracle_mod.attn_decode(pool, q, tables, [n, n - 77], 1 / 16)
    perm = np.random.default_rng(43).permutation(8)
    inv = np.argsort(perm)
    moved = oracle_mod.Pool(pool.k_words[inv].copy(), pool.k_norms[inv].copy(),
                            pool.v_words[inv].copy(), pool.v_norms[inv].copy())
    out2 = oracle_mod.attn_decode(moved, q, perm[tables].astype(np.int32), [n, n - 77], 1 / 16)
    np.testing.assert_array_equal(out, out2)


def test_prefill_rows_are_causal(oracle_mod):
    """Row t of a chunk over P0 cached positions sees exactly P0 + t + 1 keys."""
    prior, chunk = 100, 28
    pool, table = _rand_pool(oracle_mod, 4, 1, 64, prior + chunk, 51)
    q = _bf16_q(chunk, 2, 52)
    rows = np.array([0, 5, 27])
    out = oracle_mod.attn_prefill_rows(pool, q[rows], rows, table, prior, 1 / 16)
    for r, t in enumerate(rows):
        ref = oracle_mod.attn_decode(pool, q[t:t + 1], table[None], [prior + t + 1], 1 / 16)
        np.testing.assert_array_equal(out[r], ref[0])
        shorter = oracle_mod.attn_decode(pool, q[t:t + 1], table[None], [prior + t], 1 / 16)
        assert np.any(out[r] != shorter[0])


def test_verify_rows_are_causal(oracle_mod):
    """Query i of k over L cached positions equals decode at length L - k + i + 1 and differs from
    decode one position shorter; k = 1 is decode."""
    k = 4
    pool, table = _rand_pool(oracle_mod, 6, 2, 64, 300, 71)
    tables = np.stack([table, table])
    lens = [300, 130]
    q = _bf16_q(2 * k, 4, 72).reshape(2, k, 4, 256)
    out = oracle_mod.attn_verify(pool, q, tables, lens, 1 / 16)
    for b in range(2):
        for i in range(k):
            n = lens[b] - k + i + 1
            ref = oracle_mod.attn_decode(pool, q[b, i][None], table[None], [n], 1 / 16)
            np.testing.assert_array_equal(out[b, i], ref[0])
            shorter = oracle_mod.attn_decode(pool, q[b, i][None], table[None], [n - 1], 1 / 16)
            assert np.any(out[b, i] != shorter[0])
    one = oracle_mod.attn_verify(pool, q[:, :1], tables, lens, 1 / 16)
    np.testing.assert_array_equal(one[:, 0], oracle_mod.attn_decode(pool, q[:, 0], tables, lens, 1 / 16))


def test_value_scale_equivariance_over_the_fp16_norm_range(oracle_mod):
    """The record keeps one fp16 norm per vector and attention restores it ("Fitting a 27B-Parameter
    LLM into 24 GiB of Laptop Memory", section "KVExec: Fused Reconstruction with Layer-Scoped
    Lifetime"), with no range limit stated.  Scaling every source vector by 2^k leaves the indices
    unchanged and multiplies each norm by 2^k exactly while it stays a normal fp16 number, so
    attention with values scaled by 2^k is exactly 2^k times the unscaled result; scaling the keys
    changes only the scores.  k spans norms from about 2^-13 to 2^15 (the fp16 normal range)."""
    rng = np.random.default_rng(41)
    P, n_tok, n_kv = 64, 150, 2
    k_src = rng.standard_normal((n_tok, n_kv, 256)).astype(np.float32)
    v_src = rng.standard_normal((n_tok, n_kv, 256)).astype(np.float32)
    table = rng.permutation(6)[:3].astype(np.int32)
    slots = (table[np.arange(n_tok) // P] * P + np.arange(n_tok) % P).astype(np.int32)
    q = _bf16_q(2, 4, 42)
    base = oracle_mod.Pool.empty(6, n_kv, P)
    oracle_mod.encode_to_pool(base, k_src, v_src, slots)
    ref = oracle_mod.attention(base, q, table[None], [0, 0], [n_tok, 77], 1 / 16)
    n16 = oracle_mod.f16_bits_to_f64(base.v_norms)
    for k in (-17, -8, 8, 11):
        pool = oracle_mod.Pool.empty(6, n_kv, P)
        oracle_mod.encode_to_pool(pool, k_src, np.ldexp(v_src, k).astype(np.float32), slots)
        np.testing.assert_array_equal(pool.v_words, base.v_words)
        np.testing.assert_array_equal(pool.k_norms, base.k_norms)
        np.testing.assert_array_equal(oracle_mod.f16_bits_to_f64(pool.v_norms), np.ldexp(n16, k))
        out = oracle_mod.attention(pool, q, table[None], [0, 0], [n_tok, 77], 1 / 16)
        np.testing.assert_array_equal(out, np.ldexp(ref, k))
    # keys scaled by 2^k: same indices, norms times 2^k, scores times 2^k (a sharper softmax)
    pool = oracle_mod.Pool.empty(6, n_kv, P)
    oracle_mod.encode_to_pool(pool, np.ldexp(k_src, 6).astype(np.float32), v_src, slots)
    np.testing.assert_array_equal(pool.k_words, base.k_words)
    np.testing.assert_array_equal(oracle_mod.f16_bits_to_f64(pool.k_norms),
                                  np.ldexp(oracle_mod.f16_bits_to_f64(base.k_norms), 6))
    sharp = oracle_mod.attention(pool, q[:1], table[None], [0], [n_tok], 1 / 16)
    q64 = np.asarray(q, np.float64)
    sharp_by_scale = oracle_mod.attention(base, q64[:1] * 64.0, table[None], [0], [n_tok], 1 / 16)
    np.testing.assert_allclose(sharp, sharp_by_scale, rtol=1e-12, atol=1e-12)
