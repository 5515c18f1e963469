"""Pins for the oracle's unfused path (reconstruction into bf16 K/V, then dense attention):
bf16 rounding against exact rational rounding and torch, reconstruction against the pinned
record decoder and the rounding bound, dense attention against closed forms, a 50-digit brute
force, and the pinned attention over TQ4 pages."""
from fractions import Fraction

import mpmath
import numpy as np
import torch

import synth


def _bf16_exact(x: float) -> int:
    """Round-to-nearest-even onto 8-bit significands (bf16 normal range), by exact rationals."""
    if x == 0.0:
        return 0x8000 if np.signbit(x) else 0
    fr = Fraction(abs(x))
    e = 0
    while fr >= 2:
        fr /= 2
        e += 1
    while fr < 1:
        fr *= 2
        e -= 1
    assert -126 <= e <= 127
    scaled = fr * 128                      # in [128, 256)
    lo = scaled.numerator // scaled.denominator
    rem = scaled - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    if lo == 256:
        lo, e = 128, e + 1
    bits = ((e + 127) << 7) | (lo - 128)
    return (0x8000 if x < 0 else 0) | bits


def test_f64_to_bf16_matches_exact_rounding(oracle_mod):
    rng = np.random.default_rng(5)
    xs = list(rng.standard_normal(2000) * np.exp2(rng.integers(-30, 30, 2000)))
    # ties and near-ties around 1, 3 and -5
    for base in (1.0, 3.0, -5.0):
        ulp = abs(base) * 2.0 ** -7 / (2 if abs(base) >= 2 else 1)
        for k in range(8):
            xs += [base + k * ulp / 2, base + k * ulp / 2 + 2.0 ** -40, base + k * ulp / 2 - 2.0 ** -40]
    got = oracle_mod.f64_to_bf16_bits(np.array(xs))
    for x, g in zip(xs, got):
        assert int(g) == _bf16_exact(float(x)), x


def test_f64_to_bf16_matches_torch_on_fp32_values(oracle_mod):
    x = np.random.default_rng(6).standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle_mod.f64_to_bf16_bits(x.astype(np.float64)), ref)


def test_f64_to_bf16_single_step_differs_from_double_rounding(oracle_mod):
    # 1 + 2^-8 + 2^-30 rounds up to 1 + 2^-7 in one step, but to 1.0 through fp32 (tie to even)
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle_mod.f64_to_bf16_bits(np.array([x]))[0] == 0x3F81
    via_fp32 = torch.tensor([x], dtype=torch.float64).to(torch.float32).to(torch.bfloat16)
    assert via_fp32.view(torch.int16).item() == 0x3F80


def _pool(oracle_mod, seed, n_tokens, num_pages=6, n_kv=2, P=64):
    rng = np.random.default_rng(seed)
    pool = oracle_mod.Pool.empty(num_pages, n_kv, P)
    k = rng.standard_normal((n_tokens, n_kv, 256)).astype(np.float32)
    v = rng.standard_normal((n_tokens, n_kv, 256)).astype(np.float32)
    table = rng.permutation(num_pages)[: -(-n_tokens // P)].astype(np.int32)
    slots = (table[np.arange(n_tokens) // P] * P + np.arange(n_tokens) % P).astype(np.int32)
    oracle_mod.encode_to_pool(pool, k, v, slots)
    return pool, table


def test_reconstruct_is_rounded_record_decode(oracle_mod):
    L, P = 150, 64
    pool, table = _pool(oracle_mod, 41, L)
    tables = np.stack([table, table])
    k, v = oracle_mod.reconstruct(pool, tables, [L, 70], 160)
    for b, Lb in enumerate([L, 70]):
        for g in range(2):
            pages, offs = table[np.arange(Lb) // P], np.arange(Lb) % P
            for bits, words, norms in ((k, pool.k_words, pool.k_norms), (v, pool.v_words, pool.v_norms)):
                exact = oracle_mod.decode(words[pages, g, offs], norms[pages, g, offs])
                got = oracle_mod.bf16_bits_to_f64(bits[b, g, :Lb])
                np.testing.assert_array_equal(bits[b, g, :Lb], oracle_mod.f64_to_bf16_bits(exact))
                # the rounding bound: within half a bf16 unit of the exact value
                assert np.all(np.abs(got - exact) <= np.abs(exact) * 2.0 ** -8 + 1e-300)
                assert np.all(bits[b, g, Lb:] == 0)   # positions past the length are not written


def test_sdpa_dense_closed_forms(oracle_mod):
    rng = np.random.default_rng(7)
    q = synth.bf16_round(rng.standard_normal((2, 4, 256)))
    k = rng.standard_normal((2, 2, 5, 256))
    v = rng.standard_normal((2, 2, 5, 256))
    out = oracle_mod.sdpa_dense(q, k, v, [1, 0], 1 / 16)
    np.testing.assert_allclose(out[0, :2], np.repeat(v[0, 0, :1], 2, axis=0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[0, 2:], np.repeat(v[0, 1, :1], 2, axis=0), rtol=0, atol=1e-15)
    assert np.all(out[1] == 0.0)
    same = np.repeat(k[:, :, :1], 5, axis=2)
    out = oracle_mod.sdpa_dense(q, same, v, [5, 3], 1 / 16)   # identical keys: mean of the values
    np.testing.assert_allclose(out[0, 0], v[0, 0].mean(axis=0), atol=1e-14)
    np.testing.assert_allclose(out[1, 3], v[1, 1, :3].mean(axis=0), atol=1e-14)


def test_sdpa_dense_brute_force_50_digits(oracle_mod):
    mpmath.mp.dps = 50
    rng = np.random.default_rng(8)
    q = synth.bf16_round(rng.standard_normal((1, 2, 256)) * 3)
    k = synth.bf16_round(rng.standard_normal((1, 1, 4, 256)))
    v = synth.bf16_round(rng.standard_normal((1, 1, 4, 256)))
    out = oracle_mod.sdpa_dense(q, k, v, [4], 1 / 16)
    for h in range(2):
        s = [mpmath.mpf(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q[0, h], k[0, 0, j])).numerator)
             / sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q[0, h], k[0, 0, j])).denominator / 16
             for j in range(4)]
        mx = max(s)
        e = [mpmath.exp(x - mx) for x in s]
        for d in (0, 77, 255):
            ref = sum(e[j] * mpmath.mpf(float(v[0, 0, j, d])) for j in range(4)) / sum(e)
            assert abs(float(ref) - out[0, h, d]) <= 1e-13


def test_sdpa_dense_over_exact_decode_equals_tq4_attention(oracle_mod):
    L = 200
    pool, table = _pool(oracle_mod, 42, L)
    q = synth.bf16_round(np.random.default_rng(9).standard_normal((1, 4, 256)))
    P = pool.page_size
    pages, offs = table[np.arange(L) // P], np.arange(L) % P
    k = np.stack([oracle_mod.decode(pool.k_words[pages, g, offs], pool.k_norms[pages, g, offs]) for g in range(2)])
    v = np.stack([oracle_mod.decode(pool.v_words[pages, g, offs], pool.v_norms[pages, g, offs]) for g in range(2)])
    dense = oracle_mod.sdpa_dense(q, k[None], v[None], [L], 1 / 16)
    paged = oracle_mod.attn_decode(pool, q, table[None], [L], 1 / 16)
    np.testing.assert_allclose(dense, paged, rtol=1e-12, atol=1e-14)
