"""Pins for the oracle's uniform INT8 arm (per-vector fp16 scale = fp16(max |x| / 127), codes
rint(x / scale) in [-127, 127], natural domain): hand-derived records, the nearest-code
characterisation by brute force over all 255 codes, exact rational scale rounding, the
quantisation bound, symmetries, and attention over INT8 pages against a 50-digit brute force and
closed forms."""
from fractions import Fraction

import mpmath
import numpy as np

DIM = 256


def _scale(o, bits):
    return o.f16_bits_to_f64(np.asarray(bits, np.uint16))


def _f16_exact(x: Fraction) -> int:
    """Round a positive rational in fp16's normal range to nearest, ties to even (exact)."""
    e = 0
    while x >= 2:
        x /= 2
        e += 1
    while x < 1:
        x *= 2
        e -= 1
    assert -14 <= e <= 15
    sc = x * 1024
    lo = sc.numerator // sc.denominator
    rem = sc - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    if lo == 2048:
        lo, e = 1024, e + 1
    return ((e + 15) << 10) | (lo - 1024)


def _f32_div_exact(a: float, b: float) -> float:
    """Correctly rounded fp32 quotient, by exact rationals (round to nearest, ties to even)."""
    q = Fraction(a) / Fraction(b)
    lo = np.float32(float(q))  # within one ulp; fix up by comparing exact distances
    best = None
    for c in (np.nextafter(lo, np.float32(-np.inf)), lo, np.nextafter(lo, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - q)
        key = (d, int(np.float32(c).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return float(best[1])


def test_worked_record_by_hand(oracle_mod):
    # max |x| = 127 -> scale 127 / 127 = 1 (fp16 0x3C00); codes are rint with ties to even
    x = np.zeros(DIM, np.float32)
    x[:9] = [127, -63.5, 0.5, 1.5, 2.5, -0.5, -2.5, 126.49, -127]
    codes, scale = oracle_mod.int8_encode(x)
    assert int(scale) == 0x3C00
    assert list(codes[:9]) == [127, -64, 0, 2, 2, 0, -2, 126, -127]
    assert np.all(codes[9:] == 0)
    # max |x| = 127 / 8 -> scale 2^-3 (0x3000); every value a multiple of 1/8 is exact
    y = np.arange(-128, 128, dtype=np.float32) / 8
    y[0] = -127 / 8  # keep |y| <= 127/8
    c2, s2 = oracle_mod.int8_encode(y)
    assert int(s2) == 0x3000
    np.testing.assert_array_equal(c2.astype(np.int64), np.rint(y * 8).astype(np.int64))


def test_zero_vector(oracle_mod):
    codes, scale = oracle_mod.int8_encode(np.zeros((2, DIM), np.float32))
    assert np.all(codes == 0) and np.all(scale == 0)
    assert np.all(oracle_mod.int8_decode(codes, scale) == 0.0)


def test_scale_is_exactly_rounded(oracle_mod):
    rng = np.random.default_rng(40)
    x = (rng.standard_normal((300, DIM)) * np.exp2(rng.integers(-8, 8, (300, 1)))).astype(np.float32)
    _, scales = oracle_mod.int8_encode(x)
    for row, bits in zip(x, scales):
        a = float(np.abs(row).max())
        s32 = _f32_div_exact(a, 127.0)
        assert int(bits) == _f16_exact(Fraction(s32)), a


def test_codes_are_nearest_by_brute_force(oracle_mod):
    """Each code is the nearest of all 255 codes to x / scale (fp64), ties to even; the fp32
    quotient may move a value within 2^-17 of a tie, which is then allowed either way."""
    rng = np.random.default_rng(41)
    x = np.concatenate([rng.standard_normal((40, DIM)), rng.laplace(size=(40, DIM)) * 3,
                        rng.uniform(-1, 1, (40, DIM)) * 1e-3]).astype(np.float32)
    codes, scales = oracle_mod.int8_encode(x)
    cand = np.arange(-127, 128, dtype=np.float64)
    for row, c, bits in zip(x, codes, scales):
        s = float(_scale(oracle_mod, bits))
        r = row.astype(np.float64) / s
        dist = np.abs(r[:, None] - cand[None, :])
        best = cand[np.argmin(dist, axis=1)]
        near_tie = np.abs(np.abs(r - np.floor(r)) - 0.5) < 2.0 ** -17
        ok = (c == best) | (near_tie & (np.abs(c - r) <= 0.5 + 2.0 ** -17))
        exact_tie = np.abs(r - np.floor(r)) == 0.5
        ok &= ~exact_tie | (c % 2 == 0)
        assert np.all(ok)
        assert np.abs(c).max() == 127


def test_quantisation_bound_and_range(oracle_mod):
    rng = np.random.default_rng(42)
    x = (rng.standard_normal((500, DIM)) * np.exp2(rng.integers(-5, 12, (500, 1)))).astype(np.float32)
    codes, scales = oracle_mod.int8_encode(x)
    s = _scale(oracle_mod, scales)
    assert np.all(s >= 2.0 ** -14)  # normal fp16 scales: rounding moves s by at most 2^-11
    xh = oracle_mod.int8_decode(codes, scales)
    assert codes.min() >= -127 and codes.max() <= 127
    err = np.abs(xh - x.astype(np.float64))
    assert np.all(err <= s[:, None] * (0.5 + 128 * 2.0 ** -24))
    np.testing.assert_array_equal(xh, codes.astype(np.float64) * s[:, None])


def test_subnormal_scales_clamp_within_range(oracle_mod):
    """max |x| below 127 * 2^-14 gives a subnormal fp16 scale (spacing 2^-24); a scale rounded
    down can put max |x| / s above 127.5, and those codes clamp to +-127."""
    rng = np.random.default_rng(48)
    x = (rng.standard_normal((400, DIM)) * np.exp2(rng.integers(-24, -12, (400, 1)))).astype(np.float32)
    codes, scales = oracle_mod.int8_encode(x)
    s = _scale(oracle_mod, scales)
    a = np.abs(x.astype(np.float64)).max(axis=1)
    assert np.all(s < 2.0 ** -14)
    assert codes.min() >= -127 and codes.max() <= 127
    err = np.abs(oracle_mod.int8_decode(codes, scales) - x.astype(np.float64))
    over = np.maximum(a - 127.5 * s, 0.0)
    live = s > 0
    assert np.all(err[live] <= (s * (0.5 + 2.0 ** -17) + over)[live, None])
    assert np.any(over > 0)  # the clamped case occurs in this sample
    assert np.all(codes[~live] == 0)


def test_representable_vectors_round_trip(oracle_mod):
    rng = np.random.default_rng(43)
    k = rng.integers(-127, 128, (50, DIM))
    k[:, 7] = np.where(rng.random(50) < 0.5, 127, -127)  # max |k| = 127
    e = rng.integers(-10, 6, (50, 1))
    x = (k * np.exp2(e)).astype(np.float32)
    codes, scales = oracle_mod.int8_encode(x)
    np.testing.assert_array_equal(codes, k.astype(np.int8))
    np.testing.assert_array_equal(_scale(oracle_mod, scales), np.exp2(e[:, 0]).astype(np.float64))
    np.testing.assert_array_equal(oracle_mod.int8_decode(codes, scales), x.astype(np.float64))


def test_sign_and_power_of_two_symmetry(oracle_mod):
    rng = np.random.default_rng(44)
    x = rng.standard_normal((64, DIM)).astype(np.float32)
    c0, s0 = oracle_mod.int8_encode(x)
    c1, s1 = oracle_mod.int8_encode(-x)
    np.testing.assert_array_equal(c1, -c0)
    np.testing.assert_array_equal(s1, s0)
    for j in (-5, 3):
        cj, sj = oracle_mod.int8_encode(x * np.float32(2.0 ** j))
        np.testing.assert_array_equal(cj, c0)
        np.testing.assert_array_equal(_scale(oracle_mod, sj), _scale(oracle_mod, s0) * 2.0 ** j)


def _pool(oracle_mod, rng, pages, n_kv, P, lens, perm_pages=True):
    pool = oracle_mod.Int8Pool.empty(pages, n_kv, P)
    stride = max((L + P - 1) // P for L in lens)
    order = rng.permutation(pages) if perm_pages else np.arange(pages)
    table = np.full((len(lens), stride), -1, np.int32)
    nxt = 0
    for b, L in enumerate(lens):
        need = (L + P - 1) // P
        table[b, :need] = order[nxt:nxt + need]
        nxt += need
    slots = np.concatenate([table[b, np.arange(L) // P] * P + np.arange(L) % P for b, L in enumerate(lens)])
    n = slots.size
    k = (rng.standard_normal((n, n_kv, DIM)) * rng.uniform(0.2, 3.0, (n, n_kv, 1))).astype(np.float32)
    v = rng.standard_normal((n, n_kv, DIM)).astype(np.float32)
    oracle_mod.int8_encode_to_pool(pool, k, v, slots.astype(np.int32))
    return pool, table


def test_attention_brute_force_50_digits(oracle_mod):
    rng = np.random.default_rng(45)
    lens = (9, 1, 0)
    pool, table = _pool(oracle_mod, rng, 8, 2, 4, lens)
    q = rng.standard_normal((3, 4, DIM))
    scale = 1 / 16
    got = oracle_mod.int8_attn_decode(pool, q, table, lens, scale)
    mpmath.mp.dps = 50
    P = 4
    for b, L in enumerate(lens):
        for h in range(4):
            g = h // 2
            if L == 0:
                assert np.all(got[b, h] == 0.0)
                continue
            ks, vs = [], []
            for j in range(L):
                pg, off = table[b, j // P], j % P
                s_k = mpmath.mpf(float(_scale(oracle_mod, pool.k_scales[pg, g, off])))
                s_v = mpmath.mpf(float(_scale(oracle_mod, pool.v_scales[pg, g, off])))
                ks.append([int(c) * s_k for c in pool.k_codes[pg, g, off]])
                vs.append([int(c) * s_v for c in pool.v_codes[pg, g, off]])
            sc = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(a)) * kk for a, kk in zip(q[b, h], kr)) for kr in ks]
            m = max(sc)
            w = [mpmath.exp(x - m) for x in sc]
            tot = mpmath.fsum(w)
            for d in range(0, DIM, 17):
                ref = mpmath.fsum(wi * vr[d] for wi, vr in zip(w, vs)) / tot
                assert abs(float(ref) - got[b, h, d]) <= 1e-12 * max(1.0, abs(float(ref)))


def test_attention_single_key_and_page_indirection(oracle_mod):
    rng = np.random.default_rng(46)
    lens = (1, 37)
    pool, table = _pool(oracle_mod, rng, 12, 2, 8, lens)
    q = rng.standard_normal((2, 6, DIM))
    out = oracle_mod.int8_attn_decode(pool, q, table, lens, 0.0625)
    # one key: the output is that key's value, exactly
    pg = table[0, 0]
    for h in range(6):
        np.testing.assert_array_equal(out[0, h], oracle_mod.int8_decode(pool.v_codes[pg, h // 3, 0],
                                                                       pool.v_scales[pg, h // 3, 0]))
    # moving the pages of request 1 and rewriting its table leaves the output unchanged
    moved = oracle_mod.Int8Pool.empty(12, 2, 8)
    new_ids = np.arange(11, -1, -1)
    for arr_src, arr_dst in ((pool.k_codes, moved.k_codes), (pool.k_scales, moved.k_scales),
                             (pool.v_codes, moved.v_codes), (pool.v_scales, moved.v_scales)):
        arr_dst[new_ids] = arr_src[np.arange(12)]
    t2 = np.where(table >= 0, new_ids[np.maximum(table, 0)], -1).astype(np.int32)
    out2 = oracle_mod.int8_attn_decode(moved, q, t2, lens, 0.0625)
    np.testing.assert_array_equal(out, out2)


def test_attention_equal_scores_is_mean_of_values(oracle_mod):
    """A zero query scores every key 0: the output is the plain mean of the decoded values."""
    rng = np.random.default_rng(47)
    lens = (50,)
    pool, table = _pool(oracle_mod, rng, 8, 1, 8, lens)
    out = oracle_mod.int8_attn_decode(pool, np.zeros((1, 2, DIM)), table, lens, 0.1)
    P = 8
    vals = np.stack([oracle_mod.int8_decode(pool.v_codes[table[0, j // P], 0, j % P],
                                            pool.v_scales[table[0, j // P], 0, j % P]) for j in range(50)])
    np.testing.assert_allclose(out[0, 0], vals.mean(axis=0), rtol=0, atol=1e-13)
    np.testing.assert_array_equal(out[0, 0], out[0, 1])


def test_int8_bytes_per_position(oracle_mod):
    # 256 one-byte codes + a two-byte scale per vector, K and V, 4 KV heads, 16 layers
    assert oracle_mod.int8_bytes_per_position() == 16 * 4 * 2 * 258 == 33024


def test_int8_verify_rows_are_decode_at_their_lengths(oracle_mod):
    """Query i of k attends exactly the first L - k + i + 1 positions (each row equals a decode at
    that length, bit for bit), and a query with no position gets zeros."""
    rng = np.random.default_rng(49)
    lens = (20, 2)
    pool, table = _pool(oracle_mod, rng, 8, 2, 8, lens)
    k = 4
    q = rng.standard_normal((2, k, 4, DIM))
    got = oracle_mod.int8_attn_verify(pool, q, table, lens, 0.0625)
    for b, L in enumerate(lens):
        for i in range(k):
            n = L - k + i + 1
            if n <= 0:
                assert np.all(got[b, i] == 0.0)
                continue
            ref = oracle_mod.int8_attn_decode(pool, q[b, i][None], table[b:b + 1], [n], 0.0625)
            np.testing.assert_array_equal(got[b, i], ref[0])
            if n > 1:  # and differs from one position fewer
                fewer = oracle_mod.int8_attn_decode(pool, q[b, i][None], table[b:b + 1], [n - 1], 0.0625)
                assert not np.array_equal(got[b, i], fewer[0])
