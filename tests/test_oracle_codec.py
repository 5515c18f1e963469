"""Pins for the oracle's codec half: sizes, fp16 rounding, the Hadamard rotation,
the Lloyd-Max codebook, the encoder and the exact decoder.

Every check compares the oracle with something other than itself: figures the
JustFit pages print (tests/golden/page_figures.json), closed forms, scipy /
numpy library routines, or exact rational arithmetic.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg
import scipy.stats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _figures():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------- sizes (P1)

def test_record_and_position_sizes_match_pages(oracle_mod):
    fig = _figures()
    rec, geo, sz = fig["record"], fig["geometry"], fig["sizes"]
    # a vector: 32 words of 8 four-bit indices cover 256 dims, plus one fp16 norm
    assert rec["u32_words_per_vector"] * rec["indices_per_word"] == geo["head_dim"]
    assert oracle_mod.bytes_per_vector() == rec["u32_words_per_vector"] * 4 + 2 == 130
    L, H = geo["full_attention_layers"], geo["kv_heads"]
    assert oracle_mod.bytes_per_position(L, H) == sz["tq4_bytes_per_position"]
    assert oracle_mod.fp16_bytes_per_position(L, H, geo["head_dim"]) == sz["fp16_bytes_per_position"]
    mib = 2 ** 20
    assert oracle_mod.bytes_per_position(L, H) * sz["positions"] / mib == sz["tq4_mib_at_positions"]
    assert oracle_mod.fp16_bytes_per_position(L, H) * sz["positions"] / mib == sz["fp16_mib_at_positions"]
    assert round(sz["fp16_mib_at_positions"] / sz["tq4_mib_at_positions"], 2) == sz["reduction"]
    # one layer's BF16 K and V at 192K positions
    bf16_layer = sz["bf16_layer_positions"] * H * 2 * geo["head_dim"] * 2
    assert bf16_layer / mib == sz["bf16_layer_mib"]
    # the LM head expressed in cached positions
    lm = fig["lm_head"]
    assert round(lm["mib"] * mib / oracle_mod.bytes_per_position(L, H)) == lm["equivalent_positions"]
    cap = fig["capacity"]
    assert cap["input_tokens"] + cap["output_tokens"] == cap["completed_positions"]
    assert cap["pool_positions"] % cap["page_size"] == 0


# ---------------------------------------------------------- fp16 rounding

def test_f32_to_f16_matches_numpy_rne(oracle_mod):
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(30.0),
        (rng.standard_normal(20000) * 1e-5).astype(np.float32),          # fp16 subnormal range
        np.exp(rng.uniform(-20, 12, 20000)).astype(np.float32),
        np.array([0.0, -0.0, 65504.0, 65520.0, 65519.99, 1e6, -1e6, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 2.0 ** -26, np.inf, -np.inf, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, 2.0 ** -14 - 2.0 ** -26], np.float32),
    ])
    # ties: values exactly halfway between adjacent halves
    h = rng.integers(0x0001, 0x7bff, 5000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float32)
    hi = (h + 1).view(np.float16).astype(np.float32)
    vals = np.concatenate([vals, (lo + (hi - lo) / 2).astype(np.float32)])
    ours = oracle_mod.f32_to_f16_bits(vals)
    ref = vals.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = oracle_mod.f16_bits_to_f64(ours[:2000])
    np.testing.assert_array_equal(back, ref[:2000].view(np.float16).astype(np.float64))


# ------------------------------------------------------ Hadamard rotation (P2)

def _popcount_sign(i, j):
    return -1.0 if bin(i & j).count("1") % 2 else 1.0


def test_fwht_columns_are_sylvester_hadamard(oracle_mod):
    eye = np.eye(256)
    cols = oracle_mod.fwht_f64(eye)         # row j = FWHT(e_j) = column j of H
    H = scipy.linalg.hadamard(256).astype(np.float64)
    np.testing.assert_array_equal(cols.T, H)
    for i, j in [(0, 0), (3, 5), (255, 255), (128, 127), (77, 200)]:
        assert cols[j, i] == _popcount_sign(i, j)
    np.testing.assert_array_equal(H @ H.T, 256 * np.eye(256))
    np.testing.assert_array_equal(H, H.T)


def test_fwht_f32_involution_exact_on_small_integers(oracle_mod):
    rng = np.random.default_rng(2)
    x = rng.integers(-1000, 1000, (50, 256)).astype(np.float32)
    y = oracle_mod.fwht_f32(oracle_mod.fwht_f32(x))
    np.testing.assert_array_equal(y, 256 * x)


def test_fwht_f32_close_to_dense_product(oracle_mod):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((100, 256)).astype(np.float32)
    H = scipy.linalg.hadamard(256).astype(np.float64)
    ref = x.astype(np.float64) @ H.T
    got = oracle_mod.fwht_f32(x).astype(np.float64)
    assert np.max(np.abs(got - ref)) < 1e-4
    np.testing.assert_array_equal(oracle_mod.fwht_f64(x.astype(np.float64)), ref)


def test_fwht_f32_stage_order_is_ascending(oracle_mod):
    """fp32 rounding depends on the stage order; pin ascending stages h = 1..128."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((20, 256)).astype(np.float32)

    def fwht_np(v, order):
        v = v.copy()
        for h in order:
            idx = np.arange(256)
            lo = idx[(idx & h) == 0]
            a, b = v[:, lo].copy(), v[:, lo + h].copy()
            v[:, lo] = a + b
            v[:, lo + h] = a - b
        return v

    asc = fwht_np(x, [1, 2, 4, 8, 16, 32, 64, 128])
    desc = fwht_np(x, [128, 64, 32, 16, 8, 4, 2, 1])
    got = oracle_mod.fwht_f32(x)
    np.testing.assert_array_equal(got, asc)
    assert np.any(got != desc)


# ---------------------------------------------------------- codebook (P3)

def test_lloyd_max_conditions_hold_by_independent_integration(oracle_mod):
    lev, bnd, dist, iters = oracle_mod.lloyd_max16()
    assert iters > 0
    assert np.all(np.diff(lev) > 0)
    np.testing.assert_allclose(lev, -lev[::-1], atol=1e-14)
    np.testing.assert_allclose(bnd, 0.5 * (lev[:-1] + lev[1:]), atol=0)
    edges = np.concatenate([[-np.inf], bnd, [np.inf]])
    pdf = scipy.stats.norm.pdf
    d_total = 0.0
    for i in range(16):
        a, b = edges[i], edges[i + 1]
        mass = scipy.stats.norm.cdf(b) - scipy.stats.norm.cdf(a) if a < 0 else \
            scipy.stats.norm.sf(a) - scipy.stats.norm.sf(b)
        m1, _ = scipy.integrate.quad(lambda t: t * pdf(t), a, b, epsabs=1e-14, epsrel=1e-13)
        assert abs(m1 / mass - lev[i]) < 1e-9, (i, m1 / mass, lev[i])
        di, _ = scipy.integrate.quad(lambda t: (t - lev[i]) ** 2 * pdf(t), a, b,
                                     epsabs=1e-15, epsrel=1e-12)
        d_total += di
    assert abs(d_total - dist) < 1e-10
    # 16-level Gaussian Lloyd-Max distortion is about 0.0095 (Max, 1960)
    assert 0.00948 < dist < 0.00952


def test_codebook_fp32_tables(oracle_mod):
    lev, _, _, _ = oracle_mod.lloyd_max16()
    c, b = oracle_mod.codebook()
    np.testing.assert_array_equal(c, (lev / 16.0).astype(np.float32))
    np.testing.assert_array_equal(b, ((c[:-1].astype(np.float64) + c[1:]) / 2).astype(np.float32))
    np.testing.assert_array_equal(c[::-1], -c)
    assert b[7] == 0.0
    # every centroid is a multiple of 2^-30 below 2^-2 (the fp64 decode exactness argument)
    scaled = c.astype(np.float64) * 2.0 ** 30
    np.testing.assert_array_equal(scaled, np.round(scaled))
    assert np.all(np.abs(c) < 0.25)


# ------------------------------------------------------------ encoder (P4, P5)

def test_pack_worked_example(oracle_mod):
    idx = (np.arange(256) % 16).astype(np.uint8)
    words = oracle_mod.pack(idx)
    expect = np.array([0x76543210, 0xFEDCBA98] * 16, np.uint32)
    np.testing.assert_array_equal(words, expect)
    np.testing.assert_array_equal(oracle_mod.unpack(words), idx)
    rng = np.random.default_rng(5)
    w = rng.integers(0, 2 ** 32, (10, 32), dtype=np.uint64).astype(np.uint32)
    np.testing.assert_array_equal(oracle_mod.pack(oracle_mod.unpack(w)), w)


def test_encode_is_nearest_centroid_of_rotated_unit_vector(oracle_mod):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((400, 256)).astype(np.float32) * np.float32(3.0)
    words, norms = oracle_mod.encode(x)
    idx = oracle_mod.unpack(words).astype(np.int64)
    c, _ = oracle_mod.codebook()
    H = scipy.linalg.hadamard(256).astype(np.float64)
    x64 = x.astype(np.float64)
    n64 = np.linalg.norm(x64, axis=1, keepdims=True)
    z = (x64 @ H.T) / (16.0 * n64)
    brute = np.argmin(np.abs(z[..., None] - c.astype(np.float64)), axis=-1)
    mism = idx != brute
    # a disagreement may only come from fp32 rounding right at a decision boundary
    mids = (c[:-1].astype(np.float64) + c[1:]) / 2
    if mism.any():
        dist_to_mid = np.min(np.abs(z[mism][:, None] - mids), axis=1)
        assert np.all(dist_to_mid < 1e-6), dist_to_mid
    assert mism.mean() < 1e-3
    # fp16 norm: within one fp16 ulp of the true norm
    nr = oracle_mod.f16_bits_to_f64(norms)
    assert np.all(np.abs(nr - n64[:, 0]) <= np.abs(n64[:, 0]) * 2.0 ** -11 * 1.0001)


def test_encode_spike_vector_closed_form(oracle_mod):
    """x = a e_0 rotates to y = a (all dims); the unit coordinate is sign(a)/16,
    whose nearest centroid is index 11 (a > 0) or 4 (a < 0)."""
    for a, want in [(2.5, 11), (-0.75, 4), (1000.0, 11)]:
        x = np.zeros((1, 256), np.float32)
        x[0, 0] = a
        words, norms = oracle_mod.encode(x)
        assert np.all(oracle_mod.unpack(words) == want)
        assert norms[0] == np.float16(abs(a)).view(np.uint16)


def test_encode_zero_vector(oracle_mod):
    words, norms = oracle_mod.encode(np.zeros((1, 256), np.float32))
    assert norms[0] == 0 and np.all(words == 0)
    np.testing.assert_array_equal(oracle_mod.decode(words, norms), 0.0)


def test_roundtrip_of_vectors_built_from_centroids(oracle_mod):
    """x = s * H c[idx] / 16 with ||c[idx]|| near 1 must re-encode to idx exactly."""
    rng = np.random.default_rng(7)
    c, _ = oracle_mod.codebook()
    H = scipy.linalg.hadamard(256).astype(np.float64)
    lev, bnd, _, _ = oracle_mod.lloyd_max16()
    cells = np.diff(scipy.stats.norm.cdf(np.concatenate([[-np.inf], bnd, [np.inf]])))
    done = 0
    while done < 60:
        idx = rng.choice(16, size=256, p=cells / cells.sum())
        yhat = c[idx].astype(np.float64)
        r = np.linalg.norm(yhat)
        if not 0.95 < r < 1.05:
            continue
        s = float(rng.uniform(0.5, 40.0))
        x = (s * (H @ yhat) / 16.0).astype(np.float32)
        words, norms = oracle_mod.encode(x[None])
        np.testing.assert_array_equal(oracle_mod.unpack(words)[0], idx)
        nr = oracle_mod.f16_bits_to_f64(norms)[0]
        assert abs(nr - s * r) <= s * r * 2.0 ** -10
        done += 1


def test_reconstruction_mse_matches_quantiser_distortion(oracle_mod):
    """For N(0,1) sources the relative MSE is close to the Lloyd-Max distortion."""
    x = np.random.default_rng(8).standard_normal((3000, 256)).astype(np.float32)
    words, norms = oracle_mod.encode(x)
    xh = oracle_mod.decode(words, norms)
    rel = np.sum((x - xh) ** 2, axis=1) / np.sum(x.astype(np.float64) ** 2, axis=1)
    _, _, dist, _ = oracle_mod.lloyd_max16()
    assert abs(rel.mean() - dist) < 0.04 * dist


# ------------------------------------------------------------- decoder (P7)

def test_decode_is_exact_rational(oracle_mod):
    rng = np.random.default_rng(9)
    c, _ = oracle_mod.codebook()
    cF = [Fraction(float(v)) for v in c]
    H = scipy.linalg.hadamard(256)
    words = rng.integers(0, 2 ** 32, (6, 32), dtype=np.uint64).astype(np.uint32)
    norms = rng.integers(0, 0x7bff, 6).astype(np.uint16)
    got = oracle_mod.decode(words, norms)
    idx = oracle_mod.unpack(words)
    for v in range(6):
        n = Fraction(float(np.uint16(norms[v]).view(np.float16)))
        ys = [cF[i] for i in idx[v]]
        for d in (0, 1, 37, 128, 255):
            exact = n * sum(int(H[d, j]) * ys[j] for j in range(256)) / 16
            assert Fraction(float(got[v, d])) == exact
