/*
 * tq4_oracle.c -- plain, slow CPU oracle for the TQ4 KV codec and for
 * attention over a paged TQ4 KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no
 * code, header, table or constant generator with the GPU library, and it never
 * takes an input produced by the GPU library.
 *
 * Sources (cited by page title and section; no other source is used):
 *   [KVX]  "Fitting a 27B-Parameter LLM into 24 GiB of Laptop Memory"
 *          (simpleprog.com article on the JustFit preprint), section
 *          "KVExec: Fused Reconstruction with Layer-Scoped Lifetime":
 *          a vector is stored as 32 U32 words, eight indices per word, plus
 *          one FP16 norm; reconstruction = packed page IDs -> centroid lookup
 *          -> inverse Hadamard rotation -> norm restore, consumed at once by
 *          scaled dot-product attention.
 *   [MBE]  same page, section "The Memory Budget Equation": four KV heads of
 *          dimension 256 per full-attention layer, 16 such layers.
 *   [P5]   "JustFit: Run Qwen 27B Fast with its full 256K context on a 24 GB
 *          Mac" (wpnews.pro), mechanism table, KVExec row: attention in the
 *          rotated domain.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   R1  nibble order: dim 8k+j sits in bits 4j..4j+3 of word k (LSB first);
 *       words ascend with dims.
 *   R2  index i maps to the i-th smallest centroid (ascending).
 *   R3  the 16 centroids are the Lloyd-Max levels of N(0,1) divided by 16
 *       (i.e. the levels for N(0,1/256), the law of one coordinate of a
 *       rotated unit vector in 256 dims), rounded to fp32.
 *   R4  the rotation is the natural-order Sylvester Hadamard matrix H scaled
 *       by 1/16 (orthonormal, symmetric, its own inverse).
 *   R5  the stored norm is ||x||_2 of the source vector; the rotated unit
 *       vector z = (H x / 16) / ||x|| is what is quantised.
 *   R6  encoder arithmetic is fp32 with round-to-nearest-even and no fused
 *       multiply-add: squares summed by the stride-halving tree
 *       (128, 64, ..., 1); correctly rounded sqrt; FWHT butterflies in
 *       ascending stage order h = 1, 2, ..., 128 mapping (a, b) -> (a+b, a-b);
 *       thresholds t_i = b_i * (16 * n) with b_i the fp32 midpoint of
 *       adjacent centroids; idx = #{ i : y > t_i } (a tie goes low).
 *   R7  GQA: query head h reads KV head h / (n_q_heads / n_kv_heads).
 *   R8  position p of a request lives in page page_table[p / P] at in-page
 *       offset p % P.
 *
 * Decode (tq4o_decode_vec) is exact in fp64: every centroid is a multiple of
 * 2^-30 below 2^-2, so a signed sum of 256 of them needs < 37 bits and the
 * product with an 11-bit fp16 norm < 48 bits.  Attention accumulates in fp64.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define TQ4O_DIM 256
#define TQ4O_WORDS 32
#define TQ4O_LEVELS 16

/* ------------------------------------------------------------------------ */
/* Lloyd-Max quantiser for N(0,1), 16 levels (R3).                          */
/* ------------------------------------------------------------------------ */

static double std_pdf(double x) {
    if (isinf(x)) return 0.0;
    return exp(-0.5 * x * x) / sqrt(2.0 * M_PI);
}

/* Upper tail Q(x) = P(X > x). */
static double upper_tail(double x) {
    if (x == INFINITY) return 0.0;
    if (x == -INFINITY) return 1.0;
    return 0.5 * erfc(x / sqrt(2.0));
}

/* P(a < X < b), evaluated on the side that avoids cancellation. */
static double cell_mass(double a, double b) {
    if (a >= 0.0) return upper_tail(a) - upper_tail(b);
    if (b <= 0.0) return upper_tail(-b) - upper_tail(-a);
    return 1.0 - upper_tail(b) - upper_tail(-a);
}

/* E[X ; a < X < b] = pdf(a) - pdf(b). */
static double cell_first_moment(double a, double b) {
    return std_pdf(a) - std_pdf(b);
}

/* E[X^2 ; a < X < b] = mass + a pdf(a) - b pdf(b). */
static double cell_second_moment(double a, double b) {
    double ta = isinf(a) ? 0.0 : a * std_pdf(a);
    double tb = isinf(b) ? 0.0 : b * std_pdf(b);
    return cell_mass(a, b) + ta - tb;
}

/*
 * Lloyd's fixed-point iteration: boundaries are midpoints of adjacent levels,
 * levels are the conditional means of their cells.  Returns the number of
 * iterations, or -1 if it did not settle below 1e-15 within max_iter.
 * distortion = E[(X - Q(X))^2].
 */
int tq4o_lloyd_max16(double levels[TQ4O_LEVELS], double bounds[TQ4O_LEVELS - 1],
                     double *distortion, int max_iter) {
    double lev[TQ4O_LEVELS], bnd[TQ4O_LEVELS - 1];
    for (int i = 0; i < TQ4O_LEVELS; ++i)
        lev[i] = -3.0 + 6.0 * (i + 0.5) / TQ4O_LEVELS;
    int it = 0;
    for (; it < max_iter; ++it) {
        for (int i = 0; i < TQ4O_LEVELS - 1; ++i) bnd[i] = 0.5 * (lev[i] + lev[i + 1]);
        double delta = 0.0;
        for (int i = 0; i < TQ4O_LEVELS; ++i) {
            double a = i == 0 ? -INFINITY : bnd[i - 1];
            double b = i == TQ4O_LEVELS - 1 ? INFINITY : bnd[i];
            double nl = cell_first_moment(a, b) / cell_mass(a, b);
            double d = fabs(nl - lev[i]);
            if (d > delta) delta = d;
            lev[i] = nl;
        }
        if (delta < 1e-15) { ++it; break; }
    }
    for (int i = 0; i < TQ4O_LEVELS - 1; ++i) bnd[i] = 0.5 * (lev[i] + lev[i + 1]);
    double dist = 0.0;
    for (int i = 0; i < TQ4O_LEVELS; ++i) {
        double a = i == 0 ? -INFINITY : bnd[i - 1];
        double b = i == TQ4O_LEVELS - 1 ? INFINITY : bnd[i];
        /* E[(X - l)^2 ; cell] = E[X^2] - 2 l E[X] + l^2 P */
        dist += cell_second_moment(a, b) - 2.0 * lev[i] * cell_first_moment(a, b) +
                lev[i] * lev[i] * cell_mass(a, b);
    }
    memcpy(levels, lev, sizeof lev);
    memcpy(bounds, bnd, sizeof bnd);
    if (distortion) *distortion = dist;
    return it < max_iter ? it : -1;
}

/* The fp32 codebook c[16] and the fp32 decision thresholds b[15] (R3, R6). */
static float g_c[TQ4O_LEVELS];
static float g_b[TQ4O_LEVELS - 1];
static int g_ready = 0;

static void ensure_codebook(void) {
    if (g_ready) return;
    double lev[TQ4O_LEVELS], bnd[TQ4O_LEVELS - 1], dist;
    tq4o_lloyd_max16(lev, bnd, &dist, 1000000);
    for (int i = 0; i < TQ4O_LEVELS; ++i) g_c[i] = (float)(lev[i] / 16.0);
    for (int i = 0; i < TQ4O_LEVELS - 1; ++i)
        g_b[i] = (float)(((double)g_c[i] + (double)g_c[i + 1]) / 2.0);
    g_ready = 1;
}

void tq4o_codebook(float c[TQ4O_LEVELS], float b[TQ4O_LEVELS - 1]) {
    ensure_codebook();
    memcpy(c, g_c, sizeof g_c);
    memcpy(b, g_b, sizeof g_b);
}

/* ------------------------------------------------------------------------ */
/* IEEE binary16 conversions, written from the format definition.           */
/* ------------------------------------------------------------------------ */

/* fp32 -> fp16, round to nearest, ties to even. */
uint16_t tq4o_f32_to_f16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t sign = (u >> 16) & 0x8000u;
    uint32_t exp = (u >> 23) & 0xffu;
    uint32_t man = u & 0x7fffffu;
    if (exp == 0xffu) /* inf or nan */
        return (uint16_t)(sign | 0x7c00u | (man ? 0x200u | (man >> 13) : 0u));
    int e = (int)exp - 127 + 15; /* biased fp16 exponent */
    if (e >= 31) return (uint16_t)(sign | 0x7c00u);
    if (e <= 0) {
        /* subnormal half (or zero): value = m * 2^-24 */
        if (e < -10) return (uint16_t)sign; /* below half of the smallest subnormal */
        uint32_t m = man | 0x800000u;      /* 24-bit significand */
        int shift = 14 - e;                /* bits dropped: 1 - e + 13 */
        uint32_t q = m >> shift;
        uint32_t rem = m & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1);
        if (rem > half || (rem == half && (q & 1u))) ++q;
        return (uint16_t)(sign | q);
    }
    uint32_t q = ((uint32_t)e << 10) | (man >> 13);
    uint32_t rem = man & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) ++q; /* may carry into the exponent */
    return (uint16_t)(sign | q);
}

double tq4o_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (exp == 0) v = ldexp((double)man, -24);
    else if (exp == 31) v = man ? NAN : INFINITY;
    else v = ldexp((double)(man | 0x400), exp - 25);
    return sign ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Hadamard rotation (R4).                                                  */
/* ------------------------------------------------------------------------ */

/* Unnormalised fast Walsh-Hadamard transform in fp32, stages h = 1 .. 128. */
void tq4o_fwht_f32(float *x) {
    for (int h = 1; h < TQ4O_DIM; h <<= 1)
        for (int i = 0; i < TQ4O_DIM; ++i)
            if ((i & h) == 0) {
                float a = x[i], b = x[i + h];
                x[i] = a + b;
                x[i + h] = a - b;
            }
}

/* Same transform in fp64. */
void tq4o_fwht_f64(double *x) {
    for (int h = 1; h < TQ4O_DIM; h <<= 1)
        for (int i = 0; i < TQ4O_DIM; ++i)
            if ((i & h) == 0) {
                double a = x[i], b = x[i + h];
                x[i] = a + b;
                x[i + h] = a - b;
            }
}

/* ------------------------------------------------------------------------ */
/* Encode one vector (R1..R6).                                              */
/* ------------------------------------------------------------------------ */

void tq4o_encode_vec(const float *x, uint32_t *words, uint16_t *norm16) {
    ensure_codebook();
    /* squared norm by the stride-halving tree */
    float s[TQ4O_DIM];
    for (int d = 0; d < TQ4O_DIM; ++d) s[d] = x[d] * x[d];
    for (int stride = TQ4O_DIM / 2; stride >= 1; stride >>= 1)
        for (int i = 0; i < stride; ++i) s[i] = s[i] + s[i + stride];
    float n32 = sqrtf(s[0]); /* IEEE sqrt is correctly rounded */
    *norm16 = tq4o_f32_to_f16(n32);

    /* rotate: y = H x (unnormalised) */
    float y[TQ4O_DIM];
    memcpy(y, x, sizeof y);
    tq4o_fwht_f32(y);

    /* the unit rotated coordinate is y / (16 n); compare y against the
       thresholds scaled by 16 n instead of dividing */
    float m = 16.0f * n32;
    float t[TQ4O_LEVELS - 1];
    for (int i = 0; i < TQ4O_LEVELS - 1; ++i) t[i] = g_b[i] * m;

    memset(words, 0, TQ4O_WORDS * sizeof(uint32_t));
    for (int d = 0; d < TQ4O_DIM; ++d) {
        uint32_t idx = 0;
        for (int i = 0; i < TQ4O_LEVELS - 1; ++i)
            if (y[d] > t[i]) ++idx;
        words[d / 8] |= idx << (4 * (d % 8));
    }
}

/* Unpack the 256 indices of one record (R1). */
void tq4o_unpack(const uint32_t *words, uint8_t *idx) {
    for (int d = 0; d < TQ4O_DIM; ++d) idx[d] = (uint8_t)((words[d / 8] >> (4 * (d % 8))) & 0xfu);
}

/* Pack 256 indices (each < 16) into 32 words (R1). */
void tq4o_pack(const uint8_t *idx, uint32_t *words) {
    memset(words, 0, TQ4O_WORDS * sizeof(uint32_t));
    for (int d = 0; d < TQ4O_DIM; ++d) words[d / 8] |= (uint32_t)(idx[d] & 0xfu) << (4 * (d % 8));
}

/* ------------------------------------------------------------------------ */
/* Decode one vector, exact in fp64: x = n * H c[idx] / 16.                 */
/* ------------------------------------------------------------------------ */

void tq4o_decode_vec(const uint32_t *words, uint16_t norm16, double *out) {
    ensure_codebook();
    uint8_t idx[TQ4O_DIM];
    tq4o_unpack(words, idx);
    for (int d = 0; d < TQ4O_DIM; ++d) out[d] = (double)g_c[idx[d]];
    tq4o_fwht_f64(out);
    double n = tq4o_f16_to_f64(norm16);
    for (int d = 0; d < TQ4O_DIM; ++d) out[d] = n * out[d] / 16.0;
}

/* ------------------------------------------------------------------------ */
/* Pool-level helpers.                                                      */
/*                                                                          */
/* One layer's pool: words [num_pages][n_kv][P][32] (u32) and norms         */
/* [num_pages][n_kv][P] (fp16 bits), separately for K and for V.  A slot is */
/* page_id * P + offset.                                                    */
/* ------------------------------------------------------------------------ */

static size_t rec_index(int32_t page, int32_t head, int32_t off, int32_t n_kv, int32_t P) {
    return ((size_t)page * (size_t)n_kv + (size_t)head) * (size_t)P + (size_t)off;
}

/*
 * Encode n_tokens source vectors src[n_tokens][n_kv][256] (fp32) into the
 * records at slots[t].  Returns 0, or -1 on a slot outside the pool.
 */
int tq4o_encode_to_pool(uint32_t *words, uint16_t *norms, int32_t num_pages, int32_t n_kv,
                        int32_t P, const float *src, const int32_t *slots, int32_t n_tokens) {
    for (int32_t t = 0; t < n_tokens; ++t) {
        int32_t slot = slots[t];
        if (slot < 0 || slot >= num_pages * P) return -1;
        int32_t page = slot / P, off = slot % P;
        for (int32_t g = 0; g < n_kv; ++g) {
            size_t r = rec_index(page, g, off, n_kv, P);
            tq4o_encode_vec(src + ((size_t)t * n_kv + g) * TQ4O_DIM, words + r * TQ4O_WORDS,
                            norms + r);
        }
    }
    return 0;
}

/*
 * Scaled dot-product attention over TQ4 pages, fp64 throughout.
 *
 * For each row r (one query token) and each query head h in [h_begin, h_end):
 *   keys j = 0 .. row_len[r]-1 of page-table row row_table[r];
 *   s_j = scale * <q[r][h], k_j>;  p = softmax(s);  out = sum_j p_j v_j.
 * q is [n_rows][n_q][256] in fp64 (exact copies of the bf16 inputs); out is
 * [n_rows][n_q][256] fp64 (only heads in the range are written).
 * Decode is the case row = request, row_len = seq_len; a prefill chunk row t
 * at absolute position P0 + t has row_len = P0 + t + 1 (causal).
 * Returns 0, or -1 on a malformed page table entry.
 */
int tq4o_attention(const uint32_t *k_words, const uint16_t *k_norms, const uint32_t *v_words,
                   const uint16_t *v_norms, int32_t num_pages, int32_t n_kv, int32_t P,
                   const double *q, int32_t n_q, int32_t n_rows, const int32_t *page_table,
                   int32_t table_stride, const int32_t *row_table, const int32_t *row_len,
                   double scale, int32_t h_begin, int32_t h_end, double *out) {
    int32_t group = n_q / n_kv;
    double kv[TQ4O_DIM];
    for (int32_t r = 0; r < n_rows; ++r) {
        int32_t L = row_len[r];
        const int32_t *table = page_table + (size_t)row_table[r] * table_stride;
        for (int32_t g = 0; g < n_kv; ++g) {
            int32_t h0 = g * group, h1 = h0 + group;
            if (h0 < h_begin) h0 = h_begin;
            if (h1 > h_end) h1 = h_end;
            if (h0 >= h1) continue;
            int32_t nh = h1 - h0;
            double *s = (double *)malloc((size_t)L * nh * sizeof(double));
            if (!s) return -2;
            /* scores */
            for (int32_t j = 0; j < L; ++j) {
                int32_t page = table[j / P];
                if (page < 0 || page >= num_pages) { free(s); return -1; }
                size_t rec = rec_index(page, g, j % P, n_kv, P);
                tq4o_decode_vec(k_words + rec * TQ4O_WORDS, k_norms[rec], kv);
                for (int32_t hh = 0; hh < nh; ++hh) {
                    const double *qh = q + ((size_t)r * n_q + h0 + hh) * TQ4O_DIM;
                    double dot = 0.0;
                    for (int d = 0; d < TQ4O_DIM; ++d) dot += qh[d] * kv[d];
                    s[(size_t)hh * L + j] = scale * dot;
                }
            }
            /* softmax weights (max subtracted) */
            for (int32_t hh = 0; hh < nh; ++hh) {
                double *sh = s + (size_t)hh * L;
                double mx = -INFINITY;
                for (int32_t j = 0; j < L; ++j) if (sh[j] > mx) mx = sh[j];
                double sum = 0.0;
                for (int32_t j = 0; j < L; ++j) { sh[j] = exp(sh[j] - mx); sum += sh[j]; }
                for (int32_t j = 0; j < L; ++j) sh[j] /= sum;
                double *oh = out + ((size_t)r * n_q + h0 + hh) * TQ4O_DIM;
                for (int d = 0; d < TQ4O_DIM; ++d) oh[d] = 0.0;
            }
            /* weighted sum of values */
            for (int32_t j = 0; j < L; ++j) {
                int32_t page = table[j / P];
                size_t rec = rec_index(page, g, j % P, n_kv, P);
                tq4o_decode_vec(v_words + rec * TQ4O_WORDS, v_norms[rec], kv);
                for (int32_t hh = 0; hh < nh; ++hh) {
                    double p = s[(size_t)hh * L + j];
                    double *oh = out + ((size_t)r * n_q + h0 + hh) * TQ4O_DIM;
                    for (int d = 0; d < TQ4O_DIM; ++d) oh[d] += p * kv[d];
                }
            }
            free(s);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Unfused path: reconstruct K/V into the query dtype, then dense attention. */
/* ------------------------------------------------------------------------ */

/*
 * fp64 -> bf16 bits, round to nearest, ties to even, taken in one step from the
 * fp64 value (no intermediate fp32 rounding).  bf16 keeps 8 significant bits and
 * fp32's exponent range; below 2^-126 its spacing is 2^-133.  Values whose
 * magnitude rounds to 2^128 or more become infinity.  NaN maps to a quiet NaN.
 */
uint16_t tq4o_f64_to_bf16(double x) {
    if (isnan(x)) return 0x7fc0;
    const int neg = signbit(x) ? 1 : 0;
    double a = fabs(x);
    uint16_t sign = (uint16_t)(neg << 15);
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);                     /* a = m 2^e, m in [0.5, 1) */
    int qexp = e - 8;                 /* spacing of 8-bit significands in [2^(e-1), 2^e) */
    if (qexp < -133) qexp = -133;     /* subnormal spacing */
    const double r = rint(ldexp(a, -qexp));   /* exact scaling; rint rounds half to even */
    const double v = ldexp(r, qexp);
    if (v >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7f80);
    const float f = (float)v;         /* exact: v has at most 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, 4);
    return (uint16_t)(sign | ((bits >> 16) & 0x7fff));
}

/*
 * Reconstruction into contiguous K/V ([KVX]: multi-query prefill can reconstruct
 * the pages into contiguous tensors of the query dtype, and a gather-and-SDPA
 * path is the fallback).  For request b, KV head g and position p < L_b
 * (L_b = seq_lens[b] clamped to [0, max_seq]): out[b][g][p][:] = bf16(decode of
 * the record at page_table[b][p / P], offset p % P).  Positions p >= L_b are not
 * written.  Outputs are bf16 bits [batch][n_kv][max_seq][256].  Returns 0, or -1
 * on a page ID outside the pool.
 */
int tq4o_reconstruct(const uint32_t *k_words, const uint16_t *k_norms, const uint32_t *v_words,
                     const uint16_t *v_norms, int32_t num_pages, int32_t n_kv, int32_t P,
                     const int32_t *page_table, int32_t table_stride, const int32_t *seq_lens,
                     int32_t batch, int32_t max_seq, uint16_t *k_out, uint16_t *v_out) {
    double x[TQ4O_DIM];
    for (int32_t b = 0; b < batch; ++b) {
        int32_t L = seq_lens[b];
        if (L < 0) L = 0;
        if (L > max_seq) L = max_seq;
        for (int32_t g = 0; g < n_kv; ++g) {
            for (int32_t p = 0; p < L; ++p) {
                const int32_t page = page_table[(size_t)b * table_stride + p / P];
                if (page < 0 || page >= num_pages) return -1;
                const size_t rec = rec_index(page, g, p % P, n_kv, P);
                const size_t o = (((size_t)b * n_kv + g) * max_seq + p) * TQ4O_DIM;
                tq4o_decode_vec(k_words + rec * TQ4O_WORDS, k_norms[rec], x);
                for (int d = 0; d < TQ4O_DIM; ++d) k_out[o + d] = tq4o_f64_to_bf16(x[d]);
                tq4o_decode_vec(v_words + rec * TQ4O_WORDS, v_norms[rec], x);
                for (int d = 0; d < TQ4O_DIM; ++d) v_out[o + d] = tq4o_f64_to_bf16(x[d]);
            }
        }
    }
    return 0;
}

/*
 * Dense scaled dot-product attention for one query per request over contiguous
 * K/V in fp64: q [batch][n_q][256], k and v [batch][n_kv][max_seq][256], keys
 * 0 .. L_b - 1 (L_b = seq_lens[b] clamped to [0, max_seq]); query head h reads
 * KV head h / (n_q / n_kv).  out [batch][n_q][256]; a request with L_b = 0 gets
 * zeros.  Returns 0, or -2 when memory runs out.
 */
int tq4o_sdpa_dense(const double *q, const double *k, const double *v, int32_t batch, int32_t n_q,
                    int32_t n_kv, int32_t max_seq, const int32_t *seq_lens, double scale, double *out) {
    const int32_t group = n_q / n_kv;
    double *s = (double *)malloc((size_t)(max_seq > 0 ? max_seq : 1) * sizeof(double));
    if (!s) return -2;
    for (int32_t b = 0; b < batch; ++b) {
        int32_t L = seq_lens[b];
        if (L < 0) L = 0;
        if (L > max_seq) L = max_seq;
        for (int32_t h = 0; h < n_q; ++h) {
            const int32_t g = h / group;
            const double *qh = q + ((size_t)b * n_q + h) * TQ4O_DIM;
            const double *kb = k + ((size_t)b * n_kv + g) * max_seq * TQ4O_DIM;
            const double *vb = v + ((size_t)b * n_kv + g) * max_seq * TQ4O_DIM;
            double *oh = out + ((size_t)b * n_q + h) * TQ4O_DIM;
            for (int d = 0; d < TQ4O_DIM; ++d) oh[d] = 0.0;
            if (L == 0) continue;
            double mx = -INFINITY;
            for (int32_t j = 0; j < L; ++j) {
                double dot = 0.0;
                for (int d = 0; d < TQ4O_DIM; ++d) dot += qh[d] * kb[(size_t)j * TQ4O_DIM + d];
                s[j] = scale * dot;
                if (s[j] > mx) mx = s[j];
            }
            double sum = 0.0;
            for (int32_t j = 0; j < L; ++j) { s[j] = exp(s[j] - mx); sum += s[j]; }
            for (int32_t j = 0; j < L; ++j) {
                const double pj = s[j] / sum;
                for (int d = 0; d < TQ4O_DIM; ++d) oh[d] += pj * vb[(size_t)j * TQ4O_DIM + d];
            }
        }
    }
    free(s);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Uniform INT8 arm ("Fitting a 27B-Parameter LLM into 24 GiB of Laptop       */
/* Memory", section "Reasoning at 200K: 29 of 30 AIME Problems": a uniform    */
/* INT8 KV comparison).  Readings: one symmetric scale per vector, stored as  */
/* fp16 like the TQ4 norm, codes in [-127, 127], no rotation.                 */
/* ------------------------------------------------------------------------ */

/*
 * Encode, fp32 with round-to-nearest-even throughout:
 *   a = max_d |x_d|;  s16 = fp16(a / 127);  s = (float) s16;
 *   q_d = clamp(rint(x_d / s), -127, 127), or 0 for every d when s == 0.
 */
void tq4o_int8_encode_vec(const float *x, int8_t *codes, uint16_t *scale16) {
    float a = 0.0f;
    for (int d = 0; d < TQ4O_DIM; ++d) {
        const float v = fabsf(x[d]);
        if (v > a) a = v;
    }
    const float s32 = a / 127.0f;
    const uint16_t s16 = tq4o_f32_to_f16(s32);
    const float s = (float)tq4o_f16_to_f64(s16);
    *scale16 = s16;
    for (int d = 0; d < TQ4O_DIM; ++d) {
        float q = 0.0f;
        if (s > 0.0f) {
            const float r = x[d] / s;
            q = rintf(r);
            if (q > 127.0f) q = 127.0f;
            if (q < -127.0f) q = -127.0f;
        }
        codes[d] = (int8_t)q;
    }
}

/* Decode: x_d = q_d * s, exact in fp64. */
void tq4o_int8_decode_vec(const int8_t *codes, uint16_t scale16, double *out) {
    const double s = tq4o_f16_to_f64(scale16);
    for (int d = 0; d < TQ4O_DIM; ++d) out[d] = (double)codes[d] * s;
}

void tq4o_int8_encode_many(const float *x, int64_t n, int8_t *codes, uint16_t *scales) {
    for (int64_t i = 0; i < n; ++i) tq4o_int8_encode_vec(x + i * TQ4O_DIM, codes + i * TQ4O_DIM, scales + i);
}

void tq4o_int8_decode_many(const int8_t *codes, const uint16_t *scales, int64_t n, double *out) {
    for (int64_t i = 0; i < n; ++i) tq4o_int8_decode_vec(codes + i * TQ4O_DIM, scales[i], out + i * TQ4O_DIM);
}

/* Encode K or V sources [n][n_kv][256] into the INT8 pool at flat slots (page * P + offset). */
int tq4o_int8_encode_to_pool(int8_t *codes, uint16_t *scales, int32_t num_pages, int32_t n_kv, int32_t P,
                             const float *src, const int32_t *slots, int32_t n) {
    for (int32_t i = 0; i < n; ++i) {
        const int32_t slot = slots[i];
        if (slot < 0 || slot >= num_pages * P) return -1;
        for (int32_t g = 0; g < n_kv; ++g) {
            const size_t rec = rec_index(slot / P, g, slot % P, n_kv, P);
            tq4o_int8_encode_vec(src + ((size_t)i * n_kv + g) * TQ4O_DIM, codes + rec * TQ4O_DIM, scales + rec);
        }
    }
    return 0;
}

/*
 * fp64 softmax attention over INT8 pages: the same definition as tq4o_attention with each key and
 * value taken as its exact INT8 decode (codes times scale, natural domain).
 */
int tq4o_int8_attention(const int8_t *k_codes, const uint16_t *k_scales, const int8_t *v_codes,
                        const uint16_t *v_scales, int32_t num_pages, int32_t n_kv, int32_t P,
                        const double *q, int32_t n_q, int32_t n_rows, const int32_t *page_table,
                        int32_t table_stride, const int32_t *row_table, const int32_t *row_len,
                        double scale, int32_t h_begin, int32_t h_end, double *out) {
    int32_t group = n_q / n_kv;
    double kv[TQ4O_DIM];
    for (int32_t r = 0; r < n_rows; ++r) {
        int32_t L = row_len[r];
        const int32_t *table = page_table + (size_t)row_table[r] * table_stride;
        for (int32_t g = 0; g < n_kv; ++g) {
            int32_t h0 = g * group, h1 = h0 + group;
            if (h0 < h_begin) h0 = h_begin;
            if (h1 > h_end) h1 = h_end;
            if (h0 >= h1) continue;
            int32_t nh = h1 - h0;
            for (int32_t hh = 0; hh < nh; ++hh) {
                double *oh = out + ((size_t)r * n_q + h0 + hh) * TQ4O_DIM;
                for (int d = 0; d < TQ4O_DIM; ++d) oh[d] = 0.0;
            }
            if (L <= 0) continue;
            double *s = (double *)malloc((size_t)L * nh * sizeof(double));
            if (!s) return -2;
            for (int32_t j = 0; j < L; ++j) {
                int32_t page = table[j / P];
                if (page < 0 || page >= num_pages) { free(s); return -1; }
                size_t rec = rec_index(page, g, j % P, n_kv, P);
                tq4o_int8_decode_vec(k_codes + rec * TQ4O_DIM, k_scales[rec], kv);
                for (int32_t hh = 0; hh < nh; ++hh) {
                    const double *qh = q + ((size_t)r * n_q + h0 + hh) * TQ4O_DIM;
                    double dot = 0.0;
                    for (int d = 0; d < TQ4O_DIM; ++d) dot += qh[d] * kv[d];
                    s[(size_t)hh * L + j] = scale * dot;
                }
            }
            for (int32_t hh = 0; hh < nh; ++hh) {
                double *sh = s + (size_t)hh * L;
                double mx = -INFINITY;
                for (int32_t j = 0; j < L; ++j) if (sh[j] > mx) mx = sh[j];
                double sum = 0.0;
                for (int32_t j = 0; j < L; ++j) { sh[j] = exp(sh[j] - mx); sum += sh[j]; }
                for (int32_t j = 0; j < L; ++j) sh[j] /= sum;
            }
            for (int32_t j = 0; j < L; ++j) {
                int32_t page = table[j / P];
                size_t rec = rec_index(page, g, j % P, n_kv, P);
                tq4o_int8_decode_vec(v_codes + rec * TQ4O_DIM, v_scales[rec], kv);
                for (int32_t hh = 0; hh < nh; ++hh) {
                    double p = s[(size_t)hh * L + j];
                    double *oh = out + ((size_t)r * n_q + h0 + hh) * TQ4O_DIM;
                    for (int d = 0; d < TQ4O_DIM; ++d) oh[d] += p * kv[d];
                }
            }
            free(s);
        }
    }
    return 0;
}

void tq4o_f64_to_bf16_array(const double *in, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = tq4o_f64_to_bf16(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Array conveniences for the Python wrapper (loops over the above).        */
/* ------------------------------------------------------------------------ */

void tq4o_f32_to_f16_array(const float *in, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = tq4o_f32_to_f16(in[i]);
}

void tq4o_encode_many(const float *x, int64_t n, uint32_t *words, uint16_t *norms) {
    for (int64_t i = 0; i < n; ++i)
        tq4o_encode_vec(x + i * TQ4O_DIM, words + i * TQ4O_WORDS, norms + i);
}

void tq4o_decode_many(const uint32_t *words, const uint16_t *norms, int64_t n, double *out) {
    for (int64_t i = 0; i < n; ++i)
        tq4o_decode_vec(words + i * TQ4O_WORDS, norms[i], out + i * TQ4O_DIM);
}

void tq4o_fwht_f32_many(float *x, int64_t n) {
    for (int64_t i = 0; i < n; ++i) tq4o_fwht_f32(x + i * TQ4O_DIM);
}

void tq4o_fwht_f64_many(double *x, int64_t n) {
    for (int64_t i = 0; i < n; ++i) tq4o_fwht_f64(x + i * TQ4O_DIM);
}
