/*
 * tq4.h -- C ABI of the TQ4 paged-KV attention library for AMD Instinct
 * MI355X (gfx950).
 *
 * What the library computes (sources cited by page title and section):
 *
 *   [KVX] "Fitting a 27B-Parameter LLM into 24 GiB of Laptop Memory"
 *         (simpleprog.com article on the JustFit preprint), section
 *         "KVExec: Fused Reconstruction with Layer-Scoped Lifetime".
 *         Each cached key or value vector is one TQ4 record: 32 u32 words,
 *         eight 4-bit centroid indices per word (256 dims), plus one fp16
 *         norm.  Attention reads packed page IDs, looks the indices up in a
 *         16-entry centroid table, undoes the Hadamard rotation, restores the
 *         norm and feeds scaled dot-product attention at once; the attention
 *         result is complete before the call's work ends, and no
 *         full-precision K/V is ever written to memory.  Single-query decode
 *         works on the compressed pages directly; multi-query prefill
 *         reconstructs tiles and runs a floating-point attention consumer.
 *   [MBE] same page, section "The Memory Budget Equation": 4 KV heads of
 *         dimension 256 per full-attention layer.
 *   [ST]  same page, section "StateTrans: Request Transitions at Safe
 *         Boundaries": 256-token pages, page IDs shared between requests with
 *         a common prefix.
 *   [AIME] same page, section "Reasoning at 200K: 29 of 30 AIME Problems":
 *         a uniform INT8 KV cache as the comparison arm.
 *   [P5]  "JustFit: Run Qwen 27B Fast with its full 256K context on a 24 GB
 *         Mac" (wpnews.pro), mechanism table, KVExec row: bounded
 *         reconstruction and attention in the rotated domain.
 *
 * Codec conventions the pages leave open (the library and its tests use these):
 *   - dim 8k+j of a vector is held in bits 4j..4j+3 of word k;
 *   - index i selects the i-th smallest of 16 fp32 centroids, which are the
 *     16-level Lloyd-Max levels of N(0,1) divided by 16;
 *   - the rotation is H/16 with H the natural-order Sylvester Hadamard matrix
 *     of order 256 (symmetric and orthonormal, so it is its own inverse);
 *   - the norm is ||x||_2 of the source vector, rounded to fp16; the rotated
 *     unit vector H x / (16 ||x||) is what is quantised;
 *   - encoding is fp32, round-to-nearest-even, no fused multiply-add: squares
 *     summed by the stride-halving tree (128, 64, ..., 1), correctly rounded
 *     sqrt, Hadamard butterflies (a, b) -> (a + b, a - b) in ascending stage
 *     order 1, 2, ..., 128, index = number of thresholds t_i = b_i * (16 n)
 *     strictly below the rotated coordinate, b_i the fp32 midpoints of
 *     adjacent centroids.
 *   - query head h reads KV head h / (n_q_heads / n_kv_heads).
 *
 * Memory layout of one layer's pool (all device memory, caller-owned):
 *   k_words, v_words : uint32 [num_pages][n_kv_heads][page_size][32]
 *   k_norms, v_norms : fp16 bits [num_pages][n_kv_heads][page_size]
 * A slot is page_id * page_size + offset.  Position p of a request lives in
 * page page_table[p / page_size] at offset p % page_size.  One page ID names
 * the same slot range in every layer's pool.
 *
 * Conventions for every entry point:
 *   - Ownership: the caller owns every buffer; the library never allocates,
 *     frees or synchronises, and keeps no mutable global state.
 *   - Streams: `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued asynchronously; calls are thread-safe.  Calls that share a
 *     workspace must be ordered on one stream.
 *   - Errors: every argument check happens on the host before any HIP call,
 *     so a non-OK status means nothing was enqueued (except TQ4_ERR_HIP,
 *     which reports a failed launch).  No exception or abort crosses the ABI.
 *   - Device data (page tables, sequence lengths, slots) is not read on the
 *     host.  A sequence length is clamped to [0, max]; a page ID or slot
 *     outside the pool is skipped (its positions are masked, its record is
 *     not written), so bad device data never makes the library touch memory
 *     outside the buffers described here.
 */
#ifndef TQ4_H
#define TQ4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ4_ABI_VERSION 1
#define TQ4_HEAD_DIM 256
#define TQ4_WORDS_PER_VECTOR 32
#define TQ4_NUM_CENTROIDS 16
#define TQ4_MAX_GROUP 16 /* largest n_q_heads / n_kv_heads */
#define TQ4_MAX_VERIFY_ROWS 48 /* largest n_queries * n_q_heads / n_kv_heads of tq4_attn_verify */

typedef enum tq4_status {
    TQ4_OK = 0,
    TQ4_ERR_NULL = 1,      /* a required pointer is NULL */
    TQ4_ERR_SHAPE = 2,     /* a size is out of range or inconsistent */
    TQ4_ERR_DTYPE = 3,     /* unsupported element type */
    TQ4_ERR_ALIGN = 4,     /* a pointer is not aligned as documented */
    TQ4_ERR_WORKSPACE = 5, /* workspace missing or smaller than required */
    TQ4_ERR_HIP = 6,       /* the HIP runtime reported an error */
    TQ4_ERR_CAPACITY = 7,  /* not enough free pages (or host memory) for the request */
    TQ4_ERR_VALUE = 8      /* a scalar argument is outside its documented range */
} tq4_status;

typedef enum tq4_dtype {
    TQ4_F32 = 0,
    TQ4_BF16 = 1,
    TQ4_F16 = 2
} tq4_dtype;

/* One layer's page pool.  Words need 16-byte alignment, norms 8-byte.
 * Limits: head_dim == 256; page_size a multiple of 32 in [32, 1024];
 * num_pages >= 1; n_kv_heads >= 1; num_pages * n_kv_heads * page_size < 2^31. */
typedef struct tq4_layer_pool {
    uint32_t *k_words;
    uint32_t *v_words;
    uint16_t *k_norms;
    uint16_t *v_norms;
    int32_t num_pages;
    int32_t page_size;
    int32_t n_kv_heads;
    int32_t head_dim;
} tq4_layer_pool;

/* TQ4_ABI_VERSION of the loaded library. */
int tq4_abi_version(void);

/* Static description of a status code (never NULL). */
const char *tq4_status_string(tq4_status status);

/* Host copy of the codec constants: the 16 fp32 centroids in ascending order
 * and the 15 fp32 decision thresholds (midpoints of adjacent centroids).
 * Both pointers are host memory.  Returns TQ4_ERR_NULL on a NULL pointer. */
tq4_status tq4_codebook(float centroids[16], float thresholds[15]);

/*
 * tq4_encode_pages -- write TQ4 records for n_tokens new positions
 * ([KVX]: the cache is kept as TQ4 pages; a position's K and V are encoded
 * when they are written).
 *
 *   k, v      : device, [n_tokens][n_kv_heads][256] in src_dtype (TQ4_F32 or
 *               TQ4_BF16), 16-byte aligned.  Either may be NULL (that half of
 *               the pool is left untouched), not both.
 *   slots     : device int32 [n_tokens]; record t is written at slot slots[t]
 *               of every KV head.  A slot outside [0, num_pages * page_size)
 *               is skipped.  Two tokens with one slot race.
 *   n_tokens  : >= 0 (0 enqueues nothing).
 * The result is bit-identical to the conventions above for every input.
 */
tq4_status tq4_encode_pages(const tq4_layer_pool *pool, const void *k, const void *v,
                            tq4_dtype src_dtype, const int32_t *slots, int32_t n_tokens,
                            void *stream);

/*
 * Bytes of device workspace tq4_attn_decode needs for these sizes (0 for
 * invalid sizes, and 0 when one workgroup covers each request and KV head).
 * It grows with batch and KV heads, not with the sequence length beyond a
 * fixed split cap, so no per-position scratch exists.
 */
size_t tq4_attn_decode_workspace_size(int32_t batch, int32_t max_seq_len, int32_t n_q_heads,
                                      int32_t n_kv_heads, int32_t page_size);

/*
 * tq4_attn_decode -- single-query attention for each request directly on the
 * packed pages ([KVX]; rotated-domain formulation of [P5]).
 *
 *   q         : device [batch][n_q_heads][256], q_dtype == TQ4_BF16, 16-byte
 *               aligned.
 *   page_table: device int32 [batch][page_table_stride].
 *   seq_lens  : device int32 [batch]; cached positions of each request,
 *               including the current token (already encoded).  Clamped to
 *               [0, max_seq_len]; a request with 0 positions gets a zero output.
 *   max_seq_len: host upper bound of seq_lens, 1 <= max_seq_len <=
 *               page_table_stride * page_size; it sets the launch plan.
 *   n_q_heads : a multiple of n_kv_heads with n_q_heads / n_kv_heads <= 16.
 *   batch, n_kv_heads: <= 65535 each (grid dimensions).
 *   scale     : softmax scale applied to q.k (1/16 = 1/sqrt(256) usually);
 *               finite and > 0, else TQ4_ERR_VALUE.
 *   out       : device [batch][n_q_heads][256] in q_dtype, 16-byte aligned;
 *               out[b][h] = sum_j softmax_j(scale q.k_j) v_j.
 *   workspace : device, >= tq4_attn_decode_workspace_size(...) bytes,
 *               256-byte aligned (may be NULL when that size is 0).  It holds
 *               per-split partial results between the call's two kernels; its
 *               contents on entry do not matter.  Calls sharing a workspace
 *               must be ordered on one stream.
 */
tq4_status tq4_attn_decode(const tq4_layer_pool *pool, const void *q, tq4_dtype q_dtype,
                           const int32_t *page_table, int32_t page_table_stride,
                           const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                           int32_t n_q_heads, float scale, void *out, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * tq4_attn_decode_noalloc -- tq4_attn_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same arguments without the workspace, the same
 * kernels and bit-identical results.  The split partials go to a 4 MiB scratch
 * array inside the library's code object; each GPU the library runs on holds
 * its own copy until the process ends.  The scratch holds every plan whose
 * tq4_attn_decode_workspace_size(...) is at most 4 MiB (for example any batch
 * with n_q_heads / n_kv_heads <= 6); larger plans return TQ4_ERR_WORKSPACE
 * before anything is enqueued.  The call uses the current device's scratch (the
 * stream must belong to the current device), calls no allocator, and needs no
 * clearing (its contents on entry do not matter).  Every call on one GPU shares
 * that GPU's scratch: calls that may overlap on one GPU (different streams, or
 * different host threads) race; order them on one stream.
 * Errors: as tq4_attn_decode, plus TQ4_ERR_HIP if the scratch address cannot be
 * obtained on first use on a device.
 */
tq4_status tq4_attn_decode_noalloc(const tq4_layer_pool *pool, const void *q, tq4_dtype q_dtype,
                                   const int32_t *page_table, int32_t page_table_stride,
                                   const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                                   int32_t n_q_heads, float scale, void *out, void *stream);

/*
 * tq4_attn_decode_variant -- tq4_attn_decode computed another way, to measure
 * the design choices of the fused kernel.  Same arguments, workspace size and
 * errors as tq4_attn_decode, plus `variant`:
 *   TQ4_DECODE_FUSED        the fused kernel itself (tq4_attn_decode).
 *   TQ4_DECODE_VALU_ROTATED the same rotated-domain arithmetic ([P5]) on the
 *                           vector ALUs only: fp16 pair dot products with fp32
 *                           accumulation for the scores, fp32 value sums, one
 *                           key per half-wavefront, no matrix cores.
 *   TQ4_DECODE_VALU_LITERAL the reconstruction order of [KVX] taken literally:
 *                           each key and value vector is rebuilt in fp32
 *                           (centroid lookup, inverse Hadamard rotation, norm
 *                           restore) and attention runs in the natural domain.
 * The two VALU variants take n_q_heads / n_kv_heads in {1, 2, 4, 6, 8}
 * (TQ4_ERR_SHAPE otherwise); an unknown variant is TQ4_ERR_VALUE.  Results
 * agree with tq4_attn_decode to the library's attention tolerance, not bit for
 * bit (the arithmetic differs).
 */
typedef enum {
    TQ4_DECODE_FUSED = 0,
    TQ4_DECODE_VALU_ROTATED = 1,
    TQ4_DECODE_VALU_LITERAL = 2
} tq4_decode_variant;

tq4_status tq4_attn_decode_variant(const tq4_layer_pool *pool, const void *q, tq4_dtype q_dtype,
                                   const int32_t *page_table, int32_t page_table_stride,
                                   const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                                   int32_t n_q_heads, float scale, tq4_decode_variant variant, void *out,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * tq4_attn_decode_append -- the decode step of a model layer in one call: encode
 * each request's new token and attend ([KVX]: the cache is written in TQ4 and
 * read back by the attention that follows).  Results are bit-identical to
 * tq4_encode_pages(pool, k_new, v_new, src_dtype, new_slots, batch) followed by
 * tq4_attn_decode(...) with the other arguments, provided new_slots[b] is the
 * slot of position seq_lens[b] - 1 of request b (the new token is the last
 * cached position); a new slot that another position of the call also reads
 * races.
 *
 *   k_new, v_new : device [batch][n_kv_heads][256] in src_dtype (TQ4_F32 or
 *                  TQ4_BF16), 16-byte aligned; either may be NULL, not both.
 *   new_slots    : device int32 [batch]; slots outside the pool are skipped,
 *                  and so is every request whose clamped length is 0.
 *   other arguments as for tq4_attn_decode (seq_lens count the new token).
 */
tq4_status tq4_attn_decode_append(const tq4_layer_pool *pool, const void *k_new, const void *v_new,
                                  tq4_dtype src_dtype, const int32_t *new_slots, const void *q,
                                  tq4_dtype q_dtype, const int32_t *page_table, int32_t page_table_stride,
                                  const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                                  int32_t n_q_heads, float scale, void *out, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace tq4_attn_verify needs for these sizes (0 for
 * invalid sizes, and 0 when one workgroup covers each request and KV head).
 * With n_queries == 1 it equals tq4_attn_decode_workspace_size.
 */
size_t tq4_attn_verify_workspace_size(int32_t batch, int32_t max_seq_len, int32_t n_queries,
                                      int32_t n_q_heads, int32_t n_kv_heads, int32_t page_size);

/*
 * tq4_attn_verify -- packed multi-query attention on the packed pages: the
 * last n_queries positions of each request (speculative draft tokens being
 * verified, or a short chunk) attend causally in one pass over the request's
 * pages ([KVX]: besides direct reconstruction, multi-query prefill has a
 * packed verifier path).  All n_queries x group query rows of one KV head
 * share every page read, so the pages are streamed once, not n_queries times.
 *
 *   q         : device [batch][n_queries][n_q_heads][256], q_dtype ==
 *               TQ4_BF16, 16-byte aligned.
 *   n_queries : >= 1 with n_queries * (n_q_heads / n_kv_heads) <=
 *               TQ4_MAX_VERIFY_ROWS.
 *   seq_lens  : device int32 [batch]; cached positions of each request
 *               including its n_queries query tokens, whose K/V are already
 *               encoded.  Clamped to [0, max_seq_len] as L; query token i sits
 *               at position L - n_queries + i and attends positions
 *               0 .. L - n_queries + i; a query with no such position (L <
 *               n_queries - i) gets a zero output.
 *   out       : device [batch][n_queries][n_q_heads][256] in q_dtype.
 *   workspace : device, >= tq4_attn_verify_workspace_size(...) bytes, as for
 *               tq4_attn_decode.
 *   other arguments as for tq4_attn_decode.  With n_queries == 1 the result
 *   is bit-identical to tq4_attn_decode.
 */
tq4_status tq4_attn_verify(const tq4_layer_pool *pool, const void *q, tq4_dtype q_dtype, int32_t n_queries,
                           const int32_t *page_table, int32_t page_table_stride,
                           const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                           int32_t n_q_heads, float scale, void *out, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * The unfused path ([KVX]: besides the fused paths, multi-query prefill can
 * reconstruct pages into contiguous tensors of the query dtype, and gather
 * plus scaled dot-product attention is the fallback).  It materialises what
 * the fused entry points never write -- 512 B per vector instead of 130 B --
 * and exists to measure that cost and to serve callers that need plain K/V.
 *
 * tq4_reconstruct_pages -- write each cached position's K and V as bf16:
 *   k_out, v_out : device bf16 [batch][n_kv_heads][max_seq_len][256], 16-byte
 *                  aligned.  For request b and position p < L_b (seq_lens[b]
 *                  clamped to [0, max_seq_len]) the row is n * (H c[idx]) / 16
 *                  of the record at page page_table[b][p / page_size], offset
 *                  p % page_size, rounded to bf16 (nearest even).  Positions
 *                  p >= L_b are not written.  A page ID outside the pool
 *                  writes zero rows.
 *   out_dtype    : TQ4_BF16.
 *   other arguments as for tq4_attn_decode; batch <= 65535.
 * The transform runs in fp32: each value is within half a bf16 unit of the
 * exact reconstruction, plus a few fp32 units of the norm for cancellation.
 */
tq4_status tq4_reconstruct_pages(const tq4_layer_pool *pool, const int32_t *page_table,
                                 int32_t page_table_stride, const int32_t *seq_lens, int32_t batch,
                                 int32_t max_seq_len, tq4_dtype out_dtype, void *k_out, void *v_out,
                                 void *stream);

/* Bytes of device workspace tq4_sdpa_decode needs (0 for invalid sizes, and 0
 * when one workgroup covers each request and KV head). */
size_t tq4_sdpa_decode_workspace_size(int32_t batch, int32_t max_seq_len, int32_t n_q_heads,
                                      int32_t n_kv_heads);

/*
 * tq4_sdpa_decode -- single-query attention per request over dense K/V:
 *   q        : device bf16 [batch][n_q_heads][256], 16-byte aligned.
 *   k, v     : device bf16 [batch][n_kv_heads][max_seq_len][256] (the layout
 *              tq4_reconstruct_pages writes), 16-byte aligned; rows past each
 *              request's length are never read.
 *   q_dtype, kv_dtype : TQ4_BF16.
 *   seq_lens : device int32 [batch], clamped to [0, max_seq_len]; a request
 *              with 0 positions gets a zero output.
 *   n_q_heads: a multiple of n_kv_heads, n_q_heads / n_kv_heads <= 16;
 *              batch and n_kv_heads <= 65535.
 *   scale    : finite and > 0, else TQ4_ERR_VALUE.
 *   out      : device bf16 [batch][n_q_heads][256];
 *              out[b][h] = sum_j softmax_j(scale q.k_j) v_j over KV head
 *              h / (n_q_heads / n_kv_heads).
 *   workspace: device, >= tq4_sdpa_decode_workspace_size(...) bytes,
 *              256-byte aligned (may be NULL when that size is 0); contents on
 *              entry do not matter; calls sharing it must be ordered on one
 *              stream.
 */
tq4_status tq4_sdpa_decode(const void *q, tq4_dtype q_dtype, const void *k, const void *v,
                           tq4_dtype kv_dtype, const int32_t *seq_lens, int32_t batch,
                           int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads, float scale,
                           void *out, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace tq4_attn_prefill_chunk needs (0 for invalid sizes). */
size_t tq4_attn_prefill_workspace_size(int32_t prior_len, int32_t chunk_len, int32_t n_q_heads,
                                       int32_t n_kv_heads, int32_t page_size);

/*
 * tq4_attn_prefill_chunk -- causal attention of a chunk of chunk_len query
 * tokens over prior_len cached positions plus the chunk itself ([KVX]:
 * multi-query prefill reconstructs K/V tiles and runs a floating-point
 * attention consumer; here the tiles are reconstructed in the rotated domain
 * in on-chip memory and consumed by matrix-core products).
 *
 *   q         : device [chunk_len][n_q_heads][256] in q_dtype == TQ4_BF16,
 *               16-byte aligned; token t sits at absolute position
 *               prior_len + t and attends positions 0 .. prior_len + t.
 *   page_table: device int32 covering prior_len + chunk_len positions.  The
 *               chunk's own K/V must already be encoded into the pool.
 *   prior_len : >= 0; chunk_len >= 1; chunk_len * (n_q_heads / n_kv_heads) <=
 *               65535 * 128 (query rows, 128 per workgroup row of the grid).
 *   out       : device [chunk_len][n_q_heads][256] in q_dtype.
 *   scale     : as for tq4_attn_decode (finite and > 0).
 *   workspace : device, >= tq4_attn_prefill_workspace_size(...) bytes,
 *               256-byte aligned.  It holds the rotated queries and per-split
 *               partial results between the call's kernels; its contents on
 *               entry do not matter.  Calls sharing a workspace must be
 *               ordered on one stream.
 */
tq4_status tq4_attn_prefill_chunk(const tq4_layer_pool *pool, const void *q, tq4_dtype q_dtype,
                                  const int32_t *page_table, int32_t prior_len, int32_t chunk_len,
                                  int32_t n_q_heads, float scale, void *out, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * Uniform INT8 arm ([AIME]: a uniform INT8 KV cache is the comparison arm of
 * the TQ4 run).  The page gives no format;
 * the library's reading is one symmetric scale per vector:
 *   record  : 256 int8 codes q_d in [-127, 127] and one fp16 scale s; the
 *             vector is q * s (natural domain, no rotation);
 *   encoding: fp32, round to nearest even: s = fp16(max_d |x_d| / 127) (the
 *             division correctly rounded), q_d = clamp(rint(x_d / s), -127, 127);
 *             all codes 0 when s == 0.  Inputs must be finite.
 * Pool layout, like the TQ4 pools:
 *   k_codes, v_codes   : int8 [num_pages][n_kv_heads][page_size][256],
 *                        16-byte aligned
 *   k_scales, v_scales : fp16 bits [num_pages][n_kv_heads][page_size],
 *                        8-byte aligned
 * Limits as for tq4_layer_pool.  Positions, slots and page tables follow the
 * TQ4 conventions above.
 */
typedef struct tq4_int8_pool {
    int8_t *k_codes;
    int8_t *v_codes;
    uint16_t *k_scales;
    uint16_t *v_scales;
    int32_t num_pages;
    int32_t page_size;
    int32_t n_kv_heads;
    int32_t head_dim;
} tq4_int8_pool;

/* tq4_int8_encode_pages -- write INT8 records for n_tokens new positions;
 * arguments and slot rules as tq4_encode_pages.  Bit-identical to the
 * encoding rule above. */
tq4_status tq4_int8_encode_pages(const tq4_int8_pool *pool, const void *k, const void *v,
                                 tq4_dtype src_dtype, const int32_t *slots, int32_t n_tokens,
                                 void *stream);

/* Workspace bytes tq4_int8_attn_decode needs (0 for invalid sizes or when one
 * workgroup covers each request and KV head). */
size_t tq4_int8_attn_decode_workspace_size(int32_t batch, int32_t max_seq_len, int32_t n_q_heads,
                                           int32_t n_kv_heads, int32_t page_size);

/* tq4_int8_attn_decode -- single-query attention over INT8 pages:
 * out[b][h] = sum_j softmax_j(scale q.k_j) v_j with k_j, v_j the records'
 * values (codes times scale).  Arguments, limits, clamping, zero output for an
 * empty request, page-ID masking and workspace rules as tq4_attn_decode.
 * Records past a request's length may hold any bits. */
tq4_status tq4_int8_attn_decode(const tq4_int8_pool *pool, const void *q, tq4_dtype q_dtype,
                                const int32_t *page_table, int32_t page_table_stride,
                                const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                                int32_t n_q_heads, float scale, void *out, void *workspace,
                                size_t workspace_bytes, void *stream);

/* tq4_int8_attn_decode_append -- the INT8 decode step of a layer in one call:
 * encode each request's new token (the encoding rule above) and attend.
 * Results are bit-identical to tq4_int8_encode_pages(pool, k_new, v_new,
 * src_dtype, new_slots, batch) followed by tq4_int8_attn_decode(...) with the
 * other arguments, provided new_slots[b] is the slot of position
 * seq_lens[b] - 1 of request b; argument rules, the skipping of slots outside
 * the pool and of empty requests, and the race on a new slot that another
 * position of the call reads, as tq4_attn_decode_append. */
tq4_status tq4_int8_attn_decode_append(const tq4_int8_pool *pool, const void *k_new, const void *v_new,
                                       tq4_dtype src_dtype, const int32_t *new_slots, const void *q,
                                       tq4_dtype q_dtype, const int32_t *page_table, int32_t page_table_stride,
                                       const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                                       int32_t n_q_heads, float scale, void *out, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* Workspace bytes tq4_int8_attn_verify needs (as tq4_attn_verify_workspace_size). */
size_t tq4_int8_attn_verify_workspace_size(int32_t batch, int32_t max_seq_len, int32_t n_queries,
                                           int32_t n_q_heads, int32_t n_kv_heads, int32_t page_size);

/* tq4_int8_attn_verify -- the packed multi-query verifier over INT8 pages: the
 * last n_queries positions of each request attend causally in one pass over
 * its pages (query i at position L - n_queries + i attends positions 0 ..
 * L - n_queries + i; zeros if there is none).  q and out are
 * [batch][n_queries][n_q_heads][256]; n_queries * (n_q_heads / n_kv_heads) <=
 * TQ4_MAX_VERIFY_ROWS; n_queries == 1 is tq4_int8_attn_decode.  Other
 * arguments as tq4_attn_verify. */
tq4_status tq4_int8_attn_verify(const tq4_int8_pool *pool, const void *q, tq4_dtype q_dtype, int32_t n_queries,
                                const int32_t *page_table, int32_t page_table_stride,
                                const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                                int32_t n_q_heads, float scale, void *out, void *workspace,
                                size_t workspace_bytes, void *stream);

/* Workspace bytes tq4_int8_attn_prefill_chunk needs (as
 * tq4_attn_prefill_workspace_size). */
size_t tq4_int8_attn_prefill_workspace_size(int32_t prior_len, int32_t chunk_len, int32_t n_q_heads,
                                            int32_t n_kv_heads, int32_t page_size);

/* tq4_int8_attn_prefill_chunk -- causal attention of a chunk of query tokens
 * over INT8 pages: query t (absolute position prior_len + t) attends
 * positions 0 .. prior_len + t, whose records (the chunk's own included) the
 * caller has already encoded.  Arguments, limits and workspace rules as
 * tq4_attn_prefill_chunk. */
tq4_status tq4_int8_attn_prefill_chunk(const tq4_int8_pool *pool, const void *q, tq4_dtype q_dtype,
                                       const int32_t *page_table, int32_t prior_len, int32_t chunk_len,
                                       int32_t n_q_heads, float scale, void *out, void *workspace,
                                       size_t workspace_bytes, void *stream);

/*
 * Host page allocator ([ST]: admission reserves page equivalents, shared
 * prefixes are reference counted, and a departing request gives its pages back
 * only at the step boundary).  Host memory only, no HIP call; one allocator is
 * not thread-safe (the caller serialises its calls).  Page IDs index every
 * layer's pool (tq4_layer_pool) and fill page tables for the attention calls.
 *
 * Readings: the free list is first in, first out (pages are handed out from
 * its head in ID order at creation; returned pages join its tail in the
 * departing requests' finish order, each request's pages in table order).
 * Reservations are a budget: a request is admitted while the reservations of
 * all live requests fit the pool; pages beyond a request's reservation
 * (output past the guaranteed 8,192 tokens) are taken while free pages remain.
 */
typedef struct tq4_page_pool tq4_page_pool;

/* A pool of num_pages pages of page_size positions, all free (IDs 0 ..
 * num_pages - 1 in order); *out is NULL on error.  Sizes must be >= 1. */
tq4_status tq4_pages_create(int32_t num_pages, int32_t page_size, tq4_page_pool **out);
void tq4_pages_destroy(tq4_page_pool *pool);

/* Page equivalents admission reserves: ceil((prompt_len + min(output_budget,
 * 8192)) / page_size); -1 for negative sizes or page_size < 1. */
int64_t tq4_pages_admission_need(int64_t prompt_len, int64_t output_budget, int32_t page_size);

/* Admit a request: reserve tq4_pages_admission_need(...) page equivalents if
 * the live reservations still fit num_pages (else TQ4_ERR_CAPACITY, nothing
 * changes).  Its page table starts with the n_prefix shared pages (each must be
 * held by a live request; their reference counts grow by one); they must be
 * full pages of its prompt (n_prefix * page_size <= prompt_len).  *request_out
 * receives the request's handle. */
tq4_status tq4_pages_admit(tq4_page_pool *pool, int64_t prompt_len, int64_t output_budget,
                           const int32_t *prefix_pages, int32_t n_prefix, int32_t *request_out);

/* Grow a live, not departing request to hold `length` positions: pages are
 * taken from the free list's head (reference count 1) and appended to its
 * table.  TQ4_ERR_CAPACITY (nothing changes) if too few pages are free. */
tq4_status tq4_pages_extend(tq4_page_pool *pool, int32_t request, int64_t length);

/* Copy up to `capacity` of the request's page IDs (position order) into table
 * (may be NULL); returns the request's page count, -1 for a bad handle. */
int32_t tq4_pages_table(const tq4_page_pool *pool, int32_t request, int32_t *table, int32_t capacity);

/* Mark a live request as departing: its row leaves at the next boundary. */
tq4_status tq4_pages_finish(tq4_page_pool *pool, int32_t request);

/* The step boundary: for every departing request, in finish order, drop one
 * reference on each of its pages in table order (a page reaching zero joins
 * the free list's tail) and return its reservation; the handle becomes dead. */
tq4_status tq4_pages_boundary(tq4_page_pool *pool);

/* Observers: free page count; the free list in order (up to capacity entries,
 * returns its length); a page's reference count; the live reservations. */
int32_t tq4_pages_free_count(const tq4_page_pool *pool);
int32_t tq4_pages_free_list(const tq4_page_pool *pool, int32_t *pages, int32_t capacity);
int32_t tq4_pages_refcount(const tq4_page_pool *pool, int32_t page);
int64_t tq4_pages_reserved(const tq4_page_pool *pool);

#ifdef __cplusplus
}
#endif

#endif /* TQ4_H */
