// tq4_api.cpp -- the C ABI declared in include/tq4.h: argument validation
// (host only, before any HIP call), launch planning and dispatch to the gfx950
// kernels on the caller's stream.
#include "tq4.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq4_launch.h"

namespace {

constexpr int64_t kMaxRecords = (int64_t{1} << 31) - 1;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

tq4_status check_pool(const tq4_layer_pool *pool) {
    if (pool == nullptr) return TQ4_ERR_NULL;
    if (pool->head_dim != TQ4_HEAD_DIM) return TQ4_ERR_SHAPE;
    if (pool->page_size < 32 || pool->page_size > 1024 || pool->page_size % 32 != 0) return TQ4_ERR_SHAPE;
    if (pool->num_pages < 1 || pool->n_kv_heads < 1) return TQ4_ERR_SHAPE;
    const int64_t recs = int64_t{pool->num_pages} * pool->n_kv_heads * pool->page_size;
    if (recs > kMaxRecords) return TQ4_ERR_SHAPE;
    return TQ4_OK;
}

tq4_status check_int8_pool(const tq4_int8_pool *pool) {
    if (pool == nullptr) return TQ4_ERR_NULL;
    if (pool->head_dim != TQ4_HEAD_DIM) return TQ4_ERR_SHAPE;
    if (pool->page_size < 32 || pool->page_size > 1024 || pool->page_size % 32 != 0) return TQ4_ERR_SHAPE;
    if (pool->num_pages < 1 || pool->n_kv_heads < 1) return TQ4_ERR_SHAPE;
    const int64_t recs = int64_t{pool->num_pages} * pool->n_kv_heads * pool->page_size;
    if (recs > kMaxRecords) return TQ4_ERR_SHAPE;
    return TQ4_OK;
}

tq4_status check_pool_reads(const tq4_layer_pool *pool) {
    if (!pool->k_words || !pool->v_words || !pool->k_norms || !pool->v_norms) return TQ4_ERR_NULL;
    if (!aligned(pool->k_words, 16) || !aligned(pool->v_words, 16)) return TQ4_ERR_ALIGN;
    if (!aligned(pool->k_norms, 8) || !aligned(pool->v_norms, 8)) return TQ4_ERR_ALIGN;
    return TQ4_OK;
}

tq4_status check_heads(int32_t n_q_heads, int32_t n_kv_heads) {
    if (n_q_heads < 1 || n_q_heads % n_kv_heads != 0) return TQ4_ERR_SHAPE;
    if (n_q_heads / n_kv_heads > TQ4_MAX_GROUP) return TQ4_ERR_SHAPE;
    return TQ4_OK;
}

tq4_status from_hip(hipError_t e) { return e == hipSuccess ? TQ4_OK : TQ4_ERR_HIP; }

// The attention kernels take the running maximum of the scaled scores as the maximum of the scores
// times the scale, and a masked key's score (-inf) times the scale must stay -inf: the scale has
// to be finite and positive.
bool scale_ok(float scale) { return scale > 0.0f && scale <= 3.4028234663852886e38f; }

}  // namespace

extern "C" {

int tq4_abi_version(void) { return TQ4_ABI_VERSION; }

const char *tq4_status_string(tq4_status status) {
    switch (status) {
        case TQ4_OK: return "ok";
        case TQ4_ERR_NULL: return "a required pointer is NULL";
        case TQ4_ERR_SHAPE: return "a size is out of range or inconsistent";
        case TQ4_ERR_DTYPE: return "unsupported element type";
        case TQ4_ERR_ALIGN: return "a pointer is not aligned as required";
        case TQ4_ERR_WORKSPACE: return "workspace missing or too small";
        case TQ4_ERR_HIP: return "HIP runtime error";
        case TQ4_ERR_CAPACITY: return "not enough free pages or memory";
        case TQ4_ERR_VALUE: return "a scalar argument is out of range (the softmax scale must be finite and > 0)";
    }
    return "unknown status";
}

tq4_status tq4_codebook(float centroids[16], float thresholds[15]) {
    if (centroids == nullptr || thresholds == nullptr) return TQ4_ERR_NULL;
    const tq4::Codebook &cb = tq4::codebook();
    for (int i = 0; i < 16; ++i) centroids[i] = cb.centroid[i];
    for (int i = 0; i < 15; ++i) thresholds[i] = cb.threshold[i];
    return TQ4_OK;
}

tq4_status tq4_encode_pages(const tq4_layer_pool *pool, const void *k, const void *v,
                            tq4_dtype src_dtype, const int32_t *slots, int32_t n_tokens,
                            void *stream) {
    tq4_status st = check_pool(pool);
    if (st != TQ4_OK) return st;
    if (k == nullptr && v == nullptr) return TQ4_ERR_NULL;
    if (n_tokens < 0) return TQ4_ERR_SHAPE;
    if (src_dtype != TQ4_F32 && src_dtype != TQ4_BF16) return TQ4_ERR_DTYPE;
    if (k != nullptr && (!pool->k_words || !pool->k_norms)) return TQ4_ERR_NULL;
    if (v != nullptr && (!pool->v_words || !pool->v_norms)) return TQ4_ERR_NULL;
    if (n_tokens > 0 && slots == nullptr) return TQ4_ERR_NULL;
    if ((k && !aligned(k, 16)) || (v && !aligned(v, 16))) return TQ4_ERR_ALIGN;
    if ((k && !aligned(pool->k_words, 16)) || (v && !aligned(pool->v_words, 16))) return TQ4_ERR_ALIGN;
    if (!aligned(slots, 4)) return TQ4_ERR_ALIGN;
    if (n_tokens == 0) return TQ4_OK;
    tq4::EncodeParams p{};
    p.words[0] = k ? pool->k_words : nullptr;
    p.words[1] = v ? pool->v_words : nullptr;
    p.norms[0] = k ? pool->k_norms : nullptr;
    p.norms[1] = v ? pool->v_norms : nullptr;
    p.src[0] = k;
    p.src[1] = v;
    p.src_bf16 = src_dtype == TQ4_BF16;
    p.slots = slots;
    p.n_tokens = n_tokens;
    p.n_kv = pool->n_kv_heads;
    p.page_size = pool->page_size;
    p.num_slots = pool->num_pages * pool->page_size;
    return from_hip(tq4::launch_encode(p, static_cast<hipStream_t>(stream)));
}

size_t tq4_attn_decode_workspace_size(int32_t batch, int32_t max_seq_len, int32_t n_q_heads,
                                      int32_t n_kv_heads, int32_t page_size) {
    if (batch < 1 || batch > 65535 || max_seq_len < 1 || n_kv_heads < 1 || n_kv_heads > 65535) return 0;
    if (page_size < 32 || page_size > 1024 || page_size % 32 != 0) return 0;
    if (check_heads(n_q_heads, n_kv_heads) != TQ4_OK) return 0;
    return tq4::plan_decode(batch, max_seq_len, n_q_heads, n_kv_heads, 1).workspace_bytes;
}

size_t tq4_attn_verify_workspace_size(int32_t batch, int32_t max_seq_len, int32_t n_queries, int32_t n_q_heads,
                                      int32_t n_kv_heads, int32_t page_size) {
    if (batch < 1 || batch > 65535 || max_seq_len < 1 || n_kv_heads < 1 || n_kv_heads > 65535 || n_queries < 1)
        return 0;
    if (page_size < 32 || page_size > 1024 || page_size % 32 != 0) return 0;
    if (check_heads(n_q_heads, n_kv_heads) != TQ4_OK) return 0;
    if (int64_t{n_queries} * (n_q_heads / n_kv_heads) > TQ4_MAX_VERIFY_ROWS) return 0;
    return tq4::plan_decode(batch, max_seq_len, n_q_heads, n_kv_heads, n_queries).workspace_bytes;
}

namespace {

// static_ws: the call brings no workspace and uses the library's device scratch instead.
tq4_status decode_common(const tq4_layer_pool *pool, const void *k_new, const void *v_new, tq4_dtype src_dtype,
                         const int32_t *new_slots, bool append, const void *q, tq4_dtype q_dtype,
                         int32_t n_queries, const int32_t *page_table, int32_t page_table_stride, const int32_t *seq_lens,
                         int32_t batch, int32_t max_seq_len, int32_t n_q_heads, float scale, void *out,
                         void *workspace, size_t workspace_bytes, void *stream, bool static_ws = false,
                         int variant = TQ4_DECODE_FUSED) {
    tq4_status st = check_pool(pool);
    if (st != TQ4_OK) return st;
    if ((st = check_pool_reads(pool)) != TQ4_OK) return st;
    if (!q || !page_table || !seq_lens || !out) return TQ4_ERR_NULL;
    if (q_dtype != TQ4_BF16) return TQ4_ERR_DTYPE;
    if ((st = check_heads(n_q_heads, pool->n_kv_heads)) != TQ4_OK) return st;
    if (batch < 1 || batch > 65535 || max_seq_len < 1 || page_table_stride < 1) return TQ4_ERR_SHAPE;
    if (!scale_ok(scale)) return TQ4_ERR_VALUE;
    if (pool->n_kv_heads > 65535) return TQ4_ERR_SHAPE;
    if (int64_t{max_seq_len} > int64_t{page_table_stride} * pool->page_size) return TQ4_ERR_SHAPE;
    if (n_queries < 1 || int64_t{n_queries} * (n_q_heads / pool->n_kv_heads) > TQ4_MAX_VERIFY_ROWS)
        return TQ4_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(page_table, 4) || !aligned(seq_lens, 4))
        return TQ4_ERR_ALIGN;
    if (append) {
        if ((k_new == nullptr && v_new == nullptr) || new_slots == nullptr) return TQ4_ERR_NULL;
        if (src_dtype != TQ4_F32 && src_dtype != TQ4_BF16) return TQ4_ERR_DTYPE;
        if ((k_new && !aligned(k_new, 16)) || (v_new && !aligned(v_new, 16)) || !aligned(new_slots, 4))
            return TQ4_ERR_ALIGN;
    }
    const tq4::DecodePlan plan = tq4::plan_decode(batch, max_seq_len, n_q_heads, pool->n_kv_heads, n_queries);
    if (variant != TQ4_DECODE_FUSED) {
        if (variant != TQ4_DECODE_VALU_ROTATED && variant != TQ4_DECODE_VALU_LITERAL) return TQ4_ERR_VALUE;
        if (append || n_queries != 1) return TQ4_ERR_SHAPE;
        if (plan.group != 1 && plan.group != 2 && plan.group != 4 && plan.group != 6 && plan.group != 8)
            return TQ4_ERR_SHAPE;
    }
    if (static_ws) {
        if (plan.workspace_bytes > tq4::kStaticScratchBytes) return TQ4_ERR_WORKSPACE;
        workspace = nullptr;
        if (plan.workspace_bytes > 0) {
            const hipError_t e = tq4::static_scratch(&workspace);
            if (e != hipSuccess) return TQ4_ERR_HIP;
        }
    } else {
        if (plan.workspace_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.workspace_bytes))
            return TQ4_ERR_WORKSPACE;
        if (workspace != nullptr && !aligned(workspace, 256)) return TQ4_ERR_ALIGN;
    }
    tq4::DecodeParams p{};
    p.k_words = pool->k_words;
    p.v_words = pool->v_words;
    p.k_norms = pool->k_norms;
    p.v_norms = pool->v_norms;
    p.num_pages = pool->num_pages;
    p.page_size = pool->page_size;
    p.n_kv = pool->n_kv_heads;
    p.q = static_cast<const uint16_t *>(q);
    p.page_table = page_table;
    p.table_stride = page_table_stride;
    p.seq_lens = seq_lens;
    p.batch = batch;
    p.max_seq_len = max_seq_len;
    p.n_q = n_q_heads;
    p.scale = scale;
    p.out = static_cast<uint16_t *>(out);
    p.workspace = workspace;
    if (append) {
        p.k_new = k_new;
        p.v_new = v_new;
        p.new_bf16 = src_dtype == TQ4_BF16;
        p.new_slots = new_slots;
    }
    if (variant != TQ4_DECODE_FUSED)
        return from_hip(tq4::launch_decode_valu(p, plan, variant == TQ4_DECODE_VALU_LITERAL,
                                                static_cast<hipStream_t>(stream)));
    return from_hip(tq4::launch_decode(p, plan, static_cast<hipStream_t>(stream)));
}

}  // namespace

tq4_status tq4_attn_decode(const tq4_layer_pool *pool, const void *q, tq4_dtype q_dtype,
                           const int32_t *page_table, int32_t page_table_stride,
                           const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                           int32_t n_q_heads, float scale, void *out, void *workspace,
                           size_t workspace_bytes, void *stream) {
    return decode_common(pool, nullptr, nullptr, TQ4_F32, nullptr, false, q, q_dtype, 1, page_table,
                         page_table_stride, seq_lens, batch, max_seq_len, n_q_heads, scale, out, workspace,
                         workspace_bytes, stream);
}

tq4_status tq4_attn_decode_noalloc(const tq4_layer_pool *pool, const void *q, tq4_dtype q_dtype,
                                   const int32_t *page_table, int32_t page_table_stride,
                                   const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                                   int32_t n_q_heads, float scale, void *out, void *stream) {
    return decode_common(pool, nullptr, nullptr, TQ4_F32, nullptr, false, q, q_dtype, 1, page_table,
                         page_table_stride, seq_lens, batch, max_seq_len, n_q_heads, scale, out, nullptr, 0, stream,
                         true);
}

tq4_status tq4_attn_decode_variant(const tq4_layer_pool *pool, const void *q, tq4_dtype q_dtype,
                                   const int32_t *page_table, int32_t page_table_stride,
                                   const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                                   int32_t n_q_heads, float scale, tq4_decode_variant variant, void *out,
                                   void *workspace, size_t workspace_bytes, void *stream) {
    return decode_common(pool, nullptr, nullptr, TQ4_F32, nullptr, false, q, q_dtype, 1, page_table,
                         page_table_stride, seq_lens, batch, max_seq_len, n_q_heads, scale, out, workspace,
                         workspace_bytes, stream, false, static_cast<int>(variant));
}

tq4_status tq4_attn_verify(const tq4_layer_pool *pool, const void *q, tq4_dtype q_dtype, int32_t n_queries,
                           const int32_t *page_table, int32_t page_table_stride,
                           const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                           int32_t n_q_heads, float scale, void *out, void *workspace,
                           size_t workspace_bytes, void *stream) {
    return decode_common(pool, nullptr, nullptr, TQ4_F32, nullptr, false, q, q_dtype, n_queries, page_table,
                         page_table_stride, seq_lens, batch, max_seq_len, n_q_heads, scale, out, workspace,
                         workspace_bytes, stream);
}

tq4_status tq4_attn_decode_append(const tq4_layer_pool *pool, const void *k_new, const void *v_new,
                                  tq4_dtype src_dtype, const int32_t *new_slots, const void *q,
                                  tq4_dtype q_dtype, const int32_t *page_table, int32_t page_table_stride,
                                  const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                                  int32_t n_q_heads, float scale, void *out, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    return decode_common(pool, k_new, v_new, src_dtype, new_slots, true, q, q_dtype, 1, page_table,
                         page_table_stride, seq_lens, batch, max_seq_len, n_q_heads, scale, out, workspace,
                         workspace_bytes, stream);
}

tq4_status tq4_reconstruct_pages(const tq4_layer_pool *pool, const int32_t *page_table, int32_t page_table_stride,
                                 const int32_t *seq_lens, int32_t batch, int32_t max_seq_len, tq4_dtype out_dtype,
                                 void *k_out, void *v_out, void *stream) {
    tq4_status st = check_pool(pool);
    if (st != TQ4_OK) return st;
    if ((st = check_pool_reads(pool)) != TQ4_OK) return st;
    if (!page_table || !seq_lens || !k_out || !v_out) return TQ4_ERR_NULL;
    if (out_dtype != TQ4_BF16) return TQ4_ERR_DTYPE;
    if (batch < 1 || batch > 65535 || max_seq_len < 1 || page_table_stride < 1) return TQ4_ERR_SHAPE;
    if (pool->n_kv_heads > 65535) return TQ4_ERR_SHAPE;
    if (int64_t{max_seq_len} > int64_t{page_table_stride} * pool->page_size) return TQ4_ERR_SHAPE;
    if (!aligned(k_out, 16) || !aligned(v_out, 16) || !aligned(page_table, 4) || !aligned(seq_lens, 4))
        return TQ4_ERR_ALIGN;
    tq4::ReconParams p{};
    p.k_words = pool->k_words;
    p.v_words = pool->v_words;
    p.k_norms = pool->k_norms;
    p.v_norms = pool->v_norms;
    p.num_pages = pool->num_pages;
    p.page_size = pool->page_size;
    p.n_kv = pool->n_kv_heads;
    p.page_table = page_table;
    p.table_stride = page_table_stride;
    p.seq_lens = seq_lens;
    p.batch = batch;
    p.max_seq_len = max_seq_len;
    p.k_out = static_cast<uint16_t *>(k_out);
    p.v_out = static_cast<uint16_t *>(v_out);
    return from_hip(tq4::launch_reconstruct(p, static_cast<hipStream_t>(stream)));
}

size_t tq4_sdpa_decode_workspace_size(int32_t batch, int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads) {
    if (batch < 1 || max_seq_len < 1 || n_kv_heads < 1) return 0;
    if (check_heads(n_q_heads, n_kv_heads) != TQ4_OK) return 0;
    return tq4::plan_dense(batch, max_seq_len, n_q_heads, n_kv_heads).workspace_bytes;
}

tq4_status tq4_sdpa_decode(const void *q, tq4_dtype q_dtype, const void *k, const void *v, tq4_dtype kv_dtype,
                           const int32_t *seq_lens, int32_t batch, int32_t max_seq_len, int32_t n_q_heads,
                           int32_t n_kv_heads, float scale, void *out, void *workspace, size_t workspace_bytes,
                           void *stream) {
    if (!q || !k || !v || !seq_lens || !out) return TQ4_ERR_NULL;
    if (q_dtype != TQ4_BF16 || kv_dtype != TQ4_BF16) return TQ4_ERR_DTYPE;
    if (n_kv_heads < 1 || n_kv_heads > 65535) return TQ4_ERR_SHAPE;
    tq4_status st = check_heads(n_q_heads, n_kv_heads);
    if (st != TQ4_OK) return st;
    if (batch < 1 || batch > 65535 || max_seq_len < 1) return TQ4_ERR_SHAPE;
    if (!scale_ok(scale)) return TQ4_ERR_VALUE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(seq_lens, 4))
        return TQ4_ERR_ALIGN;
    const tq4::DensePlan plan = tq4::plan_dense(batch, max_seq_len, n_q_heads, n_kv_heads);
    if (plan.workspace_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.workspace_bytes))
        return TQ4_ERR_WORKSPACE;
    if (workspace != nullptr && !aligned(workspace, 256)) return TQ4_ERR_ALIGN;
    tq4::DenseParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.seq_lens = seq_lens;
    p.out = static_cast<uint16_t *>(out);
    p.workspace = workspace;
    p.batch = batch;
    p.max_seq_len = max_seq_len;
    p.n_q = n_q_heads;
    p.n_kv = n_kv_heads;
    p.scale = scale;
    return from_hip(tq4::launch_dense(p, plan, static_cast<hipStream_t>(stream)));
}

size_t tq4_attn_prefill_workspace_size(int32_t prior_len, int32_t chunk_len, int32_t n_q_heads,
                                       int32_t n_kv_heads, int32_t page_size) {
    if (prior_len < 0 || chunk_len < 1 || n_kv_heads < 1) return 0;
    if (page_size < 32 || page_size > 1024 || page_size % 32 != 0) return 0;
    if (check_heads(n_q_heads, n_kv_heads) != TQ4_OK) return 0;
    if (int64_t{prior_len} + chunk_len > (int64_t{1} << 31) - 1) return 0;
    const tq4::PrefillPlan plan = tq4::plan_prefill(prior_len, chunk_len, n_q_heads, n_kv_heads);
    if (plan.n_qblocks > 65535 || n_kv_heads > 65535) return 0;
    return plan.workspace_bytes;
}

tq4_status tq4_attn_prefill_chunk(const tq4_layer_pool *pool, const void *q, tq4_dtype q_dtype,
                                  const int32_t *page_table, int32_t prior_len, int32_t chunk_len,
                                  int32_t n_q_heads, float scale, void *out, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    tq4_status st = check_pool(pool);
    if (st != TQ4_OK) return st;
    if ((st = check_pool_reads(pool)) != TQ4_OK) return st;
    if (!q || !page_table || !out) return TQ4_ERR_NULL;
    if (q_dtype != TQ4_BF16) return TQ4_ERR_DTYPE;
    if ((st = check_heads(n_q_heads, pool->n_kv_heads)) != TQ4_OK) return st;
    if (prior_len < 0 || chunk_len < 1) return TQ4_ERR_SHAPE;
    if (int64_t{prior_len} + chunk_len > (int64_t{1} << 31) - 1) return TQ4_ERR_SHAPE;
    if (!scale_ok(scale)) return TQ4_ERR_VALUE;
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(page_table, 4)) return TQ4_ERR_ALIGN;
    const tq4::PrefillPlan plan = tq4::plan_prefill(prior_len, chunk_len, n_q_heads, pool->n_kv_heads);
    // grid (splits, query blocks, KV heads): 128 query rows per block
    if (plan.n_qblocks > 65535 || pool->n_kv_heads > 65535) return TQ4_ERR_SHAPE;
    if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) return TQ4_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return TQ4_ERR_ALIGN;
    tq4::PrefillParams p{};
    p.k_words = pool->k_words;
    p.v_words = pool->v_words;
    p.k_norms = pool->k_norms;
    p.v_norms = pool->v_norms;
    p.num_pages = pool->num_pages;
    p.page_size = pool->page_size;
    p.n_kv = pool->n_kv_heads;
    p.q = static_cast<const uint16_t *>(q);
    p.page_table = page_table;
    p.prior_len = prior_len;
    p.chunk_len = chunk_len;
    p.n_q = n_q_heads;
    p.scale = scale;
    p.out = static_cast<uint16_t *>(out);
    p.workspace = workspace;
    return from_hip(tq4::launch_prefill(p, plan, static_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- uniform INT8 arm

tq4_status tq4_int8_encode_pages(const tq4_int8_pool *pool, const void *k, const void *v,
                                 tq4_dtype src_dtype, const int32_t *slots, int32_t n_tokens,
                                 void *stream) {
    tq4_status st = check_int8_pool(pool);
    if (st != TQ4_OK) return st;
    if (k == nullptr && v == nullptr) return TQ4_ERR_NULL;
    if (n_tokens < 0) return TQ4_ERR_SHAPE;
    if (src_dtype != TQ4_F32 && src_dtype != TQ4_BF16) return TQ4_ERR_DTYPE;
    if (k != nullptr && (!pool->k_codes || !pool->k_scales)) return TQ4_ERR_NULL;
    if (v != nullptr && (!pool->v_codes || !pool->v_scales)) return TQ4_ERR_NULL;
    if (n_tokens > 0 && slots == nullptr) return TQ4_ERR_NULL;
    if ((k && !aligned(k, 16)) || (v && !aligned(v, 16))) return TQ4_ERR_ALIGN;
    if ((k && !aligned(pool->k_codes, 16)) || (v && !aligned(pool->v_codes, 16))) return TQ4_ERR_ALIGN;
    if ((k && !aligned(pool->k_scales, 8)) || (v && !aligned(pool->v_scales, 8))) return TQ4_ERR_ALIGN;
    if (!aligned(slots, 4)) return TQ4_ERR_ALIGN;
    if (n_tokens == 0) return TQ4_OK;
    tq4::Int8EncodeParams p{};
    p.codes[0] = k ? pool->k_codes : nullptr;
    p.codes[1] = v ? pool->v_codes : nullptr;
    p.scales[0] = k ? pool->k_scales : nullptr;
    p.scales[1] = v ? pool->v_scales : nullptr;
    p.src[0] = k;
    p.src[1] = v;
    p.src_bf16 = src_dtype == TQ4_BF16;
    p.slots = slots;
    p.n_tokens = n_tokens;
    p.n_kv = pool->n_kv_heads;
    p.page_size = pool->page_size;
    p.num_slots = pool->num_pages * pool->page_size;
    return from_hip(tq4::launch_int8_encode(p, static_cast<hipStream_t>(stream)));
}

size_t tq4_int8_attn_decode_workspace_size(int32_t batch, int32_t max_seq_len, int32_t n_q_heads,
                                           int32_t n_kv_heads, int32_t page_size) {
    return tq4_attn_decode_workspace_size(batch, max_seq_len, n_q_heads, n_kv_heads, page_size);
}

size_t tq4_int8_attn_verify_workspace_size(int32_t batch, int32_t max_seq_len, int32_t n_queries,
                                           int32_t n_q_heads, int32_t n_kv_heads, int32_t page_size) {
    return tq4_attn_verify_workspace_size(batch, max_seq_len, n_queries, n_q_heads, n_kv_heads, page_size);
}

namespace {

tq4_status int8_common(const tq4_int8_pool *pool, const void *k_new, const void *v_new, tq4_dtype src_dtype,
                       const int32_t *new_slots, bool append, const void *q, tq4_dtype q_dtype, int32_t n_queries,
                       const int32_t *page_table, int32_t page_table_stride, const int32_t *seq_lens,
                       int32_t batch, int32_t max_seq_len, int32_t n_q_heads, float scale, void *out,
                       void *workspace, size_t workspace_bytes, void *stream) {
    tq4_status st = check_int8_pool(pool);
    if (st != TQ4_OK) return st;
    if (!pool->k_codes || !pool->v_codes || !pool->k_scales || !pool->v_scales) return TQ4_ERR_NULL;
    if (!aligned(pool->k_codes, 16) || !aligned(pool->v_codes, 16)) return TQ4_ERR_ALIGN;
    if (!aligned(pool->k_scales, 8) || !aligned(pool->v_scales, 8)) return TQ4_ERR_ALIGN;
    if (!q || !page_table || !seq_lens || !out) return TQ4_ERR_NULL;
    if (q_dtype != TQ4_BF16) return TQ4_ERR_DTYPE;
    if ((st = check_heads(n_q_heads, pool->n_kv_heads)) != TQ4_OK) return st;
    if (batch < 1 || batch > 65535 || max_seq_len < 1 || page_table_stride < 1) return TQ4_ERR_SHAPE;
    if (!scale_ok(scale)) return TQ4_ERR_VALUE;
    if (pool->n_kv_heads > 65535) return TQ4_ERR_SHAPE;
    if (int64_t{max_seq_len} > int64_t{page_table_stride} * pool->page_size) return TQ4_ERR_SHAPE;
    if (n_queries < 1 || int64_t{n_queries} * (n_q_heads / pool->n_kv_heads) > TQ4_MAX_VERIFY_ROWS)
        return TQ4_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(page_table, 4) || !aligned(seq_lens, 4))
        return TQ4_ERR_ALIGN;
    if (append) {
        if ((k_new == nullptr && v_new == nullptr) || new_slots == nullptr) return TQ4_ERR_NULL;
        if (src_dtype != TQ4_F32 && src_dtype != TQ4_BF16) return TQ4_ERR_DTYPE;
        if ((k_new && !aligned(k_new, 16)) || (v_new && !aligned(v_new, 16)) || !aligned(new_slots, 4))
            return TQ4_ERR_ALIGN;
    }
    const tq4::DecodePlan plan = tq4::plan_decode(batch, max_seq_len, n_q_heads, pool->n_kv_heads, n_queries);
    if (plan.workspace_bytes > 0 && (workspace == nullptr || workspace_bytes < plan.workspace_bytes))
        return TQ4_ERR_WORKSPACE;
    if (workspace != nullptr && !aligned(workspace, 256)) return TQ4_ERR_ALIGN;
    tq4::Int8DecodeParams p{};
    p.k_codes = pool->k_codes;
    p.v_codes = pool->v_codes;
    p.k_scales = pool->k_scales;
    p.v_scales = pool->v_scales;
    p.num_pages = pool->num_pages;
    p.page_size = pool->page_size;
    p.n_kv = pool->n_kv_heads;
    p.q = static_cast<const uint16_t *>(q);
    p.page_table = page_table;
    p.table_stride = page_table_stride;
    p.seq_lens = seq_lens;
    p.batch = batch;
    p.max_seq_len = max_seq_len;
    p.n_q = n_q_heads;
    p.scale = scale;
    p.out = static_cast<uint16_t *>(out);
    p.workspace = workspace;
    if (append) {
        p.k_new = k_new;
        p.v_new = v_new;
        p.new_bf16 = src_dtype == TQ4_BF16;
        p.new_slots = new_slots;
    }
    return from_hip(tq4::launch_int8_decode(p, plan, static_cast<hipStream_t>(stream)));
}

}  // namespace

tq4_status tq4_int8_attn_decode(const tq4_int8_pool *pool, const void *q, tq4_dtype q_dtype,
                                const int32_t *page_table, int32_t page_table_stride,
                                const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                                int32_t n_q_heads, float scale, void *out, void *workspace,
                                size_t workspace_bytes, void *stream) {
    return int8_common(pool, nullptr, nullptr, TQ4_F32, nullptr, false, q, q_dtype, 1, page_table, page_table_stride,
                       seq_lens, batch, max_seq_len, n_q_heads, scale, out, workspace, workspace_bytes, stream);
}

tq4_status tq4_int8_attn_decode_append(const tq4_int8_pool *pool, const void *k_new, const void *v_new,
                                       tq4_dtype src_dtype, const int32_t *new_slots, const void *q,
                                       tq4_dtype q_dtype, const int32_t *page_table, int32_t page_table_stride,
                                       const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                                       int32_t n_q_heads, float scale, void *out, void *workspace,
                                       size_t workspace_bytes, void *stream) {
    return int8_common(pool, k_new, v_new, src_dtype, new_slots, true, q, q_dtype, 1, page_table, page_table_stride,
                       seq_lens, batch, max_seq_len, n_q_heads, scale, out, workspace, workspace_bytes, stream);
}

tq4_status tq4_int8_attn_verify(const tq4_int8_pool *pool, const void *q, tq4_dtype q_dtype, int32_t n_queries,
                                const int32_t *page_table, int32_t page_table_stride,
                                const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                                int32_t n_q_heads, float scale, void *out, void *workspace,
                                size_t workspace_bytes, void *stream) {
    return int8_common(pool, nullptr, nullptr, TQ4_F32, nullptr, false, q, q_dtype, n_queries, page_table,
                       page_table_stride, seq_lens, batch, max_seq_len, n_q_heads, scale, out, workspace,
                       workspace_bytes, stream);
}

size_t tq4_int8_attn_prefill_workspace_size(int32_t prior_len, int32_t chunk_len, int32_t n_q_heads,
                                            int32_t n_kv_heads, int32_t page_size) {
    return tq4_attn_prefill_workspace_size(prior_len, chunk_len, n_q_heads, n_kv_heads, page_size);
}

tq4_status tq4_int8_attn_prefill_chunk(const tq4_int8_pool *pool, const void *q, tq4_dtype q_dtype,
                                       const int32_t *page_table, int32_t prior_len, int32_t chunk_len,
                                       int32_t n_q_heads, float scale, void *out, void *workspace,
                                       size_t workspace_bytes, void *stream) {
    tq4_status st = check_int8_pool(pool);
    if (st != TQ4_OK) return st;
    if (!pool->k_codes || !pool->v_codes || !pool->k_scales || !pool->v_scales) return TQ4_ERR_NULL;
    if (!aligned(pool->k_codes, 16) || !aligned(pool->v_codes, 16)) return TQ4_ERR_ALIGN;
    if (!aligned(pool->k_scales, 8) || !aligned(pool->v_scales, 8)) return TQ4_ERR_ALIGN;
    if (!q || !page_table || !out) return TQ4_ERR_NULL;
    if (q_dtype != TQ4_BF16) return TQ4_ERR_DTYPE;
    if ((st = check_heads(n_q_heads, pool->n_kv_heads)) != TQ4_OK) return st;
    if (prior_len < 0 || chunk_len < 1) return TQ4_ERR_SHAPE;
    if (int64_t{prior_len} + chunk_len > (int64_t{1} << 31) - 1) return TQ4_ERR_SHAPE;
    if (!scale_ok(scale)) return TQ4_ERR_VALUE;
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(page_table, 4)) return TQ4_ERR_ALIGN;
    const tq4::PrefillPlan plan = tq4::plan_prefill(prior_len, chunk_len, n_q_heads, pool->n_kv_heads);
    if (plan.n_qblocks > 65535 || pool->n_kv_heads > 65535) return TQ4_ERR_SHAPE;
    if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) return TQ4_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return TQ4_ERR_ALIGN;
    tq4::Int8PrefillParams p{};
    p.k_codes = pool->k_codes;
    p.v_codes = pool->v_codes;
    p.k_scales = pool->k_scales;
    p.v_scales = pool->v_scales;
    p.num_pages = pool->num_pages;
    p.page_size = pool->page_size;
    p.n_kv = pool->n_kv_heads;
    p.q = static_cast<const uint16_t *>(q);
    p.page_table = page_table;
    p.prior_len = prior_len;
    p.chunk_len = chunk_len;
    p.n_q = n_q_heads;
    p.scale = scale;
    p.out = static_cast<uint16_t *>(out);
    p.workspace = workspace;
    return from_hip(tq4::launch_int8_prefill(p, plan, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
