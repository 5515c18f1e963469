// tq4_launch.h -- host-side launch interface between the C ABI layer and the
// gfx950 kernels.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tq4 {

struct Codebook {
    float centroid[16];   // ascending fp32 centroids (Lloyd-Max levels of N(0,1) / 16)
    float threshold[15];  // fp32 midpoints of adjacent centroids
};

// Host-computed codec constants (computed once, thread-safe).
const Codebook &codebook();

struct EncodeParams {
    uint32_t *words[2];  // K, V (NULL: skip that half)
    uint16_t *norms[2];
    const void *src[2];
    int src_bf16;
    const int32_t *slots;
    int32_t n_tokens;
    int32_t n_kv;
    int32_t page_size;
    int32_t num_slots;  // num_pages * page_size
};

hipError_t launch_encode(const EncodeParams &p, hipStream_t stream);

// Split-K plan of one decode call; a pure function of the sizes so the
// workspace query needs no device.
struct DecodePlan {
    int32_t group;        // n_q_heads / n_kv_heads
    int32_t n_queries;    // query tokens per request (1: decode)
    int32_t rows;         // n_queries * group query rows per (request, KV head)
    int32_t col_blocks;   // 16-column MFMA blocks holding the rows
    int32_t slots;        // tile slots per split workgroup (wavefronts per column block)
    int32_t n_splits;     // workgroups per (request, KV head)
    int32_t split_tiles;  // 32-key tiles per workgroup
    size_t counters_bytes;
    size_t partial_floats;  // floats per (request, KV head, split)
    size_t workspace_bytes;
};

DecodePlan plan_decode(int32_t batch, int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads,
                       int32_t n_queries);

struct DecodeParams {
    const uint32_t *k_words;
    const uint32_t *v_words;
    const uint16_t *k_norms;
    const uint16_t *v_norms;
    int32_t num_pages;
    int32_t page_size;
    int32_t n_kv;
    const uint16_t *q;  // bf16 bits [batch][n_queries][n_q][256]
    const int32_t *page_table;
    int32_t table_stride;
    const int32_t *seq_lens;
    int32_t batch;
    int32_t max_seq_len;
    int32_t n_q;
    float scale;
    uint16_t *out;  // bf16 bits [batch][n_queries][n_q][256]
    void *workspace;
    // optional: encode one new token per request before attending (NULL k_new and v_new: none)
    const void *k_new;  // [batch][n_kv][256] fp32 or bf16
    const void *v_new;
    int32_t new_bf16;
    const int32_t *new_slots;  // [batch]
};

hipError_t launch_decode(const DecodeParams &p, const DecodePlan &plan, hipStream_t stream);
// Decode on the vector ALUs only (no matrix cores), same plan and partials as launch_decode:
// rotated-domain scores and values (literal false), or per-key reconstruction in the natural
// domain (literal true).  Group sizes 1, 2, 4, 6, 8; one query token; no append.
hipError_t launch_decode_valu(const DecodeParams &p, const DecodePlan &plan, bool literal, hipStream_t stream);

// Device scratch for decode calls that bring no workspace: 4 MiB, which holds every decode plan
// with n_q / n_kv <= 6 (at most 3,394,560 bytes, any batch and length).
constexpr size_t kStaticScratchBytes = size_t{4} << 20;
// The current device's address of that scratch (looked up once per device).
hipError_t static_scratch(void **out);

constexpr int kSplitStatPad = 64;  // floats of each statistic row (M, L) in a split partial

// Merge of split-K partials into bf16 rows (shared by the fused decode and the dense path).  The
// partial of (request, KV head, split) holds M[rows] and L[rows], each padded to 64 floats, then
// O[rows][256]; row r is query token r / group, head r % group of the KV head's group.
struct CombineArgs {
    const float *parts;      // [batch][n_kv][n_splits][partial_floats]
    const int32_t *seq_lens;
    uint16_t *out;           // bf16 [batch][n_queries][n_q][256]
    int32_t max_seq_len;
    int32_t split_tiles;     // 32-key tiles per split
    int32_t n_splits;
    int32_t partial_floats;
    int32_t rows;
    int32_t group;
    int32_t n_queries;
    int32_t n_q;
    int32_t n_kv;
    int32_t batch;
};
// rotated: O is in the rotated domain (the output is H O / (256 L)); else the output is O / L.
hipError_t launch_split_combine(const CombineArgs &c, bool rotated, hipStream_t stream);

// Unfused path: reconstruction into contiguous bf16 K/V, then dense decode attention.
struct ReconParams {
    const uint32_t *k_words;
    const uint32_t *v_words;
    const uint16_t *k_norms;
    const uint16_t *v_norms;
    int32_t num_pages;
    int32_t page_size;
    int32_t n_kv;
    const int32_t *page_table;
    int32_t table_stride;
    const int32_t *seq_lens;
    int32_t batch;
    int32_t max_seq_len;
    uint16_t *k_out;  // bf16 bits [batch][n_kv][max_seq_len][256]
    uint16_t *v_out;
};

hipError_t launch_reconstruct(const ReconParams &p, hipStream_t stream);

struct DensePlan {
    int32_t group;
    int32_t waves;        // wavefronts per split workgroup
    int32_t n_splits;
    int32_t split_tiles;  // 32-key tiles per workgroup
    size_t partial_floats;
    size_t workspace_bytes;
};

DensePlan plan_dense(int32_t batch, int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads);

struct DenseParams {
    const uint16_t *q;  // bf16 bits [batch][n_q][256]
    const uint16_t *k;  // bf16 bits [batch][n_kv][max_seq_len][256]
    const uint16_t *v;
    const int32_t *seq_lens;
    uint16_t *out;      // bf16 bits [batch][n_q][256]
    void *workspace;
    int32_t batch;
    int32_t max_seq_len;
    int32_t n_q;
    int32_t n_kv;
    float scale;
};

hipError_t launch_dense(const DenseParams &p, const DensePlan &plan, hipStream_t stream);

// Uniform INT8 arm: records of 256 int8 codes and one fp16 scale, pools laid out like the TQ4 pools.
struct Int8EncodeParams {
    int8_t *codes[2];  // K, V (NULL: skip that half)
    uint16_t *scales[2];
    const void *src[2];
    int src_bf16;
    const int32_t *slots;
    int32_t n_tokens;
    int32_t n_kv;
    int32_t page_size;
    int32_t num_slots;
};

hipError_t launch_int8_encode(const Int8EncodeParams &p, hipStream_t stream);

struct Int8DecodeParams {
    const int8_t *k_codes;  // [num_pages][n_kv][page_size][256]
    const int8_t *v_codes;
    const uint16_t *k_scales;  // fp16 bits [num_pages][n_kv][page_size]
    const uint16_t *v_scales;
    int32_t num_pages;
    int32_t page_size;
    int32_t n_kv;
    const uint16_t *q;  // bf16 bits [batch][n_q][256]
    const int32_t *page_table;
    int32_t table_stride;
    const int32_t *seq_lens;
    int32_t batch;
    int32_t max_seq_len;
    int32_t n_q;
    float scale;
    uint16_t *out;  // bf16 bits [batch][n_q][256]
    void *workspace;
    // optional (decode only): encode one new token per request before attending (NULL k_new and
    // v_new: none)
    const void *k_new;  // [batch][n_kv][256] fp32 or bf16
    const void *v_new;
    int32_t new_bf16;
    const int32_t *new_slots;  // [batch]
};

// plan: plan_decode(batch, max_seq_len, n_q, n_kv, n_queries)
hipError_t launch_int8_decode(const Int8DecodeParams &p, const DecodePlan &plan, hipStream_t stream);

struct PrefillPlan {
    int32_t group;
    int32_t q_tokens_per_block;  // chunk tokens per query block
    int32_t n_qblocks;
    int32_t n_splits;            // key splits per (query block, KV head)
    int32_t split_tiles;
    size_t counters_bytes;
    size_t partial_floats;
    size_t workspace_bytes;
};

PrefillPlan plan_prefill(int32_t prior_len, int32_t chunk_len, int32_t n_q_heads, int32_t n_kv_heads);

struct PrefillParams {
    const uint32_t *k_words;
    const uint32_t *v_words;
    const uint16_t *k_norms;
    const uint16_t *v_norms;
    int32_t num_pages;
    int32_t page_size;
    int32_t n_kv;
    const uint16_t *q;  // bf16 [chunk][n_q][256]
    const int32_t *page_table;
    int32_t prior_len;
    int32_t chunk_len;
    int32_t n_q;
    float scale;
    uint16_t *out;
    void *workspace;
};

hipError_t launch_prefill(const PrefillParams &p, const PrefillPlan &plan, hipStream_t stream);

constexpr int kPfPartial = 256 + 4;  // prefill split partial per (KV head, row, split): O[256], max, sum, pad

// Merge of prefill split partials into bf16 rows (the TQ4 path with the inverse rotation, the INT8
// arm without).  Row r of a KV head is chunk token r / group, head r % group of the group.
struct PrefillCombineArgs {
    const float *parts;  // [n_kv][rows][n_splits][kPfPartial]
    uint16_t *out;       // bf16 [chunk_len][n_q][256]
    int32_t rows;
    int32_t group;
    int32_t n_splits;
    int32_t n_kv;
    int32_t n_q;
};
hipError_t launch_prefill_combine(const PrefillCombineArgs &c, bool rotated, hipStream_t stream);

struct Int8PrefillParams {
    const int8_t *k_codes;
    const int8_t *v_codes;
    const uint16_t *k_scales;
    const uint16_t *v_scales;
    int32_t num_pages;
    int32_t page_size;
    int32_t n_kv;
    const uint16_t *q;  // bf16 [chunk][n_q][256]
    const int32_t *page_table;
    int32_t prior_len;
    int32_t chunk_len;
    int32_t n_q;
    float scale;
    uint16_t *out;
    void *workspace;
};

// plan: plan_prefill(prior_len, chunk_len, n_q, n_kv) (same workspace layout as the TQ4 prefill)
hipError_t launch_int8_prefill(const Int8PrefillParams &p, const PrefillPlan &plan, hipStream_t stream);

}  // namespace tq4
