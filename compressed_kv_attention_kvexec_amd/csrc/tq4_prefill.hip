// tq4_prefill.hip -- causal attention of a chunk of query tokens over TQ4 pages, gfx950.
//
// Multi-query prefill reconstructs K/V tiles and runs a floating-point attention
// consumer ("Fitting a 27B-Parameter LLM into 24 GiB of Laptop Memory", section
// "KVExec: Fused Reconstruction with Layer-Scoped Lifetime").  Here the tiles
// are reconstructed in the rotated domain (16 c[idx], fp16) in LDS and consumed
// by v_mfma_f32_16x16x32_f16; the norms scale scores and probabilities, and each
// output row gets one inverse rotation at the end (KVExec row of the mechanism
// table in "JustFit: Run Qwen 27B Fast with its full 256K context on a 24 GB
// Mac": attention in the rotated domain).
//
// Query rows of one KV head are (token, head-in-group) pairs, row = t * G + h.
// Row r of the chunk sits at absolute position prior_len + t and sees keys
// 0 .. prior_len + t.
//
// Three kernels per call:
//   1. rotate: one wavefront per query row: Hq in fp32, a power-of-two scale,
//      fp16 row and its score factor to the workspace;
//   2. attend: grid (key split, row block, KV head); 8 wavefronts (two per
//      SIMD), each owning R blocks of 16 rows.  The wavefronts decode each
//      32-key tile once, together: each turns its share of the tile's indices
//      into fp16 MFMA operands in a double-buffered LDS image, and every
//      wavefront then feeds its blocks from that image (S^T = K Q^T,
//      O^T = V^T P^T); online softmax per row with the causal limit; a partial
//      (O, max, sum) per row and split goes to the workspace.  A wavefront's
//      decode of the next tile runs inside its work on the current one (table
//      reads issued during the score products, image writes before the value
//      products), so the decode's LDS round trip overlaps matrix work; a tile's
//      V words are fetched once per workgroup (16-byte loads into an LDS word
//      buffer) instead of eight 4-byte gathers per lane in every wavefront;
//   3. combine: one wavefront per row: merges the splits, inverse rotation,
//      bf16 output (the same kernel without the rotation serves the INT8 arm).
#include <cfloat>
#include <cstddef>
#include <type_traits>

#include "tq4_device.h"
#include "tq4_launch.h"
#include "tq4_tile.h"

namespace tq4 {

constexpr int kPfWaves = 8;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfBlocks = 1;                               // R: 16-row blocks per wavefront
constexpr int kPfRowsPerWg = kPfWaves * kPfBlocks * 16;   // 128
constexpr int kPfTargetWgs = 768;                          // 3 x 256 compute units
constexpr int kPfAhead = 4;  // operand reads in flight ahead of the MFMAs that use them
constexpr float kPfRescaleSlack = 8.0f;  // log2 headroom before a running maximum is moved
constexpr int kPfNormExpMax = 9;  // value-norm exponent for the largest finite fp16 norm (< 2^16)
constexpr int kPfScanUnroll = 8;  // 4-key groups per lane in flight in the value-norm scan

struct PrefillArgs {
    PrefillParams p;
    int32_t group;
    int32_t rows;          // chunk_len * group (per KV head)
    int32_t n_splits;
    int32_t split_tiles;
    uint64_t qrot_off;     // fp16 [chunk_len * n_q][256]
    uint64_t frow_off;     // float [chunk_len * n_q]
    uint64_t parts_off;    // float [n_kv][rows][n_splits][kPfPartial]
    int32_t page_shift;    // log2(page_size) for a power-of-two page size, else -1
    uint32_t lut_pairs[8];
};

PrefillPlan plan_prefill(int32_t prior_len, int32_t chunk_len, int32_t n_q_heads, int32_t n_kv_heads) {
    PrefillPlan pl{};
    pl.group = n_q_heads / n_kv_heads;
    const int64_t rows = static_cast<int64_t>(chunk_len) * pl.group;
    pl.q_tokens_per_block = kPfRowsPerWg;  // rows per workgroup
    pl.n_qblocks = static_cast<int32_t>((rows + kPfRowsPerWg - 1) / kPfRowsPerWg);
    const int64_t tiles = (static_cast<int64_t>(prior_len) + chunk_len + kTile - 1) / kTile;
    const int64_t units = static_cast<int64_t>(pl.n_qblocks) * n_kv_heads;
    int64_t want = (kPfTargetWgs + units - 1) / units;
    const int64_t cap = (tiles + 15) / 16;  // at least 16 tiles per split
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    pl.split_tiles = static_cast<int32_t>((tiles + want - 1) / want);
    pl.n_splits = static_cast<int32_t>((tiles + pl.split_tiles - 1) / pl.split_tiles);
    const size_t qrows = static_cast<size_t>(chunk_len) * n_q_heads;
    const size_t qrot_bytes = ((qrows * kDim * 2 + 255) / 256) * 256;
    const size_t frow_bytes = ((qrows * 4 + 255) / 256) * 256;
    pl.counters_bytes = qrot_bytes + frow_bytes;  // bytes before the partials
    pl.partial_floats = kPfPartial;
    pl.workspace_bytes = pl.counters_bytes + static_cast<size_t>(n_kv_heads) * rows * pl.n_splits * kPfPartial * 4;
    return pl;
}

// ---------------------------------------------------------------- 1. rotate

__global__ __launch_bounds__(256) void tq4_prefill_rotate_kernel(PrefillArgs a) {
    const PrefillParams &p = a.p;
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);  // t * n_q + qh
    if (row >= static_cast<int64_t>(p.chunk_len) * p.n_q) return;
    const u32x2 raw = *reinterpret_cast<const u32x2 *>(p.q + row * kDim + 4 * lane);
    float y[4] = {__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                  __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
    wave_fwht(y, lane);
    float mx = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3])));
    mx = wave_max_f32(mx, lane);
    const int e = q_exponent(mx);
    const float qs = ldexpf(1.0f, e);
    char *ws = static_cast<char *>(p.workspace);
    u32x2 hv;
    hv.x = pack_f16x2(y[0] * qs, y[1] * qs);
    hv.y = pack_f16x2(y[2] * qs, y[3] * qs);
    *reinterpret_cast<u32x2 *>(ws + a.qrot_off + row * (kDim * 2) + 8 * lane) = hv;
    if (lane == 0)
        reinterpret_cast<float *>(ws + a.frow_off)[row] =
            p.scale * 1.4426950408889634f * ldexpf(1.0f, -e) * (1.0f / 256.0f);
}

// ---------------------------------------------------------------- 2. attend

// Shared tile image: the 32 fp16 MFMA operands of a 32-key tile (16 for K, 16 for V, 1 KiB each in
// lane order) and its 64 norms, double-buffered.  Entry mt * 8 + ks is the K operand of M-tile mt,
// K-step ks; entry 16 + c * 8 + i the V operand of M-tile (c, i) (lane layouts in tq4_tile.h).
struct PfTileImage {
    half8 op[32][kWave];
};

// Rows 2p and 2p + 1 of the 8x8 nibble transpose of tq4_tile.h (in[j] nibble i -> out[i] nibble j),
// for a row pair p in 0..3 given as two v_perm selectors: half_sel = p >> 1 ? 0x07060302 :
// 0x05040100 (the high or the low 16 bits of each word), pair_sel = p & 1 ? 0x07030501 :
// 0x06020400 (which byte of each 16-bit half).  10 instructions where the full transpose takes 38.
__device__ __forceinline__ void nibble_transpose_pair(const uint32_t in[8], uint32_t half_sel, uint32_t pair_sel,
                                                      uint32_t &even, uint32_t &odd) {
    const uint32_t a0 = perm(in[4], in[0], half_sel), a1 = perm(in[5], in[1], half_sel);
    const uint32_t a2 = perm(in[6], in[2], half_sel), a3 = perm(in[7], in[3], half_sel);
    const uint32_t b0 = perm(a2, a0, pair_sel), b1 = perm(a3, a1, pair_sel);
    const uint32_t m = 0x0f0f0f0fu;
    even = (b0 & m) | ((b1 << 4) & ~m);
    odd = ((b0 >> 4) & m) | (b1 & ~m);
}

// The workgroup's LDS in one object: the two operand images (64 KiB), the centroid table at byte
// 65536, the images' norms (K norms of keys 0..31, then V norms) and the wavefront maxima.  With the
// table at 2^16, a lane's table address is (index byte) * 256 + 4 * lane + 2^16, which one v_perm
// builds from the index word and lane_hi = 4 * lane + 2^16 (no base to add).
constexpr int kPfVRow = 36;  // words per key in the V word buffer (32 + 4 of padding)
template <int NW>
struct PfShared {
    PfTileImage img[2];
    uint32_t lut[kLutWords];
    float nrm[2][64];
    float nmax[NW];
    uint32_t vbuf[2][kTile * kPfVRow];  // V words of a tile, [key][word], for the decode share
};
constexpr uint32_t kPfLutOffset = 65536;

// 8 nibbles of one word -> 8 fp16 table values (dim order), the table at kPfLutOffset in lds.
__device__ __forceinline__ half8 pf_lut_decode(uint32_t w, uint32_t lane_hi, const char *lds) {
    const uint32_t a0 = perm(w, lane_hi, 0x0c020400u);
    const uint32_t a1 = perm(w, lane_hi, 0x0c020500u);
    const uint32_t a2 = perm(w, lane_hi, 0x0c020600u);
    const uint32_t a3 = perm(w, lane_hi, 0x0c020700u);
    u32x4 r;
    r.x = *reinterpret_cast<const uint32_t *>(lds + a0);
    r.y = *reinterpret_cast<const uint32_t *>(lds + a1);
    r.z = *reinterpret_cast<const uint32_t *>(lds + a2);
    r.w = *reinterpret_cast<const uint32_t *>(lds + a3);
    return __builtin_bit_cast(half8, r);
}

template <int R, int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void tq4_prefill_kernel(PrefillArgs a) {
    constexpr int NT = NW * kWave;
    constexpr int E = 16 / NW;  // K operands and V operands each wave decodes per tile
    __shared__ __align__(16) PfShared<NW> sh;
    static_assert(offsetof(PfShared<NW>, lut) == kPfLutOffset, "table offset");
    uint32_t *const lut_mem = sh.lut;
    float *const nmax_sh = sh.nmax;
    const PrefillParams &p = a.p;
    const int G = a.group;
    const int s = blockIdx.x, rb = blockIdx.y, g = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, gq = lane >> 4;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    char *ws = static_cast<char *>(p.workspace);

    // rows of this wave: row0 + 16 j + n for block j
    const int row0 = rb * kPfRowsPerWg + wave_u * (R * 16);
    const int wg_last_row = min(rb * kPfRowsPerWg + kPfRowsPerWg, a.rows) - 1;
    const int wg_kmax = p.prior_len + wg_last_row / G + 1;  // keys any row of the workgroup sees
    const int total_keys = p.prior_len + p.chunk_len;
    const int split_keys = a.split_tiles * kTile;
    const int key_begin = s * split_keys;
    const int key_end = min(key_begin + split_keys, wg_kmax);
    const int n_tiles = key_end > key_begin ? (key_end - key_begin + kTile - 1) / kTile : 0;

    // ---- this wave's share of each tile: K operands e0 .. e0 + E - 1 and V operands
    // 16 + e0 .. 16 + e0 + E - 1, e0 = E * wave.  K operand mt * 8 + 4 h + j is word 16 h + 4 gq + j
    // of key 16 mt + n (E consecutive words, one load); V operand c * 8 + i comes from transposing
    // word 2 n + c of keys sigma(0..7), read from the workgroup's V word buffer; one norm per lane
    // (K norms in lanes 0..31, V in 32..63).
    const int e0 = E * wave_u;
    const int mt_w = e0 >> 3, h_w = (e0 >> 2) & 1, j_w = e0 & 3, i_w = e0 & 7;
    const uint32_t k_lane_off = static_cast<uint32_t>(n) * 128u + static_cast<uint32_t>(gq) * 16u +
                                2048u * mt_w + 64u * h_w + 4u * j_w;
    // transpose selectors of this wave's row pairs i_w / 2 .. (i_w + E) / 2 - 1 (all in one half)
    const uint32_t half_sel = (i_w >> 2) ? 0x07060302u : 0x05040100u;
    uint32_t pair_sel[E / 2];
#pragma unroll
    for (int k = 0; k < E / 2; ++k) pair_sel[k] = (((i_w >> 1) + k) & 1) ? 0x07030501u : 0x06020400u;
    const int32_t *pt = p.page_table;
    const int pt_last = (total_keys - 1) / p.page_size;
    using KWords = std::conditional_t<E == 4, u32x4, u32x2>;
    struct Staging {
        KWords k;
        uint32_t n;
        bool valid;
    };
    // The V words of a tile are fetched once per workgroup: waves 0..3 load 16 bytes per lane (keys
    // 8 w .. 8 w + 7) into vtmp and store them into an LDS word buffer one step later; the decode
    // share reads its eight words per lane from there.
    const bool v_loader = wave_u < kTile / 8;
    u32x4 vtmp;
    const uint32_t v_key = static_cast<uint32_t>(wave_u * 8 + (lane >> 3)), v_chunk = static_cast<uint32_t>(lane & 7);
    // page index of a key (wave-uniform; a shift for power-of-two pages)
    auto page_of = [&](int key) { return a.page_shift >= 0 ? key >> a.page_shift : key / p.page_size; };
    auto fetch_pid = [&](int t) {  // wave-uniform address: a scalar load
        return pt[min(page_of(key_begin + t * kTile), pt_last)];
    };
    // loads this wave's K share and norm of tile t; returns the tile's first record
    auto load_tile = [&](Staging &st, int t, int pid) -> int64_t {
        const int key0 = key_begin + t * kTile;  // t is clamped by the caller to a tile of this split
        const int off0 = key0 - page_of(key0) * p.page_size;
        st.valid = pid >= 0 && pid < p.num_pages;  // page IDs outside the pool read page 0, masked
        const int64_t rec = (static_cast<int64_t>(st.valid ? pid : 0) * p.n_kv + g) * p.page_size + off0;
        const char *kb = reinterpret_cast<const char *>(p.k_words) + rec * (kWords * 4);
        st.k = *reinterpret_cast<const KWords *>(kb + k_lane_off);
        const uint16_t *nb = (lane < 32 ? p.k_norms : p.v_norms) + rec + (lane & 31);
        st.n = *nb;
        return rec;
    };
    auto load_v = [&](int64_t rec) {
        if (v_loader)
            vtmp = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const char *>(p.v_words) +
                                                    (rec + v_key) * (kWords * 4) + 16u * v_chunk);
    };
    auto store_v = [&](int vb) {
        if (v_loader) *reinterpret_cast<u32x4 *>(&sh.vbuf[vb][v_key * kPfVRow + 4 * v_chunk]) = vtmp;
    };
    auto load_share = [&](Staging &st, int t) { return load_tile(st, t, fetch_pid(t)); };
    const char *lds = reinterpret_cast<const char *>(&sh);
    const uint32_t lane_hi = static_cast<uint32_t>(lane) * 4u + kPfLutOffset;
    // A wave's share of a tile's decode in two parts: the table reads (issued while the matrix
    // products of the current tile run) and the image writes.
    struct Decoded {
        half8 d[2 * E];
        float nrm;
    };
    auto decode_issue = [&](const Staging &st, Decoded &dc, int vb) {
        // word 2 n + c of keys sigma(0..7) from the V word buffer
        uint32_t vw[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int key = (j < 4) ? 4 * gq + j : 16 + 4 * gq + (j - 4);
            vw[j] = sh.vbuf[vb][key * kPfVRow + 2 * n + mt_w];
        }
#pragma unroll
        for (int j = 0; j < E; ++j) dc.d[j] = pf_lut_decode(st.k[j], lane_hi, lds);
        uint32_t uw[E];  // rows i_w .. i_w + E - 1 of the transposed words
#pragma unroll
        for (int i = 0; i < E; i += 2) nibble_transpose_pair(vw, half_sel, pair_sel[i / 2], uw[i], uw[i + 1]);
#pragma unroll
        for (int i = 0; i < E; ++i) dc.d[E + i] = pf_lut_decode(uw[i], lane_hi, lds);
        dc.nrm = f16_bits_to_f32(static_cast<uint16_t>(st.n));
    };
    auto decode_write = [&](const Decoded &dc, int b) {
        PfTileImage &im = sh.img[b];
#pragma unroll
        for (int j = 0; j < E; ++j) im.op[e0 + j][lane] = dc.d[j];
#pragma unroll
        for (int i = 0; i < E; ++i) im.op[16 + e0 + i][lane] = dc.d[E + i];
        sh.nrm[b][lane] = dc.nrm;  // every wave writes the same values
    };
    auto decode_share = [&](const Staging &st, int b, int vb) {
        Decoded dc;
        decode_issue(st, dc, vb);
        __builtin_amdgcn_sched_barrier(0);
        decode_write(dc, b);
    };

    // two staging sets, each refilled in place two tiles ahead of its decode
    Staging sa, sb;
    load_v(load_share(sa, 0));

    // ---- per-block row data: causal limit, score factor, query operand (rows past the chunk see
    // no key and are never written)
    int lim_row[R];
    float fcol[R];
    half8 qop[R][8];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int row = row0 + 16 * j + n;
        const bool live = row < a.rows;
        const int t = live ? row / G : 0;
        const int qrow = t * p.n_q + g * G + (live ? row - t * G : 0);  // index into the rotated rows
        lim_row[j] = live ? p.prior_len + t + 1 : 0;
        fcol[j] = live ? reinterpret_cast<const float *>(ws + a.frow_off)[qrow] : 1.f;
        const char *qr = ws + a.qrot_off + static_cast<int64_t>(qrow) * (kDim * 2);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int w = 16 * (ks >> 2) + 4 * gq + (ks & 3);
            u32x4 v = *reinterpret_cast<const u32x4 *>(qr + 16 * w);
            if (!live) v = u32x4{0u, 0u, 0u, 0u};
            qop[j][ks] = __builtin_bit_cast(half8, v);
        }
    }
    // ---- P operand range.  The products O^T += V^T P^T take p_j n_j (softmax weight times value
    // norm) as fp16; p_j <= 2^kPfRescaleSlack, but an fp16 norm reaches 65504 and can be as small
    // as 2^-24.  The workgroup scans the value norms of its split's keys once (4 per lane and step,
    // 8-byte loads) and keeps l_run and oacc relative to 2^eo, eo = E - 7 for the largest norm in
    // [2^(E-1), 2^E): its weights are exp2(s - m_run - eo), so P < 2^15, and a term whose norm is
    // within 2^-20 of that largest one is a normal fp16 number.  The partials are written back at
    // their true scale.
    float nmx = 0.f;
    {
        const int n_groups = (key_end - key_begin + 3) >> 2;  // key_begin is a multiple of 32
        const char *vn = reinterpret_cast<const char *>(p.v_norms);
        for (int g0 = tid; g0 < n_groups; g0 += kPfScanUnroll * NT) {
            int pid[kPfScanUnroll];
#pragma unroll
            for (int u = 0; u < kPfScanUnroll; ++u) {
                const int key = key_begin + 4 * min(g0 + u * NT, n_groups - 1);
                pid[u] = pt[min(page_of(key), pt_last)];
            }
#pragma unroll
            for (int u = 0; u < kPfScanUnroll; ++u) {
                const int grp = g0 + u * NT;
                const int key = key_begin + 4 * min(grp, n_groups - 1);
                const bool ok = grp < n_groups && pid[u] >= 0 && pid[u] < p.num_pages;
                const int64_t rec =
                    (static_cast<int64_t>(ok ? pid[u] : 0) * p.n_kv + g) * p.page_size + key - page_of(key) * p.page_size;
                const u32x2 w = *reinterpret_cast<const u32x2 *>(vn + rec * 2);
                const int live = ok ? min(key_end - key, 4) : 0;  // the group's keys inside the split
                if (live > 0) nmx = fmaxf(nmx, f16lo(w.x));
                if (live > 1) nmx = fmaxf(nmx, f16hi(w.x));
                if (live > 2) nmx = fmaxf(nmx, f16lo(w.y));
                if (live > 3) nmx = fmaxf(nmx, f16hi(w.y));
            }
        }
        // norms are nonnegative: the order of their fp32 bits is their order
        nmx = __uint_as_float(wave_max_u32(__float_as_uint(nmx), lane));
        if (lane == 0) nmax_sh[wave_u] = nmx;
    }
    build_lut<NT>(lut_mem, a.lut_pairs, tid);
    store_v(0);  // tile 0's V words
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) nmx = fmaxf(nmx, nmax_sh[w]);
    int eo = 0;  // no nonzero norm: any exponent serves
    if (nmx > 0.f) {
        int E;
        frexpf(nmx, &E);  // nmx in [2^(E-1), 2^E); +inf (a norm that overflowed fp16) takes the cap
        eo = nmx <= 65504.f ? E - 7 : kPfNormExpMax;
    }
    const int t_last = max(n_tiles - 1, 0);
    decode_share(sa, 0, 0);
    bool valid0 = sa.valid, valid1 = false;  // tiles in img[0] and img[1]
    load_v(load_share(sb, min(1, t_last)));
    store_v(1);  // tile 1's V words (waits for them here, once)
    load_v(load_share(sa, min(2, t_last)));
    __syncthreads();

    float4v oacc[R][16];
    float m_run[R], l_run[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
#pragma unroll
        for (int t = 0; t < 16; ++t) oacc[j][t] = float4v{0.f, 0.f, 0.f, 0.f};
        m_run[j] = -INFINITY;
        l_run[j] = 0.f;
    }

    // Tile t for all R blocks from image b: scores, online softmax, value products.  mid_qk runs once
    // every score operand is requested, before_pv between the softmax and the value products.
    auto compute = [&](int b, int t, bool valid, auto &&mid_qk, auto &&before_pv) {
        const PfTileImage &im = sh.img[b];
        const float *nrm = sh.nrm[b];
        const int key0 = key_begin + t * kTile;
        // ---- scores for all R blocks.  Operands are read kPfAhead entries ahead of their MFMAs
        // and the order is pinned, so only a few operands are live at once (the compiler would
        // otherwise hoist all 16 reads and run out of registers).
        float4v sacc[R][2];
#pragma unroll
        for (int j = 0; j < R; ++j) sacc[j][0] = sacc[j][1] = float4v{0.f, 0.f, 0.f, 0.f};
        half8 opb[kPfAhead + 1];
#pragma unroll
        for (int e = 0; e < kPfAhead; ++e) opb[e] = im.op[e][lane];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            if (e + kPfAhead < 16) opb[(e + kPfAhead) % (kPfAhead + 1)] = im.op[e + kPfAhead][lane];
#pragma unroll
            for (int j = 0; j < R; ++j)
                sacc[j][e >> 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(opb[e % (kPfAhead + 1)], qop[j][e & 7],
                                                                         sacc[j][e >> 3], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (e == 15 - kPfAhead) {  // every score operand is requested: start the next tile's decode
                mid_qk();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the first V operands are requested before the softmax
#pragma unroll
        for (int e = 0; e < kPfAhead; ++e) opb[e] = im.op[16 + e][lane];
        // lane holds keys sigma(j): j < 4 -> 4 gq + j, else 16 + 4 gq + j - 4
        const float4 kn0 = *reinterpret_cast<const float4 *>(&nrm[4 * gq]);
        const float4 kn1 = *reinterpret_cast<const float4 *>(&nrm[16 + 4 * gq]);
        const float4 nv0 = *reinterpret_cast<const float4 *>(&nrm[32 + 4 * gq]);
        const float4 nv1 = *reinterpret_cast<const float4 *>(&nrm[48 + 4 * gq]);
        const float kn[8] = {kn0.x, kn0.y, kn0.z, kn0.w, kn1.x, kn1.y, kn1.z, kn1.w};
        const float nv[8] = {nv0.x, nv0.y, nv0.z, nv0.w, nv1.x, nv1.y, nv1.z, nv1.w};
        // ---- online softmax per block, probabilities as the P^T operand
        half8 pop[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int lim = valid ? min(key_end, lim_row[j]) - key0 : 0;  // visible keys in this tile
            // Most tiles are visible to every row of the block: those skip the per-key masking.
            // Otherwise masked keys get score -inf and value norm 0 (their records, past the cached
            // length, may hold any bits, NaN norms included).
            float xs[8], nvm[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                xs[q] = sacc[j][q >> 2][q & 3] * kn[q];
                nvm[q] = nv[q];
            }
            if (!__all(lim >= kTile)) {  // masked in place, so the common path has no copies
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int koff = (q < 4) ? (4 * gq + q) : (16 + 4 * gq + (q - 4));
                    if (koff >= lim) {
                        xs[q] = -INFINITY;
                        nvm[q] = 0.f;
                    }
                }
            }
            float mx = xs[0];
#pragma unroll
            for (int q = 1; q < 8; ++q) mx = fmaxf(mx, xs[q]);
            float lo, hi;  // row n's maximum over the four lane groups
            lane_pair<16>(mx, lo, hi);
            mx = fmaxf(lo, hi);
            lane_pair<32>(mx, lo, hi);
            mx = fmaxf(lo, hi) * fcol[j];  // fcol > 0
            // the reference maximum moves only when a score exceeds it by more than the slack
            // (exp2(s - m_run) <= 256), so rescaling is rare
            if (__any(mx > m_run[j] + kPfRescaleSlack)) {
                const float m_new = fmaxf(m_run[j], mx);
                const float alpha = (m_new > m_run[j]) ? __builtin_amdgcn_exp2f(m_run[j] - m_new) : 1.0f;
                l_run[j] *= alpha;
                // one accumulator tile at a time (the path is rare; this keeps its registers few)
#pragma unroll
                for (int tt = 0; tt < 16; ++tt) {
                    oacc[j][tt] *= alpha;
                    __builtin_amdgcn_sched_barrier(0);
                }
                m_run[j] = m_new;
            }
            // m_run is -inf only while every key of the row so far was masked; the floor keeps
            // fcol x - m finite or -inf then, and exp2(-inf) = 0 drops masked keys
            const float neg_m = -fmaxf(m_run[j], -FLT_MAX) - static_cast<float>(eo);
            float pv[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(xs[q], fcol[j], neg_m));
                l_run[j] += e;
                pv[q] = e * nvm[q];
            }
            u32x4 pr;
            pr.x = pack_f16x2(pv[0], pv[1]);
            pr.y = pack_f16x2(pv[2], pv[3]);
            pr.z = pack_f16x2(pv[4], pv[5]);
            pr.w = pack_f16x2(pv[6], pv[7]);
            pop[j] = __builtin_bit_cast(half8, pr);
        }
        __builtin_amdgcn_sched_barrier(0);
        before_pv();
        // ---- O^T += V^T P^T for all R blocks, operands pipelined as for the scores
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            if (e + kPfAhead < 16) opb[(e + kPfAhead) % (kPfAhead + 1)] = im.op[16 + e + kPfAhead][lane];
#pragma unroll
            for (int j = 0; j < R; ++j)
                oacc[j][e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(opb[e % (kPfAhead + 1)], pop[j], oacc[j][e], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Each step computes tile t from one image while this wave's share of tile t + 1 is decoded into
    // the other: the table reads are issued once the score operands are requested, and the image
    // writes go out before the value products, so the decode's LDS round trip overlaps the matrix
    // work instead of preceding it.  The staging set just decoded is refilled with tile t + 3 (its
    // page ID requested at the start of the step).  One barrier per tile; tiles go in pairs, and a
    // pair's second tile past the end is computed fully masked (its image holds a clamped, valid
    // tile), which keeps every wave's loads and barriers the same.
    auto step = [&](Staging &st, int t_next, int b_dec, int b_cmp, int t) {
        Decoded dc;
        bool &vdec = b_dec ? valid1 : valid0;
        const bool vcmp = (b_cmp ? valid1 : valid0) && t < n_tiles;
        const int tn = min(t_next, t_last);
        const int pid_next = fetch_pid(tn);  // requested now, used after the softmax
        compute(b_cmp, t, vcmp, [&] { decode_issue(st, dc, (t + 1) & 1); }, [&] {
            decode_write(dc, b_dec);
            vdec = st.valid;
            // the staging set is free again: refill it with tile t + 3 before the value products;
            // tile t + 2's V words go to their buffer (its last reader was tile t's decode, one
            // barrier ago) and tile t + 3's are requested
            const int64_t rec = load_tile(st, tn, pid_next);
            store_v((t + 2) & 1);
            load_v(rec);
        });
        __syncthreads();
    };
    for (int t = 0; t < n_tiles; t += 2) {
        step(sb, t + 3, 1, 0, t);
        step(sa, t + 4, 0, 1, t + 1);
    }

    // ---- partials: lane (gq, n) of block j holds row n, dims 8 (2 (4 gq + r) + c) + i; sums and
    // accumulators go back from 2^eo to their true scale
    float *parts = reinterpret_cast<float *>(ws + a.parts_off);
    const float escale = ldexpf(1.0f, eo);
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int row = row0 + 16 * j + n;
        float l_tot = l_run[j] + lane_xor<16>(l_run[j], lane);
        l_tot = (l_tot + lane_xor<32>(l_tot, lane)) * escale;
        if (row >= a.rows) continue;
        float *dst = parts + ((static_cast<int64_t>(g) * a.rows + row) * a.n_splits + s) * kPfPartial;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int i = 0; i < 8; ++i) dst[8 * (2 * (4 * gq + r) + c) + i] = oacc[j][8 * c + i][r] * escale;
        if (gq == 0) {
            dst[kDim] = m_run[j];
            dst[kDim + 1] = l_tot;
        }
    }
}

// ---------------------------------------------------------------- 3. combine

template <bool kRotated>
__global__ __launch_bounds__(256) void tq4_prefill_combine_kernel(PrefillCombineArgs a) {
    const int G = a.group;
    const int lane = threadIdx.x & 63;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);  // g * rows + row
    if (idx >= static_cast<int64_t>(a.n_kv) * a.rows) return;
    const int g = static_cast<int>(idx / a.rows), row = static_cast<int>(idx % a.rows);
    const float *base = a.parts + idx * a.n_splits * kPfPartial;
    float M = -INFINITY;
    for (int k = 0; k < a.n_splits; ++k) M = fmaxf(M, base[k * kPfPartial + kDim]);
    float y[4] = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    for (int k = 0; k < a.n_splits; ++k) {
        const float *pk = base + k * kPfPartial;
        const float mk = pk[kDim];
        if (mk == -INFINITY) continue;  // a split with no visible key
        const float w = __builtin_amdgcn_exp2f(mk - M);
        L += w * pk[kDim + 1];
        const float4 v = reinterpret_cast<const float4 *>(pk)[lane];
        y[0] += w * v.x;
        y[1] += w * v.y;
        y[2] += w * v.z;
        y[3] += w * v.w;
    }
    float f = L > 0.f ? 1.0f / L : 0.f;
    if constexpr (kRotated) {  // o = H O / (256 L)
        wave_fwht(y, lane);
        f *= 1.0f / 256.0f;
    }
    const int t = row / G, qh = g * G + (row - t * G);
    u32x2 o;
    o.x = static_cast<uint32_t>(f32_to_bf16(y[0] * f)) | (static_cast<uint32_t>(f32_to_bf16(y[1] * f)) << 16);
    o.y = static_cast<uint32_t>(f32_to_bf16(y[2] * f)) | (static_cast<uint32_t>(f32_to_bf16(y[3] * f)) << 16);
    *reinterpret_cast<u32x2 *>(a.out + (static_cast<int64_t>(t) * a.n_q + qh) * kDim + 4 * lane) = o;
}

hipError_t launch_prefill_combine(const PrefillCombineArgs &c, bool rotated, hipStream_t stream) {
    const int64_t blocks = (static_cast<int64_t>(c.n_kv) * c.rows + 3) / 4;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (rotated)
        hipLaunchKernelGGL(tq4_prefill_combine_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, c);
    else
        hipLaunchKernelGGL(tq4_prefill_combine_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, c);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams &p, const PrefillPlan &plan, hipStream_t stream) {
    PrefillArgs a;
    a.p = p;
    a.group = plan.group;
    a.rows = p.chunk_len * plan.group;
    a.n_splits = plan.n_splits;
    a.split_tiles = plan.split_tiles;
    const size_t qrows = static_cast<size_t>(p.chunk_len) * p.n_q;
    a.qrot_off = 0;
    a.frow_off = ((qrows * kDim * 2 + 255) / 256) * 256;
    a.parts_off = plan.counters_bytes;
    a.page_shift = (p.page_size & (p.page_size - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(p.page_size)) : -1;
    lut_pairs_from_codebook(a.lut_pairs, codebook().centroid);
    const int64_t rot_blocks = (static_cast<int64_t>(qrows) + 3) / 4;
    const int64_t comb_blocks = (static_cast<int64_t>(p.n_kv) * a.rows + 3) / 4;
    if (rot_blocks > 0x7fffffff || comb_blocks > 0x7fffffff || plan.n_qblocks > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(tq4_prefill_rotate_kernel, dim3(static_cast<unsigned>(rot_blocks)), dim3(256), 0, stream, a);
    hipLaunchKernelGGL((tq4_prefill_kernel<kPfBlocks, kPfWaves>), dim3(plan.n_splits, plan.n_qblocks, p.n_kv), dim3(kPfThreads),
                       0, stream, a);
    PrefillCombineArgs c;
    c.parts = reinterpret_cast<const float *>(static_cast<const char *>(p.workspace) + a.parts_off);
    c.out = p.out;
    c.rows = a.rows;
    c.group = a.group;
    c.n_splits = a.n_splits;
    c.n_kv = p.n_kv;
    c.n_q = p.n_q;
    return launch_prefill_combine(c, true, stream);
}

}  // namespace tq4
