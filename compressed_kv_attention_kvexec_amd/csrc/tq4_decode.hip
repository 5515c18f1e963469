// tq4_decode.hip -- single-query decode attention directly on TQ4 pages, gfx950.
//
// What is computed ("Fitting a 27B-Parameter LLM into 24 GiB of Laptop
// Memory", section "KVExec: Fused Reconstruction with Layer-Scoped Lifetime";
// rotated-domain form from the KVExec row of the mechanism table in "JustFit:
// Run Qwen 27B Fast with its full 256K context on a 24 GB Mac"):
//
//   k_j = n_j * R c[idx_j],  R = H/16 symmetric orthonormal
//   q . k_j = n_j * (R q) . c[idx_j]            -> rotate q once, not every key
//   o = sum_j p_j v_j = R ( sum_j p_j n_j c[idx_j] )  -> rotate the output once
//
// so a page is consumed as 4-bit indices -> centroid values -> products,
// with no per-key Hadamard and no float K/V outside registers and LDS.
//
// Work decomposition: grid (split, KV head, request); 8 wavefronts per
// workgroup; a wavefront owns 32-key tiles of its workgroup's key range.
// Per tile and wavefront (GQA group of G <= 16 query heads padded to 16):
//   S^T[32 keys][16 heads] = K_tile . Q_rot^T   16 x v_mfma_f32_16x16x32_f16
//   online softmax in base 2 (norms folded into scores and weights)
//   O[16 heads][256] += P . V_tile               16 x v_mfma_f32_16x16x32_f16
// K operands: lane (row r, group gq) loads 16 bytes = 4 words of key r; each
// word (8 dims) is one MFMA A-operand slice.  V operands need 8 keys per lane
// at one dim, so a lane loads word w of 8 keys and transposes the 8x8 nibble
// block in registers (v_perm and bitfield inserts).  A nibble byte becomes two
// fp16 centroid values through an LDS table of 256 entries replicated once per
// lane (lane-private banks, conflict-free), addressed with one v_perm.
// The workgroup's partial (max, sum, accumulator) goes to the workspace; the
// last workgroup of a (request, KV head) combines the partials in fixed split
// order, applies the inverse rotation and writes bf16.
#include "tq4_device.h"
#include "tq4_launch.h"

namespace tq4 {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kTile = 32;
constexpr int kLutEntries = 256;
constexpr int kLutWords = kLutEntries * kWave;  // 64 KiB
constexpr int kMaxSplits = 512;
constexpr int kPlanCUs = 256;       // MI355X compute units
constexpr int kPlanWgsPerCU = 1;    // resident decode workgroups per CU
constexpr int kMinTilesPerWave = 2;

struct DecodeArgs {
    DecodeParams p;
    int32_t group;
    int32_t n_splits;
    int32_t split_tiles;
    int32_t partial_floats;
    uint32_t lut_pairs[8];  // fp16 bits of 16 * centroid[i], two per word (i = 2k, 2k+1)
};

// ---------------------------------------------------------------- planning

DecodePlan plan_decode(int32_t batch, int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads) {
    DecodePlan pl{};
    pl.group = n_q_heads / n_kv_heads;
    const int64_t tiles = (static_cast<int64_t>(max_seq_len) + kTile - 1) / kTile;
    const int64_t units = static_cast<int64_t>(batch) * n_kv_heads;
    int64_t want = (static_cast<int64_t>(kPlanCUs) * kPlanWgsPerCU + units - 1) / units;
    const int64_t cap = (tiles + kDecWaves * kMinTilesPerWave - 1) / (kDecWaves * kMinTilesPerWave);
    if (want > cap) want = cap;
    if (want > kMaxSplits) want = kMaxSplits;
    if (want < 1) want = 1;
    pl.split_tiles = static_cast<int32_t>((tiles + want - 1) / want);
    pl.n_splits = static_cast<int32_t>((tiles + pl.split_tiles - 1) / pl.split_tiles);
    pl.counters_bytes = ((static_cast<size_t>(units) * 4 + 255) / 256) * 256;
    pl.partial_floats = 32 + static_cast<size_t>(pl.group) * kDim;
    pl.workspace_bytes = pl.counters_bytes +
                         static_cast<size_t>(units) * pl.n_splits * pl.partial_floats * sizeof(float);
    return pl;
}

// ---------------------------------------------------------------- device helpers

struct __align__(16) TileRegs {
    u32x4 k[2][2];   // [M-tile][half]: words 16*half + 4*gq .. +3 of key 16*mt + (lane & 15)
    u32x2 v[8];      // words 2n, 2n+1 of key sigma(j)
    u32x2 kn[2];     // K norms of keys 4gq..4gq+3 and 16+4gq..16+4gq+3
    u32x2 vn[2];     // V norms of the same keys
    int valid;       // page ID in range
};

// 8 nibbles of one word -> 8 fp16 values (dim order) via the lane-private LDS table.
__device__ __forceinline__ half8 lut_decode(uint32_t w, uint32_t lane4, const char *lut) {
    const uint32_t a0 = perm(w, lane4, 0x0c0c0400u);
    const uint32_t a1 = perm(w, lane4, 0x0c0c0500u);
    const uint32_t a2 = perm(w, lane4, 0x0c0c0600u);
    const uint32_t a3 = perm(w, lane4, 0x0c0c0700u);
    u32x4 r;
    r.x = *reinterpret_cast<const uint32_t *>(lut + a0);
    r.y = *reinterpret_cast<const uint32_t *>(lut + a1);
    r.z = *reinterpret_cast<const uint32_t *>(lut + a2);
    r.w = *reinterpret_cast<const uint32_t *>(lut + a3);
    return __builtin_bit_cast(half8, r);
}

// Transpose an 8x8 block of nibbles: in[j] nibble i -> out[i] nibble j.
__device__ __forceinline__ void nibble_transpose8(const uint32_t in[8], uint32_t out[8]) {
    uint32_t a[8], b[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a[j] = perm(in[j + 4], in[j], 0x05040100u);      // low halves
        a[j + 4] = perm(in[j + 4], in[j], 0x07060302u);  // high halves
    }
#pragma unroll
    for (int k = 0; k < 8; k += 4) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int x = k + kk;
            b[x] = perm(a[x + 2], a[x], 0x06020400u);
            b[x + 2] = perm(a[x + 2], a[x], 0x07030501u);
        }
    }
    const uint32_t m = 0x0f0f0f0fu;
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
        out[k] = (b[k] & m) | ((b[k + 1] << 4) & ~m);
        out[k + 1] = ((b[k] >> 4) & m) | (b[k + 1] & ~m);
    }
}

__device__ __forceinline__ float f16lo(uint32_t w) { return f16_bits_to_f32(static_cast<uint16_t>(w)); }
__device__ __forceinline__ float f16hi(uint32_t w) { return f16_bits_to_f32(static_cast<uint16_t>(w >> 16)); }

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_f16_bits(lo)) | (static_cast<uint32_t>(f32_to_f16_bits(hi)) << 16);
}

__device__ __forceinline__ void load_tile(const DecodeArgs &a, int b, int g, int key0, int lane, TileRegs &t) {
    const DecodeParams &p = a.p;
    const int page_idx = key0 / p.page_size;
    const int off0 = key0 - page_idx * p.page_size;
    int pid = p.page_table[static_cast<int64_t>(b) * p.table_stride + page_idx];
    t.valid = (pid >= 0 && pid < p.num_pages);
    if (!t.valid) pid = 0;
    const int64_t rec0 = (static_cast<int64_t>(pid) * p.n_kv + g) * p.page_size + off0;
    const int n = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            t.k[mt][h] = *reinterpret_cast<const u32x4 *>(p.k_words + (rec0 + 16 * mt + n) * kWords + 16 * h + 4 * gq);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int key = (j < 4) ? (4 * gq + j) : (16 + 4 * gq + (j - 4));
        t.v[j] = *reinterpret_cast<const u32x2 *>(p.v_words + (rec0 + key) * kWords + 2 * n);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        t.kn[h] = *reinterpret_cast<const u32x2 *>(p.k_norms + rec0 + 16 * h + 4 * gq);
        t.vn[h] = *reinterpret_cast<const u32x2 *>(p.v_norms + rec0 + 16 * h + 4 * gq);
    }
}

// In-place unnormalised Hadamard transform of rows [G][256] in LDS by the whole workgroup.
__device__ __forceinline__ void lds_fwht_rows(float *buf, int rows, int tid) {
    for (int h = 1; h < kDim; h <<= 1) {
        for (int i = tid; i < rows * (kDim / 2); i += kDecThreads) {
            const int r = i / (kDim / 2), k = i - r * (kDim / 2);
            const int lo = ((k & ~(h - 1)) << 1) | (k & (h - 1));
            float *row = buf + r * kDim;
            const float x = row[lo], y = row[lo + h];
            row[lo] = x + y;
            row[lo + h] = x - y;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- kernel

__global__ __launch_bounds__(kDecThreads) void tq4_decode_kernel(DecodeArgs a) {
    __shared__ __align__(16) uint32_t lut_mem[kLutWords];
    __shared__ float stat_m[kDecWaves][16];
    __shared__ float stat_l[kDecWaves][16];
    __shared__ float head_f[16];
    __shared__ float head_q[16];
    __shared__ int ticket_sh;

    const DecodeParams &p = a.p;
    const int G = a.group;
    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, gq = lane >> 4;

    int L = p.seq_lens[b];
    L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
    const int split_keys = a.split_tiles * kTile;
    const int n_active = (L + split_keys - 1) / split_keys;
    uint16_t *outp = p.out + (static_cast<int64_t>(b) * p.n_q + static_cast<int64_t>(g) * G) * kDim;
    if (s >= n_active) {
        if (L == 0 && s == 0)
            for (int i = tid; i < G * kDim; i += kDecThreads) outp[i] = 0;
        return;
    }
    const int key_begin = s * split_keys;
    const int key_end = min(key_begin + split_keys, L);
    const int n_tiles = (key_end - key_begin + kTile - 1) / kTile;

    float *scratch = reinterpret_cast<float *>(lut_mem);

    // ---- rotate the group's queries: Hq (unnormalised) in LDS, per-head power-of-two scale
    {
        const uint16_t *qg = p.q + (static_cast<int64_t>(b) * p.n_q + static_cast<int64_t>(g) * G) * kDim;
        for (int i = tid; i < G * kDim; i += kDecThreads) scratch[i] = bf16_to_f32(qg[i]);
        __syncthreads();
        lds_fwht_rows(scratch, G, tid);
        for (int h = wave; h < G; h += kDecWaves) {
            float mx = 0.f;
            for (int d = lane; d < kDim; d += kWave) mx = fmaxf(mx, fabsf(scratch[h * kDim + d]));
            for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, kWave));
            if (lane == 0) {
                int e = 0;
                if (mx > 0.f) {
                    int E;
                    frexpf(mx, &E);
                    e = 14 - E;  // scaled max lies in [2^13, 2^14)
                }
                head_q[h] = ldexpf(1.0f, e);
                // score (log2 units) = acc * norm * f ; acc = (2^e H q) . (16 c)
                head_f[h] = p.scale * 1.4426950408889634f * ldexpf(1.0f, -e) * (1.0f / 256.0f);
            }
        }
        __syncthreads();
    }
    half8 qop[8];
    float fcol;
    {
        const bool live = n < G;
        const float qs = live ? head_q[n] : 0.f;
        fcol = live ? head_f[n] : 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int w = 16 * (ks >> 2) + 4 * gq + (ks & 3);
            u32x4 r;
            const float *src = scratch + (live ? n : 0) * kDim + 8 * w;
            r.x = pack_f16x2(src[0] * qs, src[1] * qs);
            r.y = pack_f16x2(src[2] * qs, src[3] * qs);
            r.z = pack_f16x2(src[4] * qs, src[5] * qs);
            r.w = pack_f16x2(src[6] * qs, src[7] * qs);
            qop[ks] = __builtin_bit_cast(half8, r);
        }
    }
    __syncthreads();
    // ---- centroid table: entry e (a nibble pair) -> fp16x2 (16 c[e & 15], 16 c[e >> 4]); one copy per lane
    for (int i = tid; i < kLutWords; i += kDecThreads) {
        const int e = i >> 6;
        const uint32_t lo = (a.lut_pairs[(e & 15) >> 1] >> (16 * (e & 1))) & 0xffffu;
        const uint32_t hi = (a.lut_pairs[(e >> 4) >> 1] >> (16 * ((e >> 4) & 1))) & 0xffffu;
        lut_mem[i] = lo | (hi << 16);
    }
    __syncthreads();

    const char *lut = reinterpret_cast<const char *>(lut_mem);
    const uint32_t lane4 = static_cast<uint32_t>(lane) * 4u;

    float4v oacc[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) oacc[t] = float4v{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    TileRegs cur, nxt;
    int t = wave;
    if (t < n_tiles) load_tile(a, b, g, key_begin + t * kTile, lane, cur);
    for (; t < n_tiles; t += kDecWaves) {
        const int tn = t + kDecWaves;
        if (tn < n_tiles) load_tile(a, b, g, key_begin + tn * kTile, lane, nxt);
        const int key0 = key_begin + t * kTile;

        // ---- scores S^T (rows: keys, columns: heads)
        float4v sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sacc[mt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const u32x4 kw = cur.k[mt][ks >> 2];
                const uint32_t w = (ks & 3) == 0 ? kw.x : (ks & 3) == 1 ? kw.y : (ks & 3) == 2 ? kw.z : kw.w;
                sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lut_decode(w, lane4, lut), qop[ks], sacc[mt], 0, 0, 0);
            }
        }
        // lane holds head n, keys sigma(j): j < 4 -> 4gq + j, else 16 + 4gq + j - 4
        float sc[8];
        float nv[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float k0 = f16lo(cur.kn[h].x), k1 = f16hi(cur.kn[h].x), k2 = f16lo(cur.kn[h].y), k3 = f16hi(cur.kn[h].y);
            sc[4 * h + 0] = sacc[h][0] * k0 * fcol;
            sc[4 * h + 1] = sacc[h][1] * k1 * fcol;
            sc[4 * h + 2] = sacc[h][2] * k2 * fcol;
            sc[4 * h + 3] = sacc[h][3] * k3 * fcol;
            nv[4 * h + 0] = f16lo(cur.vn[h].x);
            nv[4 * h + 1] = f16hi(cur.vn[h].x);
            nv[4 * h + 2] = f16lo(cur.vn[h].y);
            nv[4 * h + 3] = f16hi(cur.vn[h].y);
        }
        const int lim = cur.valid ? (key_end - key0) : 0;  // keys at tile offset >= lim are masked
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int koff = (j < 4) ? (4 * gq + j) : (16 + 4 * gq + (j - 4));
            if (koff >= lim) sc[j] = -INFINITY;
        }
        float mx = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sc[j]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        const float m_new = fmaxf(m_run, mx);
        if (__any(m_new > m_run)) {
            const float alpha = (m_new > m_run) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * gq + r, kWave);
#pragma unroll
                for (int tt = 0; tt < 16; ++tt) oacc[tt][r] *= ar;
            }
            m_run = m_new;
        }
        float pv[8];
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float e = (sc[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[j] - m_run);
            psum += e;
            pv[j] = (n < G) ? e * nv[j] : 0.f;
        }
        l_run += psum;
        u32x4 pr;
        pr.x = pack_f16x2(pv[0], pv[1]);
        pr.y = pack_f16x2(pv[2], pv[3]);
        pr.z = pack_f16x2(pv[4], pv[5]);
        pr.w = pack_f16x2(pv[6], pv[7]);
        const half8 pop = __builtin_bit_cast(half8, pr);

        // ---- O += P V over two word columns (words 2n and 2n+1 of each key)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            uint32_t wv[8], u[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) wv[j] = c == 0 ? cur.v[j].x : cur.v[j].y;
            nibble_transpose8(wv, u);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                oacc[8 * c + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pop, lut_decode(u[i], lane4, lut), oacc[8 * c + i], 0, 0, 0);
        }
        cur = nxt;
    }

    // ---- per-wave softmax totals
    float l_tot = l_run + __shfl_xor(l_run, 16, kWave);
    l_tot = l_tot + __shfl_xor(l_tot, 32, kWave);
    __syncthreads();  // table no longer needed
    if (gq == 0) {
        stat_m[wave][n] = m_run;
        stat_l[wave][n] = l_tot;
    }
    __syncthreads();

    // ---- combine the workgroup's waves (fixed order) into LDS: M, L, O[G][256]
    float *obuf = scratch;                           // [slots][G][256]
    const int per_slot = G * kDim;
    const int slots = (kLutWords - kDim * 16) / per_slot;  // the last 16 rows hold the result
    float *res = scratch + kLutWords - kDim * 16;           // [G][256] combined accumulator
    float *resM = reinterpret_cast<float *>(&head_q[0]);       // reuse: per-head max
    float *resL = reinterpret_cast<float *>(&head_f[0]);       // reuse: per-head sum
    if (tid < G) {
        float M = -INFINITY;
        for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, stat_m[w][tid]);
        float Ls = 0.f;
        for (int w = 0; w < kDecWaves; ++w)
            Ls += (stat_m[w][tid] == -INFINITY) ? 0.f : stat_l[w][tid] * __builtin_amdgcn_exp2f(stat_m[w][tid] - M);
        resM[tid] = M;
        resL[tid] = Ls;
    }
    __syncthreads();
    for (int i = tid; i < per_slot; i += kDecThreads) res[i] = 0.f;
    for (int w0 = 0; w0 < kDecWaves; w0 += slots) {
        if (wave >= w0 && wave < w0 + slots) {
            float *dst = obuf + (wave - w0) * per_slot;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int h = 4 * gq + r;
                if (h < G) {
                    const float mw = stat_m[wave][h];
                    const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - resM[h]);
#pragma unroll
                    for (int c = 0; c < 2; ++c)
#pragma unroll
                        for (int i = 0; i < 8; ++i) dst[h * kDim + 8 * (2 * n + c) + i] = oacc[8 * c + i][r] * f;
                }
            }
        }
        __syncthreads();
        const int cnt = min(slots, kDecWaves - w0);
        for (int i = tid; i < per_slot; i += kDecThreads) {
            float acc = res[i];
            for (int w = 0; w < cnt; ++w) acc += obuf[w * per_slot + i];
            res[i] = acc;
        }
        __syncthreads();
    }

    // ---- cross-workgroup combine
    if (n_active > 1) {
        const size_t bg = static_cast<size_t>(b) * p.n_kv + g;
        uint32_t *counters = static_cast<uint32_t *>(p.workspace);
        float *parts = reinterpret_cast<float *>(static_cast<char *>(p.workspace) +
                                                 ((static_cast<size_t>(p.batch) * p.n_kv * 4 + 255) / 256) * 256);
        float *mine = parts + (bg * a.n_splits + s) * static_cast<size_t>(a.partial_floats);
        if (tid < G) {
            mine[tid] = resM[tid];
            mine[16 + tid] = resL[tid];
        }
        for (int i = tid; i < per_slot; i += kDecThreads) mine[32 + i] = res[i];
        __threadfence();
        __syncthreads();
        if (tid == 0) ticket_sh = static_cast<int>(atomicAdd(&counters[bg], 1u));
        __syncthreads();
        if (ticket_sh != n_active - 1) return;
        __threadfence();
        if (tid == 0) counters[bg] = 0u;  // every workgroup of this call has arrived
        const float *all = parts + bg * a.n_splits * static_cast<size_t>(a.partial_floats);
        float *wgt = obuf;  // [n_active][16]
        if (tid < G) {
            float M = -INFINITY;
            for (int k = 0; k < n_active; ++k) M = fmaxf(M, all[k * static_cast<size_t>(a.partial_floats) + tid]);
            float Ls = 0.f;
            for (int k = 0; k < n_active; ++k) {
                const float* pk = all + k * static_cast<size_t>(a.partial_floats);
                const float w = __builtin_amdgcn_exp2f(pk[tid] - M);
                wgt[k * 16 + tid] = w;
                Ls += w * pk[16 + tid];
            }
            resL[tid] = Ls;
        }
        __syncthreads();
        for (int i = tid; i < per_slot; i += kDecThreads) {
            const int h = i / kDim;
            float acc = 0.f;
            for (int k = 0; k < n_active; ++k)
                acc += wgt[k * 16 + h] * all[k * static_cast<size_t>(a.partial_floats) + 32 + i];
            res[i] = acc;
        }
        __syncthreads();
    }

    // ---- inverse rotation and output: o = H O / (256 L)
    lds_fwht_rows(res, G, tid);
    for (int i = tid; i < per_slot; i += kDecThreads) {
        const int h = i / kDim;
        outp[i] = f32_to_bf16(res[i] * (1.0f / 256.0f) / resL[h]);
    }
}

hipError_t launch_decode(const DecodeParams &p, const DecodePlan &plan, hipStream_t stream) {
    DecodeArgs a;
    a.p = p;
    a.group = plan.group;
    a.n_splits = plan.n_splits;
    a.split_tiles = plan.split_tiles;
    a.partial_floats = static_cast<int32_t>(plan.partial_floats);
    const Codebook &cb = codebook();
    for (int k = 0; k < 8; ++k) {
        const _Float16 lo = static_cast<_Float16>(16.0f * cb.centroid[2 * k]);
        const _Float16 hi = static_cast<_Float16>(16.0f * cb.centroid[2 * k + 1]);
        a.lut_pairs[k] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
    }
    hipLaunchKernelGGL(tq4_decode_kernel, dim3(plan.n_splits, p.n_kv, p.batch), dim3(kDecThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tq4
