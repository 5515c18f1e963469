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
#include <type_traits>

#include "tq4_device.h"
#include "tq4_launch.h"

namespace tq4 {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kTile = 32;
constexpr int kLutEntries = 256;
constexpr int kLutWords = kLutEntries * kWave;  // 64 KiB
constexpr int kMaxSplits = 256;
constexpr int kPlanCUs = 256;       // MI355X compute units
constexpr int kPlanWgsPerCU = 1;    // resident decode workgroups per CU
constexpr int kMinTilesPerWave = 2;

struct DecodeArgs {
    DecodeParams p;
    int32_t group;
    int32_t n_splits;
    int32_t split_tiles;
    int32_t partial_floats;
    uint64_t parts_off;   // byte offset of the partials inside the workspace
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
    pl.counters_bytes = 0;
    pl.partial_floats = 32 + static_cast<size_t>(pl.group) * kDim;
    // one (M, L, O) partial per (request, KV head, split); nothing when there is a single split
    pl.workspace_bytes = pl.n_splits > 1 ? static_cast<size_t>(units) * pl.n_splits * pl.partial_floats * sizeof(float)
                                         : 0;
    return pl;
}

// ---------------------------------------------------------------- device helpers

// Registers of one 32-key tile held by a lane (lane = 16 * gq + n).
struct KRegs {
    u32x4 k[2][2];   // [M-tile][half]: words 16*half + 4*gq .. +3 of key 16*mt + n
    u32x2 kn[2];     // K norms of keys 4gq..4gq+3 and 16+4gq..16+4gq+3
};
struct VRegs {
    u32x2 v[8];      // words 2n, 2n+1 of key sigma(j) = j < 4 ? 4gq + j : 16 + 4gq + j - 4
    u32x2 vn[2];     // V norms of the same keys as kn
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

// First record of a tile (page `pid`, in-page offset of key0); page IDs outside the pool map to
// page 0 and the tile is masked.
__device__ __forceinline__ int64_t tile_rec0(const DecodeParams &p, int g, int key0, int pid, bool &valid) {
    const int page_idx = key0 / p.page_size;
    const int off0 = key0 - page_idx * p.page_size;
    valid = (pid >= 0 && pid < p.num_pages);
    if (!valid) pid = 0;
    return (static_cast<int64_t>(pid) * p.n_kv + g) * p.page_size + off0;
}

// Tile loads address a wave-uniform record base (scalar registers) plus fixed per-lane byte
// offsets, so each load is one instruction with no per-tile vector address arithmetic.
struct LaneOffsets {
    uint32_t k;   // (n * 32 + 4 * gq) words -> bytes; + 2048 per M-tile, + 64 per half
    uint32_t v;   // key 4gq, words 2n -> bytes; keys 4gq+j at + 128 j, keys 16+4gq+j at + 2048 + 128 j
    uint32_t nrm; // norms of key 4gq -> bytes; + 32 for keys 16+4gq..
};

__device__ __forceinline__ LaneOffsets lane_offsets(int lane) {
    const uint32_t n = lane & 15, gq = lane >> 4;
    return {n * 128u + gq * 16u, gq * 512u + n * 8u, gq * 8u};
}

__device__ __forceinline__ void load_k(const DecodeParams &p, int64_t rec0, const LaneOffsets &o, KRegs &t) {
    const char *wb = reinterpret_cast<const char *>(p.k_words) + rec0 * (kWords * 4);
    const char *nb = reinterpret_cast<const char *>(p.k_norms) + rec0 * 2;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h) t.k[mt][h] = *reinterpret_cast<const u32x4 *>(wb + o.k + (2048u * mt + 64u * h));
#pragma unroll
    for (int h = 0; h < 2; ++h) t.kn[h] = *reinterpret_cast<const u32x2 *>(nb + o.nrm + 32u * h);
}

__device__ __forceinline__ void load_v(const DecodeParams &p, int64_t rec0, const LaneOffsets &o, VRegs &t) {
    const char *wb = reinterpret_cast<const char *>(p.v_words) + rec0 * (kWords * 4);
    const char *nb = reinterpret_cast<const char *>(p.v_norms) + rec0 * 2;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t koff = (j < 4) ? 128u * j : 2048u + 128u * (j - 4);
        t.v[j] = *reinterpret_cast<const u32x2 *>(wb + o.v + koff);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) t.vn[h] = *reinterpret_cast<const u32x2 *>(nb + o.nrm + 32u * h);
}

// Unnormalised Hadamard transform of one 256-vector held by a wavefront, lane l holding dims
// 4l .. 4l+3: stages 1 and 2 in registers, stages 4 .. 128 pair lane l with lane l ^ (h / 4).
__device__ __forceinline__ void wave_fwht(float y[4], int lane) {
    {
        const float t0 = y[0] + y[1], t1 = y[0] - y[1], t2 = y[2] + y[3], t3 = y[2] - y[3];
        y[0] = t0 + t2;
        y[2] = t0 - t2;
        y[1] = t1 + t3;
        y[3] = t1 - t3;
    }
#pragma unroll
    for (int m = 1; m <= 32; m <<= 1) {
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float o = __shfl_xor(y[r], m, kWave);
            y[r] = upper ? (o - y[r]) : (y[r] + o);
        }
    }
}

// ---------------------------------------------------------------- split kernel

__global__ __launch_bounds__(kDecThreads) void tq4_decode_kernel(DecodeArgs a) {
    __shared__ __align__(16) uint32_t lut_mem[kLutWords];
    __shared__ __align__(16) half8 qop_sh[8][kWave];  // rotated-query MFMA operand per K-step and lane
    __shared__ float stat_m[kDecWaves][16];
    __shared__ float stat_l[kDecWaves][16];
    __shared__ float head_f[16];
    __shared__ float resM[16];
    __shared__ float resL[16];

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

    // ---- page IDs of this wave's tiles, 64 at a time in one VGPR (lane i: i-th tile of the chunk)
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int n_mine = wave_u < n_tiles ? (n_tiles - wave_u + kDecWaves - 1) / kDecWaves : 0;
    const int32_t *pt_row = p.page_table + static_cast<int64_t>(b) * p.table_stride;
    int pid_vec = 0;
    auto fetch_pids = [&](int chunk) {
        const int j = chunk * kWave + lane;
        const int tile = wave_u + j * kDecWaves;
        pid_vec = (j < n_mine) ? pt_row[(key_begin + tile * kTile) / p.page_size] : 0;
    };
    auto pid_of = [&](int j) -> int { return __builtin_amdgcn_readlane(pid_vec, j & (kWave - 1)); };

    const LaneOffsets lofs = lane_offsets(lane);
    auto rec_of = [&](int t, int inext, bool &valid_d) -> int64_t {
        const int key0 = __builtin_amdgcn_readfirstlane(key_begin + t * kTile);
        return tile_rec0(p, g, key0, pid_of(inext), valid_d);
    };

    // ---- start streaming before any set-up work: the first tile's loads fly during the prologue
    KRegs kr;
    VRegs vr;
    bool valid_cur = false, valid_next = false;
    int64_t rec_next = 0;
    if (n_mine > 0) {
        fetch_pids(0);
        rec_next = rec_of(wave_u, 0, valid_next);
        load_k(p, rec_next, lofs, kr);
        load_v(p, rec_next, lofs, vr);
    }

    // ---- prologue: zero the query operand, fill the centroid table, rotate the group's queries
    reinterpret_cast<u32x4 *>(&qop_sh[0][0])[tid] = u32x4{0u, 0u, 0u, 0u};  // 512 x 16 B
    // centroid table: entry e (a nibble pair) -> fp16x2 (16 c[e & 15], 16 c[e >> 4]); one copy per
    // lane, so a 256-byte row per entry, written 16 bytes at a time
    for (int i = tid; i < kLutWords / 4; i += kDecThreads) {
        const int e = i >> 4;
        const uint32_t lo = (a.lut_pairs[(e & 15) >> 1] >> (16 * (e & 1))) & 0xffffu;
        const uint32_t hi = (a.lut_pairs[(e >> 4) >> 1] >> (16 * ((e >> 4) & 1))) & 0xffffu;
        const uint32_t v = lo | (hi << 16);
        reinterpret_cast<u32x4 *>(lut_mem)[i] = u32x4{v, v, v, v};
    }
    __syncthreads();
    for (int h = wave; h < G; h += kDecWaves) {
        // one wavefront rotates query head h: y = H q (unnormalised), then a power-of-two scale
        // puts max |y| in [2^13, 2^14) for the fp16 operand
        const uint16_t *qh = p.q + ((static_cast<int64_t>(b) * p.n_q + static_cast<int64_t>(g) * G + h) * kDim);
        const u32x2 raw = *reinterpret_cast<const u32x2 *>(qh + 4 * lane);
        float y[4] = {__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                      __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
        wave_fwht(y, lane);
        float mx = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3])));
        for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, kWave));
        int e = 0;
        if (mx > 0.f) {
            int E;
            frexpf(mx, &E);
            e = 14 - E;
        }
        const float qs = ldexpf(1.0f, e);
        if (lane == 0) head_f[h] = p.scale * 1.4426950408889634f * ldexpf(1.0f, -e) * (1.0f / 256.0f);
        // dims 4l .. 4l+3 sit in word w = l / 2 at slots 4 (l & 1) ..; word w feeds K-step
        // 4 (w / 16) + (w & 3) in lane group (w / 4) & 3, column h
        const int w = lane >> 1;
        const int ks = 4 * (w >> 4) + (w & 3);
        const int dst_lane = 16 * ((w >> 2) & 3) + h;
        u32x2 hv;
        hv.x = pack_f16x2(y[0] * qs, y[1] * qs);
        hv.y = pack_f16x2(y[2] * qs, y[3] * qs);
        *reinterpret_cast<u32x2 *>(reinterpret_cast<char *>(&qop_sh[ks][dst_lane]) + 8 * (lane & 1)) = hv;
    }
    __syncthreads();
    const float fcol = (n < G) ? head_f[n] : 0.f;
    const char *lut = reinterpret_cast<const char *>(lut_mem);
    const uint32_t lane4 = static_cast<uint32_t>(lane) * 4u;

    float4v oacc[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) oacc[t] = float4v{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    // One tile per step, one register set refilled in place: the next tile's K is requested as
    // soon as this tile's scores exist, its V as soon as this tile's P.V products are issued.
    auto step = [&](int t, int inext, auto prefetch) {
        const int key0 = key_begin + t * kTile;
        const bool valid = valid_cur;
        // ---- scores S^T (rows: keys, columns: heads)
        float4v sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sacc[mt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const u32x4 kw = kr.k[mt][ks >> 2];
                const uint32_t w = (ks & 3) == 0 ? kw.x : (ks & 3) == 1 ? kw.y : (ks & 3) == 2 ? kw.z : kw.w;
                sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lut_decode(w, lane4, lut), qop_sh[ks][lane], sacc[mt], 0, 0, 0);
            }
        }
        // lane holds head n, keys sigma(j): j < 4 -> 4gq + j, else 16 + 4gq + j - 4
        float sc[8];
        const int lim = valid ? (key_end - key0) : 0;  // keys at tile offset >= lim are masked
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float kn4[4] = {f16lo(kr.kn[h].x), f16hi(kr.kn[h].x), f16lo(kr.kn[h].y), f16hi(kr.kn[h].y)};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int koff = 16 * h + 4 * gq + r;
                sc[4 * h + r] = (koff < lim) ? sacc[h][r] * kn4[r] * fcol : -INFINITY;
            }
        }
        if constexpr (decltype(prefetch)::value) {
            rec_next = rec_of(t + kDecWaves, inext, valid_next);
            __builtin_amdgcn_sched_barrier(0);
            load_k(p, rec_next, lofs, kr);
            __builtin_amdgcn_sched_barrier(0);
        }
        float mx = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sc[j]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        const float m_new = fmaxf(m_run, mx);
        // this lane's accumulators all belong to head n, so the rescale factor is lane-local
        const float alpha = (m_new > m_run) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) oacc[tt] *= alpha;
        float pv[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float nv4[4] = {f16lo(vr.vn[h].x), f16hi(vr.vn[h].x), f16lo(vr.vn[h].y), f16hi(vr.vn[h].y)};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float sj = sc[4 * h + r];
                const float e = (sj == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sj - m_run);
                l_run += e;
                pv[4 * h + r] = (n < G) ? e * nv4[r] : 0.f;
            }
        }
        u32x4 pr;
        pr.x = pack_f16x2(pv[0], pv[1]);
        pr.y = pack_f16x2(pv[2], pv[3]);
        pr.z = pack_f16x2(pv[4], pv[5]);
        pr.w = pack_f16x2(pv[6], pv[7]);
        const half8 pop = __builtin_bit_cast(half8, pr);
        // ---- O^T[dims][heads] += V^T P^T over two word columns (words 2n and 2n+1 of each key)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            uint32_t wv[8], u[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) wv[j] = c == 0 ? vr.v[j].x : vr.v[j].y;
            nibble_transpose8(wv, u);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                oacc[8 * c + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lut_decode(u[i], lane4, lut), pop, oacc[8 * c + i], 0, 0, 0);
        }
        if constexpr (decltype(prefetch)::value) {
            __builtin_amdgcn_sched_barrier(0);
            load_v(p, rec_next, lofs, vr);
            __builtin_amdgcn_sched_barrier(0);
        }
        valid_cur = valid_next;
    };

    // ---- main loop over chunks of 64 tiles; inside a chunk every load is unconditional (the
    // chunk's last tile is peeled), which keeps the wait counters exact
    for (int c0 = 0; c0 < n_mine; c0 += kWave) {
        const int cn = min(kWave, n_mine - c0);
        const int tc = wave_u + c0 * kDecWaves;  // first tile of the chunk
        if (c0 > 0) {
            fetch_pids(c0 / kWave);
            rec_next = rec_of(tc, 0, valid_next);
            load_k(p, rec_next, lofs, kr);
            load_v(p, rec_next, lofs, vr);
        }
        valid_cur = valid_next;
        for (int i = 0; i + 1 < cn; ++i) step(tc + i * kDecWaves, i + 1, std::true_type{});
        step(tc + (cn - 1) * kDecWaves, 0, std::false_type{});
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
    float *scratch = reinterpret_cast<float *>(lut_mem);
    float *obuf = scratch;                                 // [slots][G][256]
    const int per_slot = G * kDim;
    const int slots = (kLutWords - kDim * 16) / per_slot;  // the last 16 rows hold the result
    float *res = scratch + kLutWords - kDim * 16;           // [G][256] combined accumulator
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
            if (n < G) {
                const float mw = stat_m[wave][n];
                const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - resM[n]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int c = 0; c < 2; ++c)
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            dst[n * kDim + 8 * (2 * (4 * gq + r) + c) + i] = oacc[8 * c + i][r] * f;
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

    if (n_active > 1) {
        // more than one split: leave (M, L, O) for the combine kernel
        const size_t bg = static_cast<size_t>(b) * p.n_kv + g;
        float *dst = reinterpret_cast<float *>(static_cast<char *>(p.workspace) + a.parts_off) +
                     (bg * a.n_splits + s) * static_cast<size_t>(a.partial_floats);
        if (tid < G) {
            dst[tid] = resM[tid];
            dst[16 + tid] = resL[tid];
        }
        float4 *d4 = reinterpret_cast<float4 *>(dst + 32);
        const float4 *r4 = reinterpret_cast<const float4 *>(res);
        for (int i = tid; i < G * (kDim / 4); i += kDecThreads) d4[i] = r4[i];
        return;
    }

    // ---- single split: inverse rotation and output, o = H O / (256 L)
    for (int h = wave; h < G; h += kDecWaves) {
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = res[h * kDim + 4 * lane + r];
        wave_fwht(y, lane);
        const float Lh = resL[h];
        const float f = Lh > 0.f ? (1.0f / 256.0f) / Lh : 0.f;
        u32x2 o;
        o.x = static_cast<uint32_t>(f32_to_bf16(y[0] * f)) | (static_cast<uint32_t>(f32_to_bf16(y[1] * f)) << 16);
        o.y = static_cast<uint32_t>(f32_to_bf16(y[2] * f)) | (static_cast<uint32_t>(f32_to_bf16(y[3] * f)) << 16);
        *reinterpret_cast<u32x2 *>(outp + h * kDim + 4 * lane) = o;
    }
}

// ---------------------------------------------------------------- combine kernel
//
// One workgroup per (query head, KV head, request): merges the split partials of that head in
// fixed split order (max-rescaled sums), applies the inverse rotation and writes bf16.

constexpr int kCombThreads = 256;

__global__ __launch_bounds__(kCombThreads) void tq4_decode_combine_kernel(DecodeArgs a) {
    __shared__ float wgt[kMaxSplits];
    __shared__ float sL[kMaxSplits];
    __shared__ float row[kDim];
    __shared__ float totL;
    const DecodeParams &p = a.p;
    const int G = a.group;
    const int h = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int d = threadIdx.x;
    int L = p.seq_lens[b];
    L = L < 0 ? 0 : (L > p.max_seq_len ? p.max_seq_len : L);
    const int split_keys = a.split_tiles * kTile;
    const int n_active = (L + split_keys - 1) / split_keys;
    if (n_active <= 1) return;  // the split kernel wrote this output itself
    const size_t pf = static_cast<size_t>(a.partial_floats);
    const float *base = reinterpret_cast<const float *>(static_cast<const char *>(p.workspace) + a.parts_off) +
                        (static_cast<size_t>(b) * p.n_kv + g) * a.n_splits * pf;
    for (int k = d; k < n_active; k += kCombThreads) {
        wgt[k] = base[k * pf + h];
        sL[k] = base[k * pf + 16 + h];
    }
    __syncthreads();
    float M = -INFINITY;
    for (int k = 0; k < n_active; ++k) M = fmaxf(M, wgt[k]);
    __syncthreads();
    for (int k = d; k < n_active; k += kCombThreads)
        wgt[k] = (wgt[k] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(wgt[k] - M);
    __syncthreads();
    if (d == 0) {
        float t = 0.f;
        for (int k = 0; k < n_active; ++k) t += wgt[k] * sL[k];
        totL = t;
    }
    const float *col = base + 32 + h * kDim + d;
    float acc = 0.f;
    int k = 0;
    for (; k + 8 <= n_active; k += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = col[(k + u) * pf];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += wgt[k + u] * v[u];
    }
    for (; k < n_active; ++k) acc += wgt[k] * col[k * pf];
    row[d] = acc;
    __syncthreads();
    for (int hs = 1; hs < kDim; hs <<= 1) {
        float v = row[d];
        const float o = row[d ^ hs];
        __syncthreads();
        row[d] = (d & hs) ? (o - v) : (v + o);
        __syncthreads();
    }
    const float f = totL > 0.f ? (1.0f / 256.0f) / totL : 0.f;
    p.out[(static_cast<int64_t>(b) * p.n_q + static_cast<int64_t>(g) * G + h) * kDim + d] = f32_to_bf16(row[d] * f);
}

hipError_t launch_decode(const DecodeParams &p, const DecodePlan &plan, hipStream_t stream) {
    DecodeArgs a;
    a.p = p;
    a.group = plan.group;
    a.n_splits = plan.n_splits;
    a.split_tiles = plan.split_tiles;
    a.partial_floats = static_cast<int32_t>(plan.partial_floats);
    a.parts_off = plan.counters_bytes;
    const Codebook &cb = codebook();
    for (int k = 0; k < 8; ++k) {
        const _Float16 lo = static_cast<_Float16>(16.0f * cb.centroid[2 * k]);
        const _Float16 hi = static_cast<_Float16>(16.0f * cb.centroid[2 * k + 1]);
        a.lut_pairs[k] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
    }
    hipLaunchKernelGGL(tq4_decode_kernel, dim3(plan.n_splits, p.n_kv, p.batch), dim3(kDecThreads), 0, stream, a);
    if (plan.n_splits > 1)
        hipLaunchKernelGGL(tq4_decode_combine_kernel, dim3(plan.group, p.n_kv, p.batch), dim3(kCombThreads), 0,
                           stream, a);
    return hipGetLastError();
}

}  // namespace tq4
