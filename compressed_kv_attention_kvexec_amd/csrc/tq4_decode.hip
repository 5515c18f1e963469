// tq4_decode.hip -- decode attention directly on TQ4 pages, gfx950: one query token per request
// (decode) or its last n_queries tokens at once (the packed multi-query verifier).
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
// Work decomposition: grid (split, KV head, request).  The query rows of a KV head (G heads x
// n_queries tokens) are MFMA columns, 16 per block; a wavefront owns one block and every NS-th
// 32-key tile of its workgroup's range (decode: one block, 8 wavefronts).  Per tile and
// wavefront:
//   S^T[32 keys][16 rows] = K_tile . Q_rot^T   16 x v_mfma_f32_16x16x32_f16
//   online softmax in base 2 (key norms in the scores, value norms in P, a causal limit per row)
//   O^T[256][16 rows] += V_tile^T . P^T        16 x v_mfma_f32_16x16x32_f16
// Operand layouts and the centroid table are described in tq4_tile.h.  The
// workgroup merges its wavefronts in LDS; with several splits it leaves
// (max, sum, accumulator) in the workspace and tq4_decode_combine_kernel merges
// the splits in fixed order, applies the inverse rotation and writes bf16.
#include <cfloat>

#include "tq4_device.h"
#include "tq4_encode_wave.h"
#include "tq4_launch.h"
#include "tq4_tile.h"

namespace tq4 {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kMaxSplits = 256;
constexpr int kPlanCUs = 256;       // MI355X compute units
constexpr int kPlanWgsPerCU = 1;    // resident decode workgroups per CU
constexpr int kMinTilesPerWave = 1;
constexpr float kRescaleSlack = 8.0f;  // log2 headroom before the running maximum is moved
// Value-norm exponent eo of a wavefront (see the P operand below): kNormExpInit while no nonzero
// norm has been seen (every fp16 norm is >= 2^-24 or 0), at most kNormExpMax (a finite fp16 norm
// is below 2^16).
constexpr int kNormExpInit = -40;
constexpr int kNormExpMax = 9;

// eo for a largest value norm nmx (>= 0): nmx in [2^(eo + 6), 2^(eo + 7)); kNormExpInit for 0,
// kNormExpMax for +inf or NaN (a norm that overflowed fp16 on encoding, or unwritten bits).
__device__ __forceinline__ int norm_exponent(float nmx) {
    if (nmx == 0.f) return kNormExpInit;
    if (!(nmx <= 65504.f)) return kNormExpMax;
    int E;
    frexpf(nmx, &E);  // nmx in [2^(E-1), 2^E)
    return E - 7;
}

struct DecodeArgs {
    DecodeParams p;
    int32_t group;
    int32_t n_queries;  // query tokens per request (1: decode)
    int32_t rows;       // n_queries * group
    int32_t n_splits;
    int32_t split_tiles;
    int32_t partial_floats;
    uint64_t parts_off;   // byte offset of the partials inside the workspace
    uint32_t lut_pairs[8];  // fp16 bits of 16 * centroid[i], two per word (i = 2k, 2k+1)
    float thr[15];          // encoder thresholds (append path)
};

// ---------------------------------------------------------------- planning

DecodePlan plan_decode(int32_t batch, int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads, int32_t n_queries) {
    DecodePlan pl{};
    pl.group = n_q_heads / n_kv_heads;
    pl.n_queries = n_queries;
    pl.rows = n_queries * pl.group;
    pl.col_blocks = (pl.rows + 15) / 16;
    pl.slots = pl.col_blocks == 1 ? kDecWaves : kDecWaves / 2;  // tile slots per workgroup
    const int64_t tiles = (static_cast<int64_t>(max_seq_len) + kTile - 1) / kTile;
    const int64_t units = static_cast<int64_t>(batch) * n_kv_heads;
    int64_t want = (static_cast<int64_t>(kPlanCUs) * kPlanWgsPerCU + units - 1) / units;
    const int64_t cap = (tiles + pl.slots * kMinTilesPerWave - 1) / (pl.slots * kMinTilesPerWave);
    if (want > cap) want = cap;
    if (want > kMaxSplits) want = kMaxSplits;
    if (want < 1) want = 1;
    pl.split_tiles = static_cast<int32_t>((tiles + want - 1) / want);
    pl.n_splits = static_cast<int32_t>((tiles + pl.split_tiles - 1) / pl.split_tiles);
    pl.counters_bytes = 0;
    // per split: M[rows] and L[rows], each padded to kSplitStatPad floats, then O[rows][256]
    pl.partial_floats = 2 * kSplitStatPad + static_cast<size_t>(pl.rows) * kDim;
    // one partial per (request, KV head, split); nothing when there is a single split
    pl.workspace_bytes = pl.n_splits > 1 ? static_cast<size_t>(units) * pl.n_splits * pl.partial_floats * sizeof(float)
                                         : 0;
    return pl;
}

// ---------------------------------------------------------------- split kernel

// The query rows of one (request, KV head) -- row r = i G + h for query token i of n_queries and
// head h of the group -- fill NB blocks of 16 MFMA columns.  A workgroup has NS tile slots per
// block: wavefront w = blk NS + slot owns column block blk and every NS-th tile from its slot, so
// the NB wavefronts of a slot read the same tiles (one HBM read, the others hit the caches) and
// each keeps one block's 64 accumulators.  Decode is NB = 1, NS = 8 (two wavefronts per SIMD);
// the multi-query verifier uses NB = 2 or 3 with NS = 4 (two or three per SIMD).
//
// The leading scalar arguments repeat what the first loads need (the pool, the page table and
// its geometry): the library is built to preload them into scalar registers at wave launch, so
// the page-ID and first-tile requests do not wait for a read of the argument block.
template <int NB, int NS>
__global__ __launch_bounds__(NB * NS * kWave) void tq4_attn_split_kernel(
    const uint32_t *k_words, const uint32_t *v_words, const uint16_t *k_norms, const uint16_t *v_norms,
    const int32_t *page_table, int32_t table_stride, int32_t split_tiles, int32_t num_pages,
    uint32_t page_size_nkv, DecodeArgs a) {
    constexpr int NW = NB * NS;
    constexpr int NT = NW * kWave;
    constexpr int NCOL = 16 * NB;
    __shared__ __align__(16) uint32_t lut_mem[kLutWords];
    __shared__ __align__(16) half8 qop_sh[NB][8][kWave];  // rotated-query operand per block, K-step, lane
    __shared__ float stat_m[NW][16];
    __shared__ float stat_l[NW][16];
    __shared__ float row_f[NCOL];
    __shared__ float resM[NCOL];
    __shared__ float resL[NCOL];
    __shared__ int32_t progress[NW];  // tiles each wavefront has started

    DecodeParams p = a.p;
    p.k_words = k_words;
    p.v_words = v_words;
    p.k_norms = k_norms;
    p.v_norms = v_norms;
    p.page_table = page_table;
    p.table_stride = table_stride;
    p.num_pages = num_pages;
    p.page_size = static_cast<int32_t>(page_size_nkv & 0xffffu);
    p.n_kv = static_cast<int32_t>(page_size_nkv >> 16);
    const int G = a.group;
    const int KQ = a.n_queries;
    const int ROWS = a.rows;  // KQ * G <= NCOL
    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, gq = lane >> 4;

    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int slot = wave_u % NS, blk = wave_u / NS;
    const int split_keys = split_tiles * kTile;
    const int key_begin = s * split_keys;
    const int32_t *pt_row = p.page_table + static_cast<int64_t>(b) * p.table_stride;
    const bool append_mode = p.k_new != nullptr || p.v_new != nullptr;
    // element offset of query row r (token i, head h) in q and out: [request][token][q head][256]
    auto row_off = [&](int r) -> int64_t {
        const int i = r / G, h = r - i * G;
        return ((static_cast<int64_t>(b) * KQ + i) * p.n_q + static_cast<int64_t>(g) * G + h) * kDim;
    };

    // ---- page IDs of this wave's tiles, 64 at a time in one VGPR (lane i: i-th tile of the
    // chunk).  The table index is clamped into the row, so the load never depends on the
    // request's length and can fly alongside it; entries past the length are never used.
    int pid_vec = 0;
    auto fetch_pids = [&](int chunk) {
        const int tile = slot + (chunk * kWave + lane) * NS;
        pid_vec = pt_row[min((key_begin + tile * kTile) / p.page_size, p.table_stride - 1)];
    };
    auto pid_of = [&](int j) -> int { return __builtin_amdgcn_readlane(pid_vec, j & (kWave - 1)); };

    const LaneOffsets lofs = lane_offsets(lane);
    auto rec_of = [&](int t, int inext, bool &valid_d) -> int64_t {
        const int key0 = __builtin_amdgcn_readfirstlane(key_begin + t * kTile);
        return tile_rec0(p, g, key0, pid_of(inext), valid_d);
    };

    // One register set is refilled in place with the wavefront's next tile; a refill past the
    // chunk's end is a dead load of one line (every lane at the pool's first record) that is
    // never read.  It keeps every step's load count fixed, which keeps the compiler's wait counts
    // exact.
    KRegs kr;
    VRegs vr;
    bool valid_t = false;
    const LaneOffsets dead_ofs{0u, 0u, 0u};
    auto issue = [&](int t, int inext, bool live) {
        const int64_t rec = rec_of(t, inext, valid_t);
        const int64_t r = live ? rec : 0;
        const LaneOffsets o = live ? lofs : dead_ofs;
        __builtin_amdgcn_sched_barrier(0);  // same issue order on every path into the loop
        load_k(p, r, o, kr);
        __builtin_amdgcn_sched_barrier(0);
        load_v(p, r, o, vr);
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- start streaming before anything else: the query row of this wavefront's first column
    // (clamped: waves past the rows load a valid row and ignore it), the page IDs and the first
    // tile, all before the length is known.  A first tile past the length is a real but unused
    // load of a valid record.  Every path issues exactly these loads in this order, so the
    // compiler's wait counts stay exact through the prologue.
    fetch_pids(0);  // preloaded arguments only
    __builtin_amdgcn_sched_barrier(0);
    const int L_req = p.seq_lens[b];  // scalar load; used after the tile issue
    const u32x2 q_raw0 = *reinterpret_cast<const u32x2 *>(p.q + row_off(min(wave_u, ROWS - 1)) + 4 * lane);
    issue(slot, 0, true);

    const int L = L_req < 0 ? 0 : (L_req > p.max_seq_len ? p.max_seq_len : L_req);
    const int n_active = (L + split_keys - 1) / split_keys;
    if (s >= n_active) {
        if (L == 0 && s == 0)
            for (int i = tid; i < ROWS * kDim; i += NT) p.out[row_off(i / kDim) + (i % kDim)] = 0;
        return;
    }
    const int key_end = min(key_begin + split_keys, L);
    const int n_tiles = (key_end - key_begin + kTile - 1) / kTile;
    const int n_mine = slot < n_tiles ? (n_tiles - slot + NS - 1) / NS : 0;

    // ---- prologue: fill the centroid table and the rotated-query operand (each column written
    // once: query rows by the wavefront r % NW, padding columns zeroed), one barrier
    constexpr int kLutThreads = NT >= 1024 ? 1024 : (NT >= 512 ? 512 : 256);  // the first waves fill it
    if (tid < kLutThreads) build_lut<kLutThreads>(lut_mem, a.lut_pairs, tid);
    if (tid < NW) progress[tid] = 0;
    auto rotate_row = [&](int r, u32x2 raw) {
        // one wavefront rotates query row r: y = H q (unnormalised), then a power-of-two scale
        // puts max |y| in [2^13, 2^14) for the fp16 operand
        float y[4] = {__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                      __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
        wave_fwht(y, lane);
        float mx = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3])));
        mx = wave_max_f32(mx, lane);
        const int e = q_exponent(mx);
        const float qs = ldexpf(1.0f, e);
        if (lane == 0) row_f[r] = p.scale * 1.4426950408889634f * ldexpf(1.0f, -e) * (1.0f / 256.0f);
        // dims 4l .. 4l+3 sit in word w = l / 2 at slots 4 (l & 1) ..; word w feeds K-step
        // 4 (w / 16) + (w & 3) in lane group (w / 4) & 3, column r % 16 of block r / 16
        const int w = lane >> 1;
        const int ks = 4 * (w >> 4) + (w & 3);
        const int dst_lane = 16 * ((w >> 2) & 3) + (r & 15);
        u32x2 hv;
        hv.x = pack_f16x2(y[0] * qs, y[1] * qs);
        hv.y = pack_f16x2(y[2] * qs, y[3] * qs);
        *reinterpret_cast<u32x2 *>(reinterpret_cast<char *>(&qop_sh[r >> 4][ks][dst_lane]) + 8 * (lane & 1)) = hv;
    };
    auto zero_column = [&](int r) {  // 8 K-steps x 4 lane groups of 16 bytes
        if (lane < 32)
            reinterpret_cast<u32x4 *>(&qop_sh[r >> 4][lane & 7][16 * (lane >> 3) + (r & 15)])[0] = u32x4{0u, 0u, 0u, 0u};
    };
    if (wave_u < ROWS)
        rotate_row(wave_u, q_raw0);  // the row requested before the tiles
    else
        zero_column(wave_u);
    for (int r = wave_u + NW; r < NCOL; r += NW) {  // more columns than wavefronts
        if (r < ROWS)
            rotate_row(r, *reinterpret_cast<const u32x2 *>(p.q + row_off(r) + 4 * lane));
        else
            zero_column(r);
    }
    __syncthreads();

    // ---- append path (decode only): only the wavefront that owns the request's last tile ever
    // loads it, so that wavefront writes the new token's K and V records (position seq_len - 1)
    // here, before its loop; if its first tile, requested above, is that last tile, it requests it
    // again.
    if constexpr (NB == 1) {
        if (append_mode && s == n_active - 1 && n_tiles > 0 && slot == (n_tiles - 1) % NS) {
            const int slot_new = p.new_slots[b];
            if (slot_new >= 0 && slot_new < p.num_pages * p.page_size) {
                const int page = slot_new / p.page_size;
                const int64_t rec =
                    (static_cast<int64_t>(page) * p.n_kv + g) * p.page_size + (slot_new - page * p.page_size);
                const size_t off = (static_cast<size_t>(b) * p.n_kv + g) * kDim * (p.new_bf16 ? 2 : 4);
                float xk[4], xv[4];
                if (p.k_new != nullptr) encode_load(static_cast<const char *>(p.k_new) + off, p.new_bf16 != 0, lane, xk);
                if (p.v_new != nullptr) encode_load(static_cast<const char *>(p.v_new) + off, p.new_bf16 != 0, lane, xv);
                if (p.k_new != nullptr)
                    encode_values(xk, a.thr, const_cast<uint32_t *>(p.k_words) + rec * kWords,
                                  const_cast<uint16_t *>(p.k_norms) + rec, lane);
                if (p.v_new != nullptr)
                    encode_values(xv, a.thr, const_cast<uint32_t *>(p.v_words) + rec * kWords,
                                  const_cast<uint16_t *>(p.v_norms) + rec, lane);
            }
            // vmcnt(0): the record stores (and the stale first tile) have completed before the
            // wavefront loads the last tile (vmcnt bits [3:0] and [15:14] zero, expcnt and
            // lgkmcnt left at max)
            __builtin_amdgcn_s_waitcnt(0x0F70);
            if (n_mine == 1) issue(slot, 0, true);
        }
    }
    // this lane's column r = 16 blk + n: score factor and causal limit (visible keys: query token
    // i sees positions 0 .. L - KQ + i; padding columns see everything and are never written)
    const int col = 16 * blk + n;
    const float fcol = col < ROWS ? row_f[col] : 1.f;
    const int lim_col = col < ROWS ? L - KQ + col / G + 1 : L;
    const half8 *qop = &qop_sh[blk][0][lane];
    const char *lut = reinterpret_cast<const char *>(lut_mem);
    const uint32_t lane4 = static_cast<uint32_t>(lane) * 4u;

    float4v oacc[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) oacc[t] = float4v{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    // P operand range.  The products O^T += V^T P^T take p_j n_j (softmax weight times value
    // norm) as fp16.  p_j <= 2^kRescaleSlack, but an fp16 norm reaches 65504 and can be as small
    // as 2^-24, so the wavefront keeps l_run and oacc relative to 2^eo: its weights are
    // exp2(s_j - m_run - eo) and P_j = that times n_j.  eo is moved (rarely, in the same branch
    // that moves the running maximum) so every value norm seen is below 2^(eo + 7): P_j < 2^15
    // never overflows fp16, and a term whose norm is within 2^-20 of the largest seen is a normal
    // fp16 number.  The merge below returns l_run and oacc to their true scale (a power of two).
    int eo = kNormExpInit;
    // 2^(eo + 7) as fp32 bits: norms are nonnegative, so an unsigned compare of the bits orders them
    uint32_t n_hi_bits = static_cast<uint32_t>(kNormExpInit + 7 + 127) << 23;

    // One tile per step, its register set refilled in place with tile t + NS: the next K is
    // requested as soon as this tile's scores exist, the next V as soon as its P.V products are
    // issued.  live == false makes the refill a dead load (past the chunk's end).
    // Issue priority (two wavefronts per SIMD, w and w ^ 4): the pair has equal shares of tiles
    // but would be served oldest first, so the younger one would finish much later.  Each
    // wavefront publishes how many tiles it has started; the younger one takes the higher
    // priority while it is not ahead of its partner, the older one only while it is behind.
    // Tile assignment stays static, so results do not depend on timing.
    constexpr bool kPaired = NW == 8;
    const int partner = wave_u ^ (NW / 2);
    const bool younger = wave_u >= NW / 2;
    auto step = [&](int t, int inext, bool live, int done) {
        int other = 0;
        if constexpr (kPaired) {
            if (lane == 0) progress[wave_u] = done;
            other = __builtin_amdgcn_readfirstlane(progress[partner]);
        }
        const int key0 = key_begin + t * kTile;
        const bool valid = valid_t;
        // ---- scores S^T (rows: keys, columns: query rows)
        float4v sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sacc[mt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const u32x4 kw = kr.k[mt][ks >> 2];
                const uint32_t w = (ks & 3) == 0 ? kw.x : (ks & 3) == 1 ? kw.y : (ks & 3) == 2 ? kw.z : kw.w;
                const half8 kop = lut_decode(w, lane4, lut);
                sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[ks * kWave], sacc[mt], 0, 0, 0);
            }
        }
        // lane holds column n, keys sigma(j): j < 4 -> 4gq + j, else 16 + 4gq + j - 4
        float kn[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            kn[4 * h + 0] = f16lo(kr.kn[h].x);
            kn[4 * h + 1] = f16hi(kr.kn[h].x);
            kn[4 * h + 2] = f16lo(kr.kn[h].y);
            kn[4 * h + 3] = f16hi(kr.kn[h].y);
        }
        // x = (q_rot . c[idx]) n_k; the score in log2 units is fcol x.  Masked keys get -inf (below).
        float xs[8];
        const int lim = valid ? (min(key_end, lim_col) - key0) : 0;  // keys at offset >= lim are masked
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) xs[4 * h + r] = sacc[h][r] * kn[4 * h + r];
        const int64_t rec = rec_of(t + NS, inext, valid_t);
        const int64_t rec_pf = live ? rec : 0;
        const LaneOffsets ofs_pf = live ? lofs : dead_ofs;
        __builtin_amdgcn_sched_barrier(0);
        load_k(p, rec_pf, ofs_pf, kr);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kPaired) {
            if (younger ? (done <= other) : (done < other))
                __builtin_amdgcn_s_setprio(1);
            else
                __builtin_amdgcn_s_setprio(0);
        }
        float nv[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            nv[4 * h + 0] = f16lo(vr.vn[h].x);
            nv[4 * h + 1] = f16hi(vr.vn[h].x);
            nv[4 * h + 2] = f16lo(vr.vn[h].y);
            nv[4 * h + 3] = f16hi(vr.vn[h].y);
        }
        // Masking, only for tiles some column does not see in full (in place, so the common path
        // has no copies): score -inf, and value norm 0, since a masked key's record (past the
        // length, or never written) may hold any bits and exp2(-inf) * NaN would not be 0.
        if (!__all(lim >= kTile)) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if ((j < 4 ? 4 * gq + j : 12 + 4 * gq + j) >= lim) {
                    xs[j] = -INFINITY;
                    nv[j] = 0.f;
                }
        }
        float mx = xs[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, xs[j]);
        float lo, hi;  // column n's maximum over the four lane groups
        lane_pair<16>(mx, lo, hi);
        mx = fmaxf(lo, hi);
        lane_pair<32>(mx, lo, hi);
        mx = fmaxf(lo, hi) * fcol;  // fcol > 0
        // the largest value norm this lane's column sees in the tile
        const float nmx = fmaxf(fmaxf(fmaxf(nv[0], nv[1]), fmaxf(nv[2], nv[3])), fmaxf(fmaxf(nv[4], nv[5]), fmaxf(nv[6], nv[7])));
        const bool norm_up = __float_as_uint(nmx) >= n_hi_bits;
        // The reference maximum moves only when a score exceeds it by more than kRescaleSlack (so
        // exp2(s - m_run) <= 256): the softmax does not depend on the reference, and rescaling
        // the 64 accumulators becomes rare.  This lane's accumulators all belong to column n, so
        // the rescale factor is lane-local.  The same rare branch moves eo.
        if (__any(mx > m_run + kRescaleSlack || norm_up)) {
            float f = 1.0f;
            if (__any(norm_up)) {
                // a value norm at or above 2^(eo + 7): move eo so the wavefront's largest norm of
                // the tile is in [2^(eo + 6), 2^(eo + 7)); the sums scale by the power of two
                const int ne = norm_exponent(__uint_as_float(wave_max_u32(__float_as_uint(nmx), lane)));
                const int eo_new = __builtin_amdgcn_readfirstlane(min(max(ne, eo + 1), kNormExpMax));
                f = ldexpf(1.0f, eo - eo_new);
                eo = eo_new;
                n_hi_bits = static_cast<uint32_t>(eo + 7 + 127) << 23;
            }
            const float m_new = fmaxf(m_run, mx);
            const float alpha = ((m_new > m_run) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f) * f;
            l_run *= alpha;
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) oacc[tt] *= alpha;
            m_run = m_new;
        }
        // m_run is -inf only while every key of the column so far was masked; the floor keeps
        // fcol x - m finite or -inf then, and exp2(-inf) = 0 drops masked keys
        const float neg_m = -fmaxf(m_run, -FLT_MAX) - static_cast<float>(eo);
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(xs[j], fcol, neg_m));
            l_run += e;
            pv[j] = e * nv[j];
        }
        u32x4 pr;
        pr.x = pack_f16x2(pv[0], pv[1]);
        pr.y = pack_f16x2(pv[2], pv[3]);
        pr.z = pack_f16x2(pv[4], pv[5]);
        pr.w = pack_f16x2(pv[6], pv[7]);
        const half8 pop = __builtin_bit_cast(half8, pr);
        // ---- O^T[dims][columns] += V^T P^T over two word columns (words 2n and 2n+1 of each key)
#pragma unroll
        for (int cw = 0; cw < 2; ++cw) {
            uint32_t wv[8], u[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) wv[j] = cw == 0 ? vr.v[j].x : vr.v[j].y;
            nibble_transpose8(wv, u);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const half8 vop = lut_decode(u[i], lane4, lut);
                oacc[8 * cw + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop, oacc[8 * cw + i], 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        load_v(p, rec_pf, ofs_pf, vr);
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- main loop over chunks of 64 tiles (one VGPR of page IDs)
    for (int c0 = 0; c0 < n_mine; c0 += kWave) {
        const int cn = min(kWave, n_mine - c0);
        const int tc = slot + c0 * NS;  // first tile of the chunk
        if (c0 > 0) {
            fetch_pids(c0 / kWave);
            issue(tc, 0, true);
        }
        for (int i = 0; i < cn; ++i) step(tc + i * NS, i + 1, i + 1 < cn, c0 + i);
    }
    if constexpr (kPaired) __builtin_amdgcn_s_setprio(0);

    // ---- per-wave softmax totals (the statistics live outside the table, so they are written
    // before the barrier that retires the table).  These two exchanges go through the LDS
    // crossbar: their lane-swap form needs two more registers here, where every accumulator is
    // live, and spills in the three-block verifier.
    float l_tot = l_run + __shfl_xor(l_run, 16, kWave);
    l_tot = ldexpf(l_tot + __shfl_xor(l_tot, 32, kWave), eo);  // true scale: relative to m_run
    if (gq == 0) {
        stat_m[wave][n] = m_run;
        stat_l[wave][n] = l_tot;
    }
    __syncthreads();  // table no longer needed; statistics visible

    // LDS rows of 64 float4 quads of dims, quads swizzled within groups of 8 so that both the
    // accumulator scatter (lanes (gq, n) -> row n, quad 16 gq + ...) and row reads spread over
    // the banks
    auto quad_at = [](int h, int qd) { return h * 64 + (qd ^ ((h + 2 * (qd >> 4)) & 7)); };
    const size_t bg = static_cast<size_t>(b) * p.n_kv + g;
    float *dst = reinterpret_cast<float *>(static_cast<char *>(p.workspace) + a.parts_off) +
                 (bg * a.n_splits + s) * static_cast<size_t>(a.partial_floats);
    float4v *res4;  // single split: the merged rows [ROWS][64 quads] for the inverse rotation

    if constexpr (NB == 1) {
        // ---- merge the 8 waves in one round.  Every lane takes its column's maximum M and sum
        // over the waves; each wave writes its rows scaled to M (and back from 2^eo) into its own
        // LDS slot, and thread (row, quad) adds the 8 slots in a fixed order (the pairing of a
        // binary tree: slots s and s + 4, then + 2, then + 1), with all 8 reads in flight.
        // Rows go in passes of kMergeRows (6 x 8 slots x 1 KiB = 48 KiB of the table's space; the
        // merged rows of a single split take the last 16 KiB).
        constexpr int kMergeRows = 6;
        static_assert(NS == 8, "the one-round merge adds 8 slots");
        float mj[NS], lj[NS];
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            mj[j] = stat_m[j][n];
            lj[j] = stat_l[j][n];
        }
        float M = -INFINITY;
#pragma unroll
        for (int j = 0; j < NS; ++j) M = fmaxf(M, mj[j]);
        float Ls = 0.f;
#pragma unroll
        for (int j = 0; j < NS; ++j) Ls += (mj[j] == -INFINITY) ? 0.f : lj[j] * __builtin_amdgcn_exp2f(mj[j] - M);
        if (wave_u == 0 && lane < ROWS) {  // lane < 16: column n = lane
            resL[lane] = Ls;
            if (n_active > 1) {
                dst[lane] = M;
                dst[kSplitStatPad + lane] = Ls;
            }
        }
        const float f = (m_run == -INFINITY) ? 0.f : ldexpf(__builtin_amdgcn_exp2f(m_run - M), eo);
        float4v *slots4 = reinterpret_cast<float4v *>(lut_mem);
        res4 = slots4 + NS * kMergeRows * 64;
        for (int r0 = 0; r0 < ROWS; r0 += kMergeRows) {
            const int rp = min(kMergeRows, ROWS - r0);
            if (col >= r0 && col < r0 + rp) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int c = 0; c < 2; ++c)
#pragma unroll
                        for (int hf = 0; hf < 2; ++hf) {
                            const int qd = 16 * gq + 4 * r + 2 * c + hf;
                            const int t = 8 * c + 4 * hf;
                            slots4[wave_u * (kMergeRows * 64) + quad_at(col - r0, qd)] =
                                float4v{oacc[t][r] * f, oacc[t + 1][r] * f, oacc[t + 2][r] * f, oacc[t + 3][r] * f};
                        }
            }
            __syncthreads();
            if (tid < rp * 64) {
                const int rr = tid >> 6, qd = tid & 63;
                float4v v[NS];
#pragma unroll
                for (int j = 0; j < NS; ++j) v[j] = slots4[j * (kMergeRows * 64) + quad_at(rr, qd)];
                const float4v sum = ((v[0] + v[4]) + (v[2] + v[6])) + ((v[1] + v[5]) + (v[3] + v[7]));
                if (n_active > 1)
                    *reinterpret_cast<float4v *>(dst + 2 * kSplitStatPad + (r0 + rr) * kDim + 4 * qd) = sum;
                else
                    res4[quad_at(r0 + rr, qd)] = sum;
            }
            if (n_active > 1 && r0 + kMergeRows >= ROWS) return;  // partial stored, no LDS reuse follows
            __syncthreads();
        }
    } else {
        // ---- merge the waves of each block.  Each lane rescales its accumulators (all of column
        // n) to the block's maximum over its waves (and back from 2^eo); then a fixed-order tree in
        // LDS adds slots NS/2 .. NS-1 into 0 .. NS/2-1, and so on down to slot 0.  The LDS image
        // keeps the accumulator lane layout ([block][slot][register][lane] as 16-byte rows), so
        // every access is conflict-free.  kTreeBlocks blocks fit the table's 64 KiB at once.
        {
            float M = -INFINITY;
#pragma unroll
            for (int j = 0; j < NS; ++j) M = fmaxf(M, stat_m[blk * NS + j][n]);
            const float f = (m_run == -INFINITY) ? 0.f : ldexpf(__builtin_amdgcn_exp2f(m_run - M), eo);
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) oacc[tt] *= f;
        }
        if (tid < NCOL) {
            const int cb = tid >> 4, cn = tid & 15;
            float M = -INFINITY;
            for (int j = 0; j < NS; ++j) M = fmaxf(M, stat_m[cb * NS + j][cn]);
            float Ls = 0.f;
            for (int j = 0; j < NS; ++j) {
                const float mj = stat_m[cb * NS + j][cn];
                Ls += (mj == -INFINITY) ? 0.f : stat_l[cb * NS + j][cn] * __builtin_amdgcn_exp2f(mj - M);
            }
            resM[tid] = M;
            resL[tid] = Ls;
        }
        float4v *tree = reinterpret_cast<float4v *>(lut_mem);
        constexpr int kTreeBlocks = (NS >= 2) ? 8 / NS : NB;  // blocks per round: [blocks][NS/2][16][64] rows
#pragma unroll
        for (int b0 = 0; b0 < NB; b0 += kTreeBlocks) {
            const bool mine = blk >= b0 && blk < b0 + kTreeBlocks;
#pragma unroll
            for (int half = NS / 2; half >= 1; half >>= 1) {
                // only lanes of query-row columns take part (padding columns are never written out)
                if (mine && slot >= half && slot < 2 * half && col < ROWS) {
#pragma unroll
                    for (int tt = 0; tt < 16; ++tt)
                        tree[(((blk - b0) * (NS / 2) + slot - half) * 16 + tt) * kWave + lane] = oacc[tt];
                }
                __syncthreads();
                if (mine && slot < half && col < ROWS) {
#pragma unroll
                    for (int tt = 0; tt < 16; ++tt)
                        oacc[tt] += tree[(((blk - b0) * (NS / 2) + slot) * 16 + tt) * kWave + lane];
                }
                __syncthreads();
            }
        }

        if (n_active > 1) {
            // more than one split: the slot-0 wave of each block leaves its rows of
            // (M[rows], L[rows], O[rows][256]) for the combine kernel; lane (gq, n) holds dims
            // 8 (2 (4 gq + r) + c) + i of column n in oacc[8 c + i][r]
            if (wave_u == 0 && lane < ROWS) {
                dst[lane] = resM[lane];
                dst[kSplitStatPad + lane] = resL[lane];
            }
            if (slot == 0 && col < ROWS) {
                float *row = dst + 2 * kSplitStatPad + col * kDim;
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        const int d0 = 8 * (2 * (4 * gq + r) + c);
                        *reinterpret_cast<float4 *>(row + d0) =
                            make_float4(oacc[8 * c][r], oacc[8 * c + 1][r], oacc[8 * c + 2][r], oacc[8 * c + 3][r]);
                        *reinterpret_cast<float4 *>(row + d0 + 4) =
                            make_float4(oacc[8 * c + 4][r], oacc[8 * c + 5][r], oacc[8 * c + 6][r], oacc[8 * c + 7][r]);
                    }
            }
            return;
        }

        // single split: the slot-0 waves write O to LDS as [row][64 quads of dims]
        res4 = tree;
        if (slot == 0 && col < ROWS) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        const int qd = 16 * gq + 4 * r + 2 * c + hf;
                        res4[quad_at(col, qd)] = float4v{oacc[8 * c + 4 * hf][r], oacc[8 * c + 4 * hf + 1][r],
                                                         oacc[8 * c + 4 * hf + 2][r], oacc[8 * c + 4 * hf + 3][r]};
                    }
        }
        __syncthreads();
    }

    // ---- single split: one wave per row applies the inverse rotation, o = H O / (256 L)
    for (int r = wave_u; r < ROWS; r += NW) {
        const float4v v = res4[quad_at(r, lane)];
        float y[4] = {v[0], v[1], v[2], v[3]};
        wave_fwht(y, lane);
        const float Lh = resL[r];
        const float f = Lh > 0.f ? (1.0f / 256.0f) / Lh : 0.f;
        u32x2 o;
        o.x = static_cast<uint32_t>(f32_to_bf16(y[0] * f)) | (static_cast<uint32_t>(f32_to_bf16(y[1] * f)) << 16);
        o.y = static_cast<uint32_t>(f32_to_bf16(y[2] * f)) | (static_cast<uint32_t>(f32_to_bf16(y[3] * f)) << 16);
        *reinterpret_cast<u32x2 *>(p.out + row_off(r) + 4 * lane) = o;
    }
}

// ---------------------------------------------------------------- combine kernel
//
// One workgroup of four wavefronts per (query row, KV head, request) merges the split partials
// of that row: every wavefront reduces the splits' maxima in registers (lane i holds split
// 64 c + i), then wavefront w sums splits w, w + 4, ... for dims 4 l .. 4 l + 3 in lane l (16-byte
// loads), and wavefront 0 adds the four sums in fixed order, applies the inverse rotation and
// writes bf16.

constexpr int kCombWaves = 4;
constexpr int kCombThreads = kCombWaves * kWave;
constexpr int kCombPerWave = kWave / kCombWaves;  // splits per wavefront in each group of 64

// The leading scalar arguments repeat what the first loads need, preloaded into scalar registers
// at wave launch as in the split kernel.
template <bool kRotated>
__global__ __launch_bounds__(kCombThreads) void tq4_decode_combine_kernel(const float *parts, const int32_t *seq_lens,
                                                                          int32_t n_splits, int32_t partial_floats,
                                                                          int32_t n_kv, CombineArgs a) {
    __shared__ float4v part[kCombWaves][kWave];
    const int G = a.group;
    const int r = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int L_req = seq_lens[b];
    const size_t pf = static_cast<size_t>(partial_floats);
    const float *base = parts + (static_cast<size_t>(b) * n_kv + g) * n_splits * pf;
    const float *mrow = base + r;
    const float *lrow = base + kSplitStatPad + r;
    const float *orow = base + 2 * kSplitStatPad + static_cast<size_t>(r) * kDim + 4 * lane;
    const int ns = n_splits;
    // Every load of the first group of 64 splits is issued before the length is known (slots past
    // the live splits hold stale data and are dropped by selection, never multiplied in).
    const int s_l = min(lane, ns - 1);
    const float m0 = mrow[s_l * pf];
    const float l0 = lrow[s_l * pf];
    float4v v[kCombPerWave];
#pragma unroll
    for (int u = 0; u < kCombPerWave; ++u) {
        const int s = min(wave + kCombWaves * u, ns - 1);
        v[u] = *reinterpret_cast<const float4v *>(orow + s * pf);
    }
    const int L = L_req < 0 ? 0 : (L_req > a.max_seq_len ? a.max_seq_len : L_req);
    const int split_keys = a.split_tiles * kTile;
    const int n_active = (L + split_keys - 1) / split_keys;
    // With one live split the split kernel wrote this output itself; such a request still runs
    // the (harmless, in-bounds) arithmetic below but stores nothing.  An early return here would
    // let the compiler sink the loads above behind the length's own load.
    const bool merge = n_active > 1;
    const int n_groups = (n_active + kWave - 1) / kWave;

    // maximum over the live splits' reference maxima
    float mx = lane < n_active ? m0 : -INFINITY;
    for (int c = 1; c < n_groups; ++c) {
        const int s = c * kWave + lane;
        if (s < n_active) mx = fmaxf(mx, mrow[s * pf]);
    }
    const float M = wave_max_f32(mx, lane);

    auto weight = [&](float m) { return m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M); };
    float w_l = lane < n_active ? weight(m0) : 0.f;  // lane i: weight of split i
    float lsum = lane < n_active ? w_l * l0 : 0.f;
    float4v acc = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kCombPerWave; ++u) {
        const int s = wave + kCombWaves * u;
        if (s < n_active) acc += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w_l), s)) * v[u];
    }
    for (int c = 1; c < n_groups; ++c) {  // more than 64 splits
        const int s = c * kWave + lane;
        const float mc = s < n_active ? mrow[s * pf] : -INFINITY;
        const float wc = s < n_active ? weight(mc) : 0.f;
        lsum += s < n_active ? wc * lrow[s * pf] : 0.f;
        for (int u = 0; u < kCombPerWave; ++u) {
            const int s2 = c * kWave + wave + kCombWaves * u;
            if (s2 < n_active) {
                const float ws = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wc), wave + kCombWaves * u));
                acc += ws * *reinterpret_cast<const float4v *>(orow + s2 * pf);
            }
        }
    }
    const float Ltot = wave_sum_f32(lsum, lane);
    part[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && merge) {
        const float4v t = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
        float y[4] = {t[0], t[1], t[2], t[3]};
        float f = Ltot > 0.f ? 1.0f / Ltot : 0.f;
        if constexpr (kRotated) {  // o = H O / (256 L)
            wave_fwht(y, lane);
            f *= 1.0f / 256.0f;
        }
        u32x2 o;
        o.x = static_cast<uint32_t>(f32_to_bf16(y[0] * f)) | (static_cast<uint32_t>(f32_to_bf16(y[1] * f)) << 16);
        o.y = static_cast<uint32_t>(f32_to_bf16(y[2] * f)) | (static_cast<uint32_t>(f32_to_bf16(y[3] * f)) << 16);
        const int i = r / G, h = r - i * G;
        *reinterpret_cast<u32x2 *>(
            a.out + ((static_cast<int64_t>(b) * a.n_queries + i) * a.n_q + static_cast<int64_t>(g) * G + h) * kDim +
            4 * lane) = o;
    }
}

hipError_t launch_split_combine(const CombineArgs &c, bool rotated, hipStream_t stream) {
    const dim3 grid(c.rows, c.n_kv, c.batch);
    if (rotated)
        hipLaunchKernelGGL(tq4_decode_combine_kernel<true>, grid, dim3(kCombThreads), 0, stream, c.parts, c.seq_lens,
                           c.n_splits, c.partial_floats, c.n_kv, c);
    else
        hipLaunchKernelGGL(tq4_decode_combine_kernel<false>, grid, dim3(kCombThreads), 0, stream, c.parts, c.seq_lens,
                           c.n_splits, c.partial_floats, c.n_kv, c);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams &p, const DecodePlan &plan, hipStream_t stream) {
    DecodeArgs a;
    a.p = p;
    a.group = plan.group;
    a.n_queries = plan.n_queries;
    a.rows = plan.rows;
    a.n_splits = plan.n_splits;
    a.split_tiles = plan.split_tiles;
    a.partial_floats = static_cast<int32_t>(plan.partial_floats);
    a.parts_off = plan.counters_bytes;
    lut_pairs_from_codebook(a.lut_pairs, codebook().centroid);
    for (int i = 0; i < 15; ++i) a.thr[i] = codebook().threshold[i];
    const dim3 grid(plan.n_splits, p.n_kv, p.batch);
    const uint32_t ps_nkv = static_cast<uint32_t>(p.page_size) | (static_cast<uint32_t>(p.n_kv) << 16);
#define TQ4_SPLIT_ARGS                                                                                   \
    p.k_words, p.v_words, p.k_norms, p.v_norms, p.page_table, p.table_stride, plan.split_tiles, p.num_pages, \
        ps_nkv, a
    switch (plan.col_blocks) {
        case 1:
            hipLaunchKernelGGL((tq4_attn_split_kernel<1, 8>), grid, dim3(8 * kWave), 0, stream, TQ4_SPLIT_ARGS);
            break;
        case 2:
            hipLaunchKernelGGL((tq4_attn_split_kernel<2, 4>), grid, dim3(8 * kWave), 0, stream, TQ4_SPLIT_ARGS);
            break;
        case 3:
            hipLaunchKernelGGL((tq4_attn_split_kernel<3, 4>), grid, dim3(12 * kWave), 0, stream, TQ4_SPLIT_ARGS);
            break;
        default:
            return hipErrorInvalidValue;
    }
#undef TQ4_SPLIT_ARGS
    if (plan.n_splits > 1) {
        CombineArgs c;
        c.parts = reinterpret_cast<const float *>(static_cast<const char *>(p.workspace) + plan.counters_bytes);
        c.seq_lens = p.seq_lens;
        c.out = p.out;
        c.max_seq_len = p.max_seq_len;
        c.split_tiles = plan.split_tiles;
        c.n_splits = plan.n_splits;
        c.partial_floats = static_cast<int32_t>(plan.partial_floats);
        c.rows = plan.rows;
        c.group = plan.group;
        c.n_queries = plan.n_queries;
        c.n_q = p.n_q;
        c.n_kv = p.n_kv;
        c.batch = p.batch;
        return launch_split_combine(c, true, stream);
    }
    return hipGetLastError();
}

}  // namespace tq4
