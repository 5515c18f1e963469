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
// workgroup; a wavefront owns every 8th 32-key tile of its workgroup's range.
// Per tile and wavefront (GQA group of G <= 16 query heads padded to 16):
//   S^T[32 keys][16 heads] = K_tile . Q_rot^T   16 x v_mfma_f32_16x16x32_f16
//   online softmax in base 2 (key norms in the scores, value norms in P)
//   O^T[256][16 heads] += V_tile^T . P^T        16 x v_mfma_f32_16x16x32_f16
// Operand layouts and the centroid table are described in tq4_tile.h.  The
// workgroup merges its wavefronts in LDS; with several splits it leaves
// (max, sum, accumulator) in the workspace and tq4_decode_combine_kernel merges
// the splits in fixed order, applies the inverse rotation and writes bf16.
#include <type_traits>

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
constexpr int kMinTilesPerWave = 2;
constexpr float kRescaleSlack = 8.0f;  // log2 headroom before the running maximum is moved

struct DecodeArgs {
    DecodeParams p;
    int32_t group;
    int32_t n_splits;
    int32_t split_tiles;
    int32_t partial_floats;
    uint64_t parts_off;   // byte offset of the partials inside the workspace
    uint32_t lut_pairs[8];  // fp16 bits of 16 * centroid[i], two per word (i = 2k, 2k+1)
    float thr[15];          // encoder thresholds (append path)
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

// ---------------------------------------------------------------- split kernel

__global__ __launch_bounds__(kDecThreads) void tq4_decode_kernel(DecodeArgs a) {
    __shared__ __align__(16) uint32_t lut_mem[kLutWords];
    __shared__ __align__(16) half8 qop_sh[8][kWave];  // rotated-query MFMA operand per K-step and lane
    __shared__ float stat_m[kDecWaves][16];
    __shared__ float stat_l[kDecWaves][16];
    __shared__ float head_f[16];
    __shared__ float resM[16];
    __shared__ float resL[16];
    __shared__ int32_t progress[kDecWaves];  // tiles each wavefront has started

    const DecodeParams &p = a.p;
    const int G = a.group;
    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, gq = lane >> 4;

    const int L_req = p.seq_lens[b];  // scalar load, requested first; used after the tile issue
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int split_keys = a.split_tiles * kTile;
    const int key_begin = s * split_keys;
    const int32_t *pt_row = p.page_table + static_cast<int64_t>(b) * p.table_stride;
    const bool append_mode = p.k_new != nullptr || p.v_new != nullptr;

    // ---- page IDs of this wave's tiles, 64 at a time in one VGPR (lane i: i-th tile of the
    // chunk).  The table index is clamped into the row, so the load never depends on the
    // request's length and can fly alongside it; entries past the length are never used.
    int pid_vec = 0;
    auto fetch_pids = [&](int chunk) {
        const int tile = wave_u + (chunk * kWave + lane) * kDecWaves;
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

    // ---- start streaming before anything else: the query row of this wavefront's first head
    // (clamped: waves past the group load a valid row and ignore it), the page IDs and the first
    // tile, all before the length is known.  A first tile past the length is a real but unused
    // load of a valid record.  Every path issues exactly these loads in this order, so the
    // compiler's wait counts stay exact through the prologue.
    const int q_h0 = min(wave_u, G - 1);
    const u32x2 q_raw0 = *reinterpret_cast<const u32x2 *>(
        p.q + (static_cast<int64_t>(b) * p.n_q + static_cast<int64_t>(g) * G + q_h0) * kDim + 4 * lane);
    fetch_pids(0);
    issue(wave_u, 0, true);

    const int L = L_req < 0 ? 0 : (L_req > p.max_seq_len ? p.max_seq_len : L_req);
    const int n_active = (L + split_keys - 1) / split_keys;
    uint16_t *outp = p.out + (static_cast<int64_t>(b) * p.n_q + static_cast<int64_t>(g) * G) * kDim;
    if (s >= n_active) {
        if (L == 0 && s == 0)
            for (int i = tid; i < G * kDim; i += kDecThreads) outp[i] = 0;
        return;
    }
    const int key_end = min(key_begin + split_keys, L);
    const int n_tiles = (key_end - key_begin + kTile - 1) / kTile;
    const int n_mine = wave_u < n_tiles ? (n_tiles - wave_u + kDecWaves - 1) / kDecWaves : 0;

    // ---- prologue: fill the centroid table and the rotated-query operand (each column written
    // once: query heads by their wavefront, padding columns zeroed), one barrier
    build_lut<kDecThreads>(lut_mem, a.lut_pairs, tid);
    if (tid < kDecWaves) progress[tid] = 0;
    auto rotate_head = [&](int h, u32x2 raw) {
        // one wavefront rotates query head h: y = H q (unnormalised), then a power-of-two scale
        // puts max |y| in [2^13, 2^14) for the fp16 operand
        float y[4] = {__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                      __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
        wave_fwht(y, lane);
        float mx = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3])));
        for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, kWave));
        const int e = q_exponent(mx);
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
    };
    auto zero_column = [&](int c) {  // 8 K-steps x 4 lane groups of 16 bytes
        if (lane < 32) reinterpret_cast<u32x4 *>(&qop_sh[lane & 7][16 * (lane >> 3) + c])[0] = u32x4{0u, 0u, 0u, 0u};
    };
    if (wave_u < G)
        rotate_head(wave_u, q_raw0);  // the row requested before the tiles
    else
        zero_column(wave_u);
    if (wave_u + kDecWaves < G)  // groups of more than 8 heads
        rotate_head(wave_u + kDecWaves,
                    *reinterpret_cast<const u32x2 *>(p.q + (static_cast<int64_t>(b) * p.n_q +
                                                            static_cast<int64_t>(g) * G + wave_u + kDecWaves) * kDim +
                                                     4 * lane));
    else
        zero_column(wave_u + kDecWaves);
    __syncthreads();

    // ---- append path: only the wavefront that owns the request's last tile ever loads it, so
    // that wavefront writes the new token's K and V records (position seq_len - 1) here, before
    // its loop; if its first tile, requested above, is that last tile, it requests it again.
    if (append_mode && s == n_active - 1 && n_tiles > 0 && wave_u == (n_tiles - 1) % kDecWaves) {
        const int slot = p.new_slots[b];
        if (slot >= 0 && slot < p.num_pages * p.page_size) {
            const int page = slot / p.page_size;
            const int64_t rec = (static_cast<int64_t>(page) * p.n_kv + g) * p.page_size + (slot - page * p.page_size);
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
        // wavefront loads the last tile (vmcnt bits [3:0] and [15:14] zero, expcnt and lgkmcnt
        // left at max)
        __builtin_amdgcn_s_waitcnt(0x0F70);
        if (n_mine == 1) issue(wave_u, 0, true);
    }
    const float fcol = (n < G) ? head_f[n] : 0.f;
    const char *lut = reinterpret_cast<const char *>(lut_mem);
    const uint32_t lane4 = static_cast<uint32_t>(lane) * 4u;

    float4v oacc[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) oacc[t] = float4v{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;

    // One tile per step, its register set refilled in place with tile t + 8: the next K is
    // requested as soon as this tile's scores exist, the next V as soon as its P.V products are
    // issued.  live == false makes the refill a dead load (past the chunk's end).
    // Issue priority: the two wavefronts sharing a SIMD (w and w ^ 4) would otherwise be served
    // oldest first, and the younger one would finish its equal share of tiles much later.  Each
    // wavefront publishes how many tiles it has started; the younger one takes the higher
    // priority while it is not ahead of its partner, the older one only while it is behind.
    // Tile assignment stays static, so results do not depend on timing.
    const int partner = wave_u ^ (kDecWaves / 2);
    const bool younger = wave_u >= kDecWaves / 2;
    auto step = [&](int t, int inext, bool live, int done) {
        if (lane == 0) progress[wave_u] = done;
        const int other = __builtin_amdgcn_readfirstlane(progress[partner]);
        const int key0 = key_begin + t * kTile;
        const bool valid = valid_t;
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
        const int64_t rec = rec_of(t + kDecWaves, inext, valid_t);
        const int64_t rec_pf = live ? rec : 0;
        const LaneOffsets ofs_pf = live ? lofs : dead_ofs;
        __builtin_amdgcn_sched_barrier(0);
        load_k(p, rec_pf, ofs_pf, kr);
        __builtin_amdgcn_sched_barrier(0);
        if (younger ? (done <= other) : (done < other))
            __builtin_amdgcn_s_setprio(1);
        else
            __builtin_amdgcn_s_setprio(0);
        float mx = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sc[j]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        // The reference maximum moves only when a score exceeds it by more than kRescaleSlack
        // (so exp2(s - m_run) <= 256, well inside fp16): the softmax does not depend on the
        // reference, and rescaling the 64 accumulators becomes rare.  This lane's accumulators
        // all belong to head n, so the rescale factor is lane-local.
        if (__any(mx > m_run + kRescaleSlack)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = (m_new > m_run) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            l_run *= alpha;
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) oacc[tt] *= alpha;
            m_run = m_new;
        }
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
        __builtin_amdgcn_sched_barrier(0);
        load_v(p, rec_pf, ofs_pf, vr);
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- main loop over chunks of 64 tiles (one VGPR of page IDs)
    for (int c0 = 0; c0 < n_mine; c0 += kWave) {
        const int cn = min(kWave, n_mine - c0);
        const int tc = wave_u + c0 * kDecWaves;  // first tile of the chunk
        if (c0 > 0) {
            fetch_pids(c0 / kWave);
            issue(tc, 0, true);
        }
        for (int i = 0; i < cn; ++i) step(tc + i * kDecWaves, i + 1, i + 1 < cn, c0 + i);
    }
    __builtin_amdgcn_s_setprio(0);

    // ---- per-wave softmax totals
    float l_tot = l_run + __shfl_xor(l_run, 16, kWave);
    l_tot = l_tot + __shfl_xor(l_tot, 32, kWave);
    __syncthreads();  // table no longer needed
    if (gq == 0) {
        stat_m[wave][n] = m_run;
        stat_l[wave][n] = l_tot;
    }
    __syncthreads();

    // ---- merge the workgroup's waves.  Each lane rescales its accumulators (all of head n) to
    // the workgroup maximum; then a fixed-order tree in LDS adds waves 4..7 into 0..3, 2..3 into
    // 0..1 and 1 into 0.  The LDS image keeps the accumulator lane layout ([wave][register][lane]
    // as 16-byte rows), so every access is conflict-free.
    {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, stat_m[w][n]);
        const float f = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) oacc[tt] *= f;
        if (tid < G) {
            float Ls = 0.f;
            for (int w = 0; w < kDecWaves; ++w)
                Ls += (stat_m[w][tid] == -INFINITY) ? 0.f : stat_l[w][tid] * __builtin_amdgcn_exp2f(stat_m[w][tid] - M);
            resM[tid] = M;
            resL[tid] = Ls;
        }
    }
    float4v *tree = reinterpret_cast<float4v *>(lut_mem);  // [4][16][64] rows of 16 bytes = 64 KiB
#pragma unroll
    for (int half = kDecWaves / 2; half >= 1; half >>= 1) {
        if (wave_u >= half && wave_u < 2 * half) {
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) tree[((wave_u - half) * 16 + tt) * kWave + lane] = oacc[tt];
        }
        __syncthreads();
        if (wave_u < half) {
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) oacc[tt] += tree[(wave_u * 16 + tt) * kWave + lane];
        }
        __syncthreads();
    }

    if (n_active > 1) {
        // more than one split: wave 0 leaves (M, L, O[G][256]) for the combine kernel; lane
        // (gq, n) holds dims 8 (2 (4 gq + r) + c) + i of head n in oacc[8 c + i][r]
        if (wave_u == 0) {
            const size_t bg = static_cast<size_t>(b) * p.n_kv + g;
            float *dst = reinterpret_cast<float *>(static_cast<char *>(p.workspace) + a.parts_off) +
                         (bg * a.n_splits + s) * static_cast<size_t>(a.partial_floats);
            if (lane < G) {
                dst[lane] = resM[lane];
                dst[16 + lane] = resL[lane];
            }
            if (n < G) {
                float *row = dst + 32 + n * kDim;
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
        }
        return;
    }

    // ---- single split: wave 0 writes O to LDS as [head][64 quads of dims], quads swizzled
    // within groups of 8 so both this scatter and the row reads below spread over the banks;
    // then one wave per head applies the inverse rotation, o = H O / (256 L)
    auto quad_at = [](int h, int qd) { return h * 64 + (qd ^ ((h + 2 * (qd >> 4)) & 7)); };
    float4v *res4 = tree;
    if (wave_u == 0 && n < G) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int qd = 16 * gq + 4 * r + 2 * c + hf;
                    res4[quad_at(n, qd)] = float4v{oacc[8 * c + 4 * hf][r], oacc[8 * c + 4 * hf + 1][r],
                                                   oacc[8 * c + 4 * hf + 2][r], oacc[8 * c + 4 * hf + 3][r]};
                }
    }
    __syncthreads();
    for (int h = wave; h < G; h += kDecWaves) {
        const float4v v = res4[quad_at(h, lane)];
        float y[4] = {v[0], v[1], v[2], v[3]};
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
// One workgroup of four wavefronts per (query head, KV head, request) merges the split partials
// of that head: every wavefront reduces the splits' maxima in registers (lane i holds split
// 64 c + i), then wavefront w sums splits w, w + 4, ... for dims 4 l .. 4 l + 3 in lane l (16-byte
// loads), and wavefront 0 adds the four sums in fixed order, applies the inverse rotation and
// writes bf16.

constexpr int kCombWaves = 4;
constexpr int kCombThreads = kCombWaves * kWave;
constexpr int kCombPerWave = kWave / kCombWaves;  // splits per wavefront in each group of 64

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

__global__ __launch_bounds__(kCombThreads) void tq4_decode_combine_kernel(DecodeArgs a) {
    __shared__ float4v part[kCombWaves][kWave];
    const DecodeParams &p = a.p;
    const int G = a.group;
    const int h = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int L_req = p.seq_lens[b];
    const size_t pf = static_cast<size_t>(a.partial_floats);
    const float *base = reinterpret_cast<const float *>(static_cast<const char *>(p.workspace) + a.parts_off) +
                        (static_cast<size_t>(b) * p.n_kv + g) * a.n_splits * pf;
    const int ns = a.n_splits;
    // Every load of the first group of 64 splits is issued before the length is known (slots past
    // the live splits hold stale data and are dropped by selection, never multiplied in).
    const int s_l = min(lane, ns - 1);
    const float m0 = base[s_l * pf + h];
    const float l0 = base[s_l * pf + 16 + h];
    float4v v[kCombPerWave];
#pragma unroll
    for (int u = 0; u < kCombPerWave; ++u) {
        const int s = min(wave + kCombWaves * u, ns - 1);
        v[u] = *reinterpret_cast<const float4v *>(base + s * pf + 32 + h * kDim + 4 * lane);
    }
    const int L = L_req < 0 ? 0 : (L_req > p.max_seq_len ? p.max_seq_len : L_req);
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
        if (s < n_active) mx = fmaxf(mx, base[s * pf + h]);
    }
    const float M = wave_max(mx);

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
        const float mc = s < n_active ? base[s * pf + h] : -INFINITY;
        const float wc = s < n_active ? weight(mc) : 0.f;
        lsum += s < n_active ? wc * base[s * pf + 16 + h] : 0.f;
        for (int u = 0; u < kCombPerWave; ++u) {
            const int s2 = c * kWave + wave + kCombWaves * u;
            if (s2 < n_active) {
                const float ws = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wc), wave + kCombWaves * u));
                acc += ws * *reinterpret_cast<const float4v *>(base + s2 * pf + 32 + h * kDim + 4 * lane);
            }
        }
    }
    const float Ltot = wave_sum(lsum);
    part[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && merge) {
        const float4v t = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
        float y[4] = {t[0], t[1], t[2], t[3]};
        wave_fwht(y, lane);
        const float f = Ltot > 0.f ? (1.0f / 256.0f) / Ltot : 0.f;
        u32x2 o;
        o.x = static_cast<uint32_t>(f32_to_bf16(y[0] * f)) | (static_cast<uint32_t>(f32_to_bf16(y[1] * f)) << 16);
        o.y = static_cast<uint32_t>(f32_to_bf16(y[2] * f)) | (static_cast<uint32_t>(f32_to_bf16(y[3] * f)) << 16);
        *reinterpret_cast<u32x2 *>(p.out + (static_cast<int64_t>(b) * p.n_q + static_cast<int64_t>(g) * G + h) * kDim +
                                   4 * lane) = o;
    }
}

hipError_t launch_decode(const DecodeParams &p, const DecodePlan &plan, hipStream_t stream) {
    DecodeArgs a;
    a.p = p;
    a.group = plan.group;
    a.n_splits = plan.n_splits;
    a.split_tiles = plan.split_tiles;
    a.partial_floats = static_cast<int32_t>(plan.partial_floats);
    a.parts_off = plan.counters_bytes;
    lut_pairs_from_codebook(a.lut_pairs, codebook().centroid);
    for (int i = 0; i < 15; ++i) a.thr[i] = codebook().threshold[i];
    hipLaunchKernelGGL(tq4_decode_kernel, dim3(plan.n_splits, p.n_kv, p.batch), dim3(kDecThreads), 0, stream, a);
    if (plan.n_splits > 1)
        hipLaunchKernelGGL(tq4_decode_combine_kernel, dim3(plan.group, p.n_kv, p.batch), dim3(kCombThreads), 0,
                           stream, a);
    return hipGetLastError();
}

}  // namespace tq4
