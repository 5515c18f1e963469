// tq4_dense.hip -- the unfused path, gfx950: reconstruct TQ4 pages into contiguous bf16 K/V, then
// dense decode attention over those tensors.
//
// "Fitting a 27B-Parameter LLM into 24 GiB of Laptop Memory", section "KVExec: Fused Reconstruction
// with Layer-Scoped Lifetime": besides the fused paths, multi-query prefill can reconstruct pages
// into contiguous tensors of the query dtype, and a gather-and-SDPA path is the fallback.  This
// file is that path, kept beside the fused kernels so the cost of not fusing can be measured: the
// reconstruction writes 512 B per vector that the attention reads back, against 130 B per vector
// read once by the fused kernels.
//
//   tq4_reconstruct_kernel: one wavefront per run of 16 positions (their K and V records), lane l
//     holding dims 4l .. 4l+3: centroid lookup, 256-point Hadamard transform in fp32 (two stages
//     in registers, six by lane exchange), times norm / 16, bf16 (round to nearest even).
//   tq4_sdpa_split_kernel: split-K decode attention over bf16 K/V [batch][n_kv][max_seq][256].
//     Per 32-key tile and wavefront: S^T[32 keys][16 heads] = K Q^T with 16 bf16 MFMAs (K rows
//     are MFMA operands as stored), base-2 online softmax, then O[heads][256] += P V on the vector
//     ALUs with lane l owning dims 4l .. 4l+3 (P goes through LDS).  Partials use the decode
//     kernel's layout and its combine (without the inverse rotation).
#include <cfloat>

#include "tq4_device.h"
#include "tq4_encode_wave.h"
#include "tq4_launch.h"
#include "tq4_tile.h"

namespace tq4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- reconstruction

constexpr int kRecWaves = 4;
constexpr int kRecPositionsPerWave = 16;

struct ReconArgs {
    ReconParams p;
    float centroid[16];
};

__global__ __launch_bounds__(kRecWaves * kWave) void tq4_reconstruct_kernel(ReconArgs a) {
    __shared__ float cent[16];
    const ReconParams &p = a.p;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave_u = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int g = blockIdx.y, b = blockIdx.z;
    if (threadIdx.x < 16) cent[threadIdx.x] = a.centroid[threadIdx.x];
    __syncthreads();
    const int L_req = p.seq_lens[b];
    const int L = L_req < 0 ? 0 : (L_req > p.max_seq_len ? p.max_seq_len : L_req);
    // this wave's run: kRecPositionsPerWave consecutive positions inside one page (page sizes are
    // multiples of 32), so one table entry and consecutive records cover it
    const int pos0 = (blockIdx.x * kRecWaves + wave_u) * kRecPositionsPerWave;
    if (pos0 >= L) return;
    const int cnt = min(kRecPositionsPerWave, L - pos0);
    const int page = p.page_table[static_cast<int64_t>(b) * p.table_stride + pos0 / p.page_size];
    const bool valid = page >= 0 && page < p.num_pages;  // a page outside the pool reads as zeros
    const int64_t rec0 = valid ? (static_cast<int64_t>(page) * p.n_kv + g) * p.page_size + pos0 % p.page_size : 0;
    // every load of the run first: word lane / 2 of each record, and the run's norms one per lane
    uint32_t kw[kRecPositionsPerWave], vw[kRecPositionsPerWave];
#pragma unroll
    for (int j = 0; j < kRecPositionsPerWave; ++j) {
        const int64_t r = valid ? rec0 + min(j, cnt - 1) : 0;
        kw[j] = p.k_words[r * kWords + (lane >> 1)];
        vw[j] = p.v_words[r * kWords + (lane >> 1)];
    }
    const int64_t rn = valid ? rec0 + min(lane & (kRecPositionsPerWave - 1), cnt - 1) : 0;
    const uint32_t nk = p.k_norms[rn], nv = p.v_norms[rn];
    const uint32_t shift = 16u * static_cast<uint32_t>(lane & 1);
    const int64_t o0 = ((static_cast<int64_t>(b) * p.n_kv + g) * p.max_seq_len + pos0) * kDim + 4 * lane;
    auto vector_out = [&](uint32_t w, uint32_t norm_bits, uint16_t *dst) {
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = cent[(w >> (shift + 4u * j)) & 15u];
        {  // stages h = 1, 2 inside the lane, then h = 4 .. 128 across lanes
            const float t0 = y[0] + y[1], t1 = y[0] - y[1], t2 = y[2] + y[3], t3 = y[2] - y[3];
            y[0] = t0 + t2;
            y[2] = t0 - t2;
            y[1] = t1 + t3;
            y[3] = t1 - t3;
        }
        enc_stage<1>(y, lane);
        enc_stage<2>(y, lane);
        enc_stage<4>(y, lane);
        enc_stage<8>(y, lane);
        enc_stage<16>(y, lane);
        enc_stage<32>(y, lane);
        const float f = valid ? f16_bits_to_f32(static_cast<uint16_t>(norm_bits)) * (1.0f / 16.0f) : 0.f;  // n (H c) / 16
        *reinterpret_cast<u32x2 *>(dst) = u32x2{pack_bf16x2(y[0] * f, y[1] * f), pack_bf16x2(y[2] * f, y[3] * f)};
    };
#pragma unroll
    for (int j = 0; j < kRecPositionsPerWave; ++j) {
        if (j < cnt) {  // wave-uniform; a guard, not a break, so the loop unrolls
            vector_out(kw[j], __builtin_amdgcn_readlane(nk, j), p.k_out + o0 + j * kDim);
            vector_out(vw[j], __builtin_amdgcn_readlane(nv, j), p.v_out + o0 + j * kDim);
        }
    }
}

hipError_t launch_reconstruct(const ReconParams &p, hipStream_t stream) {
    ReconArgs a;
    a.p = p;
    for (int i = 0; i < 16; ++i) a.centroid[i] = codebook().centroid[i];
    static_assert(32 % kRecPositionsPerWave == 0, "a run must stay inside one page");
    const int per_block = kRecWaves * kRecPositionsPerWave;
    const int blocks = (p.max_seq_len + per_block - 1) / per_block;
    hipLaunchKernelGGL(tq4_reconstruct_kernel, dim3(blocks, p.n_kv, p.batch), dim3(kRecWaves * kWave), 0, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- dense decode attention

constexpr int kDenseMaxSplits = 256;
constexpr int kDensePlanCUs = 256;
constexpr int kDenseMinTilesPerWave = 2;
constexpr int kPRow = 20;  // floats per key row of the P staging area: 16 columns + pad (16-byte rows, no bank conflicts)
constexpr float kDenseRescaleSlack = 8.0f;

DensePlan plan_dense(int32_t batch, int32_t max_seq_len, int32_t n_q_heads, int32_t n_kv_heads) {
    DensePlan pl{};
    pl.group = n_q_heads / n_kv_heads;
    pl.waves = pl.group <= 8 ? 8 : 4;
    const int64_t tiles = (static_cast<int64_t>(max_seq_len) + kTile - 1) / kTile;
    const int64_t units = static_cast<int64_t>(batch) * n_kv_heads;
    int64_t want = (kDensePlanCUs + units - 1) / units;
    const int64_t cap = (tiles + pl.waves * kDenseMinTilesPerWave - 1) / (pl.waves * kDenseMinTilesPerWave);
    if (want > cap) want = cap;
    if (want > kDenseMaxSplits) want = kDenseMaxSplits;
    if (want < 1) want = 1;
    pl.split_tiles = static_cast<int32_t>((tiles + want - 1) / want);
    pl.n_splits = static_cast<int32_t>((tiles + pl.split_tiles - 1) / pl.split_tiles);
    pl.partial_floats = 2 * kSplitStatPad + static_cast<size_t>(pl.group) * kDim;
    pl.workspace_bytes = pl.n_splits > 1 ? static_cast<size_t>(units) * pl.n_splits * pl.partial_floats * sizeof(float)
                                         : 0;
    return pl;
}

struct DenseArgs {
    DenseParams p;
    int32_t group;
    int32_t n_splits;
    int32_t split_tiles;
    int32_t partial_floats;
};

// GMAX: largest group (query heads per KV head) the instance handles; NW wavefronts per workgroup.
template <int GMAX, int NW>
__global__ __launch_bounds__(NW * kWave) void tq4_sdpa_split_kernel(DenseArgs a) {
    constexpr int NT = NW * kWave;
    __shared__ __align__(16) float p_sh[NW][kTile][kPRow];  // per wavefront: P[key][column]
    __shared__ __align__(16) float alpha_sh[NW][16];        // per wavefront: rescale factor per column
    __shared__ float stat_m[NW][16];
    __shared__ float stat_l[NW][16];
    __shared__ float resM[16];
    __shared__ float resL[16];
    __shared__ __align__(16) float4v tree[NW / 2][GMAX][kWave];

    const DenseParams &p = a.p;
    const int G = a.group;
    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int n = lane & 15, gq = lane >> 4;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int L_req = p.seq_lens[b];
    const int split_keys = a.split_tiles * kTile;
    const int key_begin = s * split_keys;

    // ---- query operand (B of S^T = K Q^T): lane (gq, n) holds column n (head g G + n; zero past
    // the group) at dims 32 ks + 8 gq .. + 7 of K-step ks
    const uint16_t *qrow = p.q + (static_cast<int64_t>(b) * p.n_q + static_cast<int64_t>(g) * G + min(n, G - 1)) * kDim;
    bf16x8 qop[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        u32x4 raw = *reinterpret_cast<const u32x4 *>(qrow + 32 * ks + 8 * gq);
        if (n >= G) raw = u32x4{0u, 0u, 0u, 0u};
        qop[ks] = __builtin_bit_cast(bf16x8, raw);
    }

    const int L = L_req < 0 ? 0 : (L_req > p.max_seq_len ? p.max_seq_len : L_req);
    const int n_active = (L + split_keys - 1) / split_keys;
    if (s >= n_active) {
        if (L == 0 && s == 0)
            for (int i = tid; i < G * kDim; i += NT)
                p.out[(static_cast<int64_t>(b) * p.n_q + static_cast<int64_t>(g) * G + i / kDim) * kDim + i % kDim] = 0;
        return;
    }
    const int key_end = min(key_begin + split_keys, L);
    const int n_tiles = (key_end - key_begin + kTile - 1) / kTile;
    const int n_mine = wave_u < n_tiles ? (n_tiles - wave_u + NW - 1) / NW : 0;
    const uint16_t *kbase = p.k + (static_cast<int64_t>(b) * p.n_kv + g) * p.max_seq_len * kDim;
    const uint16_t *vbase = p.v + (static_cast<int64_t>(b) * p.n_kv + g) * p.max_seq_len * kDim;

    // Tile registers, refilled in place: K as MFMA operands (key 16 mt + n, dims 32 ks + 8 gq ..),
    // V as rows (key j, dims 4 lane ..).  Key indices are clamped to L - 1, so every load reads a
    // written row; keys past the split's end are masked in the scores.
    u32x4 kt[2][8];
    u32x2 vt[kTile];
    auto load_k = [&](int t) {
        const int key0 = key_begin + t * kTile;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int key = min(key0 + 16 * mt + n, L - 1);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                kt[mt][ks] = *reinterpret_cast<const u32x4 *>(kbase + static_cast<int64_t>(key) * kDim + 32 * ks + 8 * gq);
        }
    };
    auto load_v = [&](int t) {
        const int key0 = key_begin + t * kTile;
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            const int key = min(key0 + j, L - 1);
            vt[j] = *reinterpret_cast<const u32x2 *>(vbase + static_cast<int64_t>(key) * kDim + 4 * lane);
        }
    };
    // the first tile in the loop's own order (K, then V), so the wait counts agree on entry
    const int t_first = min(wave_u, n_tiles - 1);
    __builtin_amdgcn_sched_barrier(0);
    load_k(t_first);
    __builtin_amdgcn_sched_barrier(0);
    load_v(t_first);
    __builtin_amdgcn_sched_barrier(0);

    float4v acc[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) acc[h] = float4v{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;  // of column n
    const float fscale = p.scale * 1.4426950408889634f;
    float(*pw)[kPRow] = p_sh[wave_u];

    for (int i = 0; i < n_mine; ++i) {
        const int t = wave_u + i * NW;
        const int key0 = key_begin + t * kTile;
        const int t_next = i + 1 < n_mine ? t + NW : t;  // past the end: a repeated, unused load
        // ---- S^T[keys][columns]
        float4v sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            sacc[mt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kt[mt][ks]), qop[ks],
                                                                  sacc[mt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);  // the refills stay where they are issued
        load_k(t_next);
        __builtin_amdgcn_sched_barrier(0);
        // lane (gq, n) holds column n at keys 16 mt + 4 gq + r
        const int lim = key_end - key0;
        float xs[8];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int koff = 16 * mt + 4 * gq + r;
                xs[4 * mt + r] = koff < lim ? sacc[mt][r] : -INFINITY;
            }
        float mx = xs[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) mx = fmaxf(mx, xs[j]);
        float lo, hi;
        lane_pair<16>(mx, lo, hi);
        mx = fmaxf(lo, hi);
        lane_pair<32>(mx, lo, hi);
        mx = fmaxf(lo, hi) * fscale;
        if (__any(mx > m_run + kDenseRescaleSlack)) {  // rare: move the reference, rescale the column
            const float m_new = fmaxf(m_run, mx);
            const float alpha = (m_new > m_run) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            l_run *= alpha;
            m_run = m_new;
            if (gq == 0) alpha_sh[wave_u][n] = alpha;
#pragma unroll
            for (int h = 0; h < GMAX; ++h) acc[h] *= alpha_sh[wave_u][h];
        }
        const float neg_m = -fmaxf(m_run, -FLT_MAX);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(xs[4 * mt + r], fscale, neg_m));
                l_run += e;
                pw[16 * mt + 4 * gq + r][n] = e;
            }
        // ---- O[h][dims 4 lane ..] += sum_j P[j][h] V[j][dims]
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            const float4v v = float4v{__uint_as_float(vt[j].x << 16), __uint_as_float(vt[j].x & 0xffff0000u),
                                      __uint_as_float(vt[j].y << 16), __uint_as_float(vt[j].y & 0xffff0000u)};
#pragma unroll
            for (int h4 = 0; h4 < GMAX; h4 += 4) {
                const float4v pj = *reinterpret_cast<const float4v *>(&pw[j][h4]);
#pragma unroll
                for (int hh = 0; hh < 4; ++hh) acc[h4 + hh] += pj[hh] * v;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        load_v(t_next);
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- per-wave totals, then the workgroup's maximum per column and the wave factors
    float l_tot = l_run;
    {
        float lo, hi;
        lane_pair<16>(l_tot, lo, hi);
        l_tot = lo + hi;
        lane_pair<32>(l_tot, lo, hi);
        l_tot = lo + hi;
    }
    if (gq == 0) {
        stat_m[wave_u][n] = m_run;
        stat_l[wave_u][n] = l_tot;
    }
    __syncthreads();
    if (tid < 16) {
        float M = -INFINITY;
        for (int w = 0; w < NW; ++w) M = fmaxf(M, stat_m[w][tid]);
        float Ls = 0.f;
        for (int w = 0; w < NW; ++w)
            Ls += stat_m[w][tid] == -INFINITY ? 0.f : stat_l[w][tid] * __builtin_amdgcn_exp2f(stat_m[w][tid] - M);
        resM[tid] = M;
        resL[tid] = Ls;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        const float mw = stat_m[wave_u][h];
        acc[h] *= mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - resM[h]);
    }
    // ---- fixed-order tree over the wavefronts: waves NW/2 .. NW-1 into 0 .., down to wave 0
#pragma unroll
    for (int half = NW / 2; half >= 1; half >>= 1) {
        if (wave_u >= half && wave_u < 2 * half) {
#pragma unroll
            for (int h = 0; h < GMAX; ++h) tree[wave_u - half][h][lane] = acc[h];
        }
        __syncthreads();
        if (wave_u < half) {
#pragma unroll
            for (int h = 0; h < GMAX; ++h) acc[h] += tree[wave_u][h][lane];
        }
        __syncthreads();
    }
    if (wave_u != 0) return;
    if (n_active > 1) {
        const size_t bg = static_cast<size_t>(b) * p.n_kv + g;
        float *dst = static_cast<float *>(p.workspace) + (bg * a.n_splits + s) * static_cast<size_t>(a.partial_floats);
        if (lane < G) {
            dst[lane] = resM[lane];
            dst[kSplitStatPad + lane] = resL[lane];
        }
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
            if (h < G) *reinterpret_cast<float4v *>(dst + 2 * kSplitStatPad + h * kDim + 4 * lane) = acc[h];
        return;
    }
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        if (h >= G) break;
        const float Lh = resL[h];
        const float f = Lh > 0.f ? 1.0f / Lh : 0.f;
        u32x2 o;
        o.x = static_cast<uint32_t>(f32_to_bf16(acc[h][0] * f)) | (static_cast<uint32_t>(f32_to_bf16(acc[h][1] * f)) << 16);
        o.y = static_cast<uint32_t>(f32_to_bf16(acc[h][2] * f)) | (static_cast<uint32_t>(f32_to_bf16(acc[h][3] * f)) << 16);
        *reinterpret_cast<u32x2 *>(p.out + (static_cast<int64_t>(b) * p.n_q + static_cast<int64_t>(g) * G + h) * kDim +
                                   4 * lane) = o;
    }
}

hipError_t launch_dense(const DenseParams &p, const DensePlan &plan, hipStream_t stream) {
    DenseArgs a;
    a.p = p;
    a.group = plan.group;
    a.n_splits = plan.n_splits;
    a.split_tiles = plan.split_tiles;
    a.partial_floats = static_cast<int32_t>(plan.partial_floats);
    const dim3 grid(plan.n_splits, p.n_kv, p.batch);
    if (plan.group <= 8)
        hipLaunchKernelGGL((tq4_sdpa_split_kernel<8, 8>), grid, dim3(8 * kWave), 0, stream, a);
    else
        hipLaunchKernelGGL((tq4_sdpa_split_kernel<16, 4>), grid, dim3(4 * kWave), 0, stream, a);
    if (plan.n_splits > 1) {
        CombineArgs c;
        c.parts = static_cast<const float *>(p.workspace);
        c.seq_lens = p.seq_lens;
        c.out = p.out;
        c.max_seq_len = p.max_seq_len;
        c.split_tiles = plan.split_tiles;
        c.n_splits = plan.n_splits;
        c.partial_floats = static_cast<int32_t>(plan.partial_floats);
        c.rows = plan.group;
        c.group = plan.group;
        c.n_queries = 1;
        c.n_q = p.n_q;
        c.n_kv = p.n_kv;
        c.batch = p.batch;
        return launch_split_combine(c, false, stream);
    }
    return hipGetLastError();
}

}  // namespace tq4
