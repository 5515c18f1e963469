// tq4_prefill.hip -- causal attention of a chunk of query tokens over TQ4 pages, gfx950.
//
// Multi-query prefill reconstructs K/V tiles and runs a floating-point attention
// consumer ("Fitting a 27B-Parameter LLM into 24 GiB of Laptop Memory", section
// "KVExec: Fused Reconstruction with Layer-Scoped Lifetime").  Here the tiles
// are reconstructed in the rotated domain (16 c[idx], fp16) inside registers
// and consumed by v_mfma_f32_16x16x32_f16; the norms scale scores and
// probabilities, and each output row gets one inverse rotation at the end
// (KVExec row of the mechanism table in "JustFit: Run Qwen 27B Fast with its
// full 256K context on a 24 GB Mac": attention in the rotated domain).
//
// Query rows of one KV head are (token, head-in-group) pairs, row = t * G + h.
// Row r of the chunk sits at absolute position prior_len + t and sees keys
// 0 .. prior_len + t.
//
// Three kernels per call:
//   1. rotate: one wavefront per query row: Hq in fp32, a power-of-two scale,
//      fp16 row and its score factor to the workspace;
//   2. attend: grid (key split, row block, KV head); 4 wavefronts, one per
//      SIMD, each owning R blocks of 16 rows; every wavefront walks the
//      workgroup's key tiles, decodes each tile once and feeds its R blocks
//      (S^T = K Q^T and O^T = V^T P^T on the same decoded operands); online
//      softmax per row with the causal limit; a partial (O, max, sum) per row
//      and split goes to the workspace;
//   3. combine: one wavefront per row: merges the splits, inverse rotation,
//      bf16 output.
#include <type_traits>

#include "tq4_device.h"
#include "tq4_launch.h"
#include "tq4_tile.h"

namespace tq4 {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfBlocks = 2;                               // R: 16-row blocks per wavefront
constexpr int kPfRowsPerWg = kPfWaves * kPfBlocks * 16;   // 128
constexpr int kPfPartial = kDim + 4;                       // O[256], max, sum, pad
constexpr int kPfTargetWgs = 768;                          // 3 x 256 compute units
constexpr float kPfRescaleSlack = 8.0f;  // log2 headroom before a running maximum is moved

struct PrefillArgs {
    PrefillParams p;
    int32_t group;
    int32_t rows;          // chunk_len * group (per KV head)
    int32_t n_splits;
    int32_t split_tiles;
    uint64_t qrot_off;     // fp16 [chunk_len * n_q][256]
    uint64_t frow_off;     // float [chunk_len * n_q]
    uint64_t parts_off;    // float [n_kv][rows][n_splits][kPfPartial]
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
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, kWave));
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

template <int R>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void tq4_prefill_kernel(PrefillArgs a) {
    __shared__ __align__(16) uint32_t lut_mem[kLutWords];
    const PrefillParams &p = a.p;
    const int G = a.group;
    const int s = blockIdx.x, rb = blockIdx.y, g = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, gq = lane >> 4;
    char *ws = static_cast<char *>(p.workspace);

    // rows of this wave: row0 + 16 j + n for block j
    const int row0 = rb * kPfRowsPerWg + wave * (R * 16);
    const int wg_last_row = min(rb * kPfRowsPerWg + kPfRowsPerWg, a.rows) - 1;
    const int wg_kmax = p.prior_len + wg_last_row / G + 1;  // keys any row of the workgroup sees
    const int split_keys = a.split_tiles * kTile;
    const int key_begin = s * split_keys;
    const int key_end = min(key_begin + split_keys, wg_kmax);
    const int n_tiles = key_end > key_begin ? (key_end - key_begin + kTile - 1) / kTile : 0;

    // ---- per-block row data: causal limit, score factor, query operand
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
        fcol[j] = live ? reinterpret_cast<const float *>(ws + a.frow_off)[qrow] : 0.f;
        const char *qr = ws + a.qrot_off + static_cast<int64_t>(qrow) * (kDim * 2);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int w = 16 * (ks >> 2) + 4 * gq + (ks & 3);
            u32x4 v = *reinterpret_cast<const u32x4 *>(qr + 16 * w);
            if (!live) v = u32x4{0u, 0u, 0u, 0u};
            qop[j][ks] = __builtin_bit_cast(half8, v);
        }
    }
    build_lut<kPfThreads>(lut_mem, a.lut_pairs, tid);
    __syncthreads();
    const char *lut = reinterpret_cast<const char *>(lut_mem);
    const uint32_t lane4 = static_cast<uint32_t>(lane) * 4u;
    const LaneOffsets lofs = lane_offsets(lane);
    const int32_t *pt = p.page_table;

    float4v oacc[R][16];
    float m_run[R], l_run[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
#pragma unroll
        for (int t = 0; t < 16; ++t) oacc[j][t] = float4v{0.f, 0.f, 0.f, 0.f};
        m_run[j] = -INFINITY;
        l_run[j] = 0.f;
    }

    KRegs kr;
    VRegs vr;
    bool valid_cur = false, valid_next = false;
    int64_t rec_next = 0;
    auto rec_of = [&](int t, bool &valid_d) -> int64_t {
        const int key0 = key_begin + t * kTile;
        const int pid = pt[key0 / p.page_size];  // wave-uniform address: a scalar load
        return tile_rec0(p, g, key0, pid, valid_d);
    };
    if (n_tiles > 0) {
        rec_next = rec_of(0, valid_next);
        load_k(p, rec_next, lofs, kr);
        load_v(p, rec_next, lofs, vr);
    }

    auto step = [&](int t, auto prefetch) {
        const int key0 = key_begin + t * kTile;
        const bool valid = valid_cur;
        // ---- scores for all R blocks from one decode of the K tile
        float4v sacc[R][2];
#pragma unroll
        for (int j = 0; j < R; ++j) sacc[j][0] = sacc[j][1] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const u32x4 kw = kr.k[mt][ks >> 2];
                const uint32_t w = (ks & 3) == 0 ? kw.x : (ks & 3) == 1 ? kw.y : (ks & 3) == 2 ? kw.z : kw.w;
                const half8 kop = lut_decode(w, lane4, lut);
#pragma unroll
                for (int j = 0; j < R; ++j)
                    sacc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[j][ks], sacc[j][mt], 0, 0, 0);
            }
        float kn[8], nv[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            kn[4 * h + 0] = f16lo(kr.kn[h].x);
            kn[4 * h + 1] = f16hi(kr.kn[h].x);
            kn[4 * h + 2] = f16lo(kr.kn[h].y);
            kn[4 * h + 3] = f16hi(kr.kn[h].y);
            nv[4 * h + 0] = f16lo(vr.vn[h].x);
            nv[4 * h + 1] = f16hi(vr.vn[h].x);
            nv[4 * h + 2] = f16lo(vr.vn[h].y);
            nv[4 * h + 3] = f16hi(vr.vn[h].y);
        }
        if constexpr (decltype(prefetch)::value) {
            rec_next = rec_of(t + 1, valid_next);
            __builtin_amdgcn_sched_barrier(0);
            load_k(p, rec_next, lofs, kr);
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- online softmax per block, probabilities as the P^T operand
        half8 pop[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int lim = valid ? min(key_end, lim_row[j]) - key0 : 0;  // visible keys in this tile
            float sc[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int koff = (q < 4) ? (4 * gq + q) : (16 + 4 * gq + (q - 4));
                sc[q] = (koff < lim) ? sacc[j][q >> 2][q & 3] * kn[q] * fcol[j] : -INFINITY;
            }
            float mx = sc[0];
#pragma unroll
            for (int q = 1; q < 8; ++q) mx = fmaxf(mx, sc[q]);
            mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
            mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
            // the reference maximum moves only when a score exceeds it by more than the slack
            // (exp2(s - m_run) <= 256 stays well inside fp16), so rescaling is rare
            if (__any(mx > m_run[j] + kPfRescaleSlack)) {
                const float m_new = fmaxf(m_run[j], mx);
                const float alpha = (m_new > m_run[j]) ? __builtin_amdgcn_exp2f(m_run[j] - m_new) : 1.0f;
                l_run[j] *= alpha;
#pragma unroll
                for (int tt = 0; tt < 16; ++tt) oacc[j][tt] *= alpha;
                m_run[j] = m_new;
            }
            float pv[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float e = (sc[q] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sc[q] - m_run[j]);
                l_run[j] += e;
                pv[q] = e * nv[q];
            }
            u32x4 pr;
            pr.x = pack_f16x2(pv[0], pv[1]);
            pr.y = pack_f16x2(pv[2], pv[3]);
            pr.z = pack_f16x2(pv[4], pv[5]);
            pr.w = pack_f16x2(pv[6], pv[7]);
            pop[j] = __builtin_bit_cast(half8, pr);
        }
        // ---- O^T += V^T P^T for all R blocks from one decode of the V tile
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            uint32_t wv[8], u[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) wv[q] = c == 0 ? vr.v[q].x : vr.v[q].y;
            nibble_transpose8(wv, u);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const half8 vop = lut_decode(u[i], lane4, lut);
#pragma unroll
                for (int j = 0; j < R; ++j)
                    oacc[j][8 * c + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop[j], oacc[j][8 * c + i], 0, 0, 0);
            }
        }
        if constexpr (decltype(prefetch)::value) {
            __builtin_amdgcn_sched_barrier(0);
            load_v(p, rec_next, lofs, vr);
            __builtin_amdgcn_sched_barrier(0);
        }
        valid_cur = valid_next;
    };
    valid_cur = valid_next;
    for (int t = 0; t + 1 < n_tiles; ++t) step(t, std::true_type{});
    if (n_tiles > 0) step(n_tiles - 1, std::false_type{});

    // ---- partials: lane (gq, n) of block j holds row n, dims 8 (2 (4 gq + r) + c) + i
    float *parts = reinterpret_cast<float *>(ws + a.parts_off);
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const int row = row0 + 16 * j + n;
        float l_tot = l_run[j] + __shfl_xor(l_run[j], 16, kWave);
        l_tot = l_tot + __shfl_xor(l_tot, 32, kWave);
        if (row >= a.rows) continue;
        float *dst = parts + ((static_cast<int64_t>(g) * a.rows + row) * a.n_splits + s) * kPfPartial;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int i = 0; i < 8; ++i) dst[8 * (2 * (4 * gq + r) + c) + i] = oacc[j][8 * c + i][r];
        if (gq == 0) {
            dst[kDim] = m_run[j];
            dst[kDim + 1] = l_tot;
        }
    }
}

// ---------------------------------------------------------------- 3. combine

__global__ __launch_bounds__(256) void tq4_prefill_combine_kernel(PrefillArgs a) {
    const PrefillParams &p = a.p;
    const int G = a.group;
    const int lane = threadIdx.x & 63;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);  // g * rows + row
    if (idx >= static_cast<int64_t>(p.n_kv) * a.rows) return;
    const int g = static_cast<int>(idx / a.rows), row = static_cast<int>(idx % a.rows);
    const float *base = reinterpret_cast<const float *>(static_cast<const char *>(p.workspace) + a.parts_off) +
                        idx * a.n_splits * kPfPartial;
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
    wave_fwht(y, lane);
    const float f = L > 0.f ? (1.0f / 256.0f) / L : 0.f;
    const int t = row / G, qh = g * G + (row - t * G);
    u32x2 o;
    o.x = static_cast<uint32_t>(f32_to_bf16(y[0] * f)) | (static_cast<uint32_t>(f32_to_bf16(y[1] * f)) << 16);
    o.y = static_cast<uint32_t>(f32_to_bf16(y[2] * f)) | (static_cast<uint32_t>(f32_to_bf16(y[3] * f)) << 16);
    *reinterpret_cast<u32x2 *>(p.out + (static_cast<int64_t>(t) * p.n_q + qh) * kDim + 4 * lane) = o;
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
    lut_pairs_from_codebook(a.lut_pairs, codebook().centroid);
    const int64_t rot_blocks = (static_cast<int64_t>(qrows) + 3) / 4;
    const int64_t comb_blocks = (static_cast<int64_t>(p.n_kv) * a.rows + 3) / 4;
    if (rot_blocks > 0x7fffffff || comb_blocks > 0x7fffffff || plan.n_qblocks > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(tq4_prefill_rotate_kernel, dim3(static_cast<unsigned>(rot_blocks)), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(tq4_prefill_kernel<kPfBlocks>, dim3(plan.n_splits, plan.n_qblocks, p.n_kv), dim3(kPfThreads),
                       0, stream, a);
    hipLaunchKernelGGL(tq4_prefill_combine_kernel, dim3(static_cast<unsigned>(comb_blocks)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tq4
