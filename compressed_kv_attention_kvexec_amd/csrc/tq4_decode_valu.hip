// tq4_decode_valu.hip -- decode attention over TQ4 pages without matrix cores: two alternatives
// to the fused decode kernel (tq4_decode.hip), built to measure its design choices.
//
//  rotated  the same arithmetic as the fused kernel (rotated domain, KVExec row of the mechanism
//           table in "JustFit: Run Qwen 27B Fast with its full 256K context on a 24 GB Mac"):
//           scores are fp16 pair dot products (v_dot2, fp32 accumulation) of the rotated query
//           with 16 c[idx], values accumulate n_v p 16 c[idx] in fp32, one key at a time on the
//           vector ALUs; the output is H O / (256 L).
//  literal  the reconstruction order of "Fitting a 27B-Parameter LLM into 24 GiB of Laptop
//           Memory", section "KVExec: Fused Reconstruction with Layer-Scoped Lifetime": every
//           key and value vector is rebuilt in fp32 -- centroid lookup, inverse Hadamard rotation
//           (a 256-point butterfly: 3 stages in registers, 5 across lanes), norm restore n / 16 --
//           and attention runs in the natural domain on the rebuilt vectors.
//
// Both run the fused kernel's split plan (grid (split, KV head, request), 8 wavefronts, every 8th
// 32-key tile of the split per wavefront) and leave the same split partials (max, sum, O per query
// row) for tq4_decode_combine_kernel (with the inverse rotation for the rotated variant).  A
// half-wavefront takes one key at a time: lane w holds word w of the record, dims 8w .. 8w + 7.
#include <cfloat>

#include "tq4_device.h"
#include "tq4_launch.h"
#include "tq4_tile.h"

namespace tq4 {

constexpr int kValuWaves = 8;
constexpr int kValuThreads = kValuWaves * kWave;
constexpr float kValuSlack = 8.0f;  // log2 headroom before a running maximum is moved

struct ValuArgs {
    DecodeParams p;
    int32_t group;
    int32_t n_splits;
    int32_t split_tiles;
    int32_t partial_floats;
    uint64_t parts_off;
    uint32_t lut_pairs[8];  // fp16 bits of 16 * centroid[i], two per word (rotated)
    float centroid[16];     // fp32 centroids in ascending order (literal)
};

template <int M>
__device__ __forceinline__ void fwht_lane_stage(float x[8], int lane) {
    const bool upper = (lane & M) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float o = lane_xor<M>(x[i], lane);
        x[i] = upper ? (o - x[i]) : (x[i] + o);
    }
}

// 256-point unnormalised Hadamard transform of a vector held by 32 lanes, lane w holding dims
// 8w .. 8w + 7: stages 1, 2, 4 in registers, stages 8 .. 128 pair lane w with lane w ^ (h / 8).
__device__ __forceinline__ void half_wave_fwht(float x[8], int lane) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if ((i & h) == 0) {
                const float a = x[i], c = x[i + h];
                x[i] = a + c;
                x[i + h] = a - c;
            }
    fwht_lane_stage<1>(x, lane);
    fwht_lane_stage<2>(x, lane);
    fwht_lane_stage<4>(x, lane);
    fwht_lane_stage<8>(x, lane);
    fwht_lane_stage<16>(x, lane);
}

// Sum of v over the 32 lanes of a half-wavefront, in every lane of that half.
__device__ __forceinline__ float half_wave_sum(float v, int lane) {
    v += lane_xor<1>(v, lane);
    v += lane_xor<2>(v, lane);
    v += lane_xor<4>(v, lane);
    v += lane_xor<8>(v, lane);
    v += lane_xor<16>(v, lane);
    return v;
}

template <bool kLiteral, int GG>
__global__ __launch_bounds__(kValuThreads) void tq4_attn_valu_kernel(ValuArgs a) {
    __shared__ __align__(16) uint32_t lut_mem[kLutWords];  // pair table; after the loop: merge rows
    __shared__ float cent_sh[16];                             // literal: 16 entries in 16 banks
    __shared__ __align__(16) float qsh[GG][kDim];             // query rows (rotated and scaled, or natural)
    __shared__ float qf_sh[GG];                               // score factor per row (log2 units)
    __shared__ float stat_m[kValuWaves][GG];
    __shared__ float stat_l[kValuWaves][GG];
    __shared__ float resL[GG];

    const DecodeParams &p = a.p;
    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5, w = lane & 31;
    const int L_req = p.seq_lens[b];
    const int L = L_req < 0 ? 0 : (L_req > p.max_seq_len ? p.max_seq_len : L_req);
    const int split_keys = a.split_tiles * kTile;
    const int key_begin = s * split_keys;
    const int n_active = (L + split_keys - 1) / split_keys;
    auto row_off = [&](int h) -> int64_t {
        return (static_cast<int64_t>(b) * p.n_q + static_cast<int64_t>(g) * GG + h) * kDim;
    };
    if (s >= n_active) {
        if (L == 0 && s == 0)
            for (int i = tid; i < GG * kDim; i += kValuThreads) p.out[row_off(i / kDim) + (i % kDim)] = 0;
        return;
    }
    const int key_end = min(key_begin + split_keys, L);
    const int n_tiles = (key_end - key_begin + kTile - 1) / kTile;
    const int32_t *pt_row = p.page_table + static_cast<int64_t>(b) * p.table_stride;

    // ---- tables and query rows (wave h rotates row h: y = H q, scaled by a power of two into
    // [2^13, 2^14) for the fp16 operands; the literal variant keeps q as it is)
    if constexpr (!kLiteral) {
        build_lut<kValuThreads>(lut_mem, a.lut_pairs, tid);
    } else {
        if (tid < 16) cent_sh[tid] = a.centroid[tid];
    }
    for (int h = wave; h < GG; h += kValuWaves) {
        const u32x2 raw = *reinterpret_cast<const u32x2 *>(p.q + row_off(h) + 4 * lane);
        float y[4] = {__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                      __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
        float f = p.scale * 1.4426950408889634f;
        if constexpr (!kLiteral) {
            wave_fwht(y, lane);
            float mx = fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3])));
            mx = wave_max_f32(mx, lane);
            const int e = q_exponent(mx);
            const float qs = ldexpf(1.0f, e);
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] *= qs;
            f *= ldexpf(1.0f, -e) * (1.0f / 256.0f);
        }
        *reinterpret_cast<float4v *>(&qsh[h][4 * lane]) = float4v{y[0], y[1], y[2], y[3]};
        if (lane == 0) qf_sh[h] = f;
    }
    __syncthreads();

    // this lane's 8 dims of every row: fp16 pairs (rotated) or fp32 (literal)
    uint32_t qp[GG][4];
    float qv[GG][8];
    float fh[GG];
#pragma unroll
    for (int h = 0; h < GG; ++h) {
        fh[h] = qf_sh[h];
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[h][i] = qsh[h][8 * w + i];
        if constexpr (!kLiteral) {
#pragma unroll
            for (int i = 0; i < 4; ++i) qp[h][i] = pack_f16x2(qv[h][2 * i], qv[h][2 * i + 1]);
        }
    }
    const char *lut = reinterpret_cast<const char *>(lut_mem);
    const uint32_t lane4 = static_cast<uint32_t>(lane) * 4u;

    float m_run[GG], l_run[GG], acc[GG][8];
#pragma unroll
    for (int h = 0; h < GG; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
    }

    // centroids of the 8 nibbles of word wd: fp32 from the 16-entry table (literal), or 16 c as fp16
    // pairs through the replicated pair table (rotated)
    auto centroids = [&](uint32_t wd, float c[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = cent_sh[(wd >> (4 * i)) & 15u];
    };
    auto pairs = [&](uint32_t wd, uint32_t pr[4]) {
        const half8 d = lut_decode(wd, lane4, lut);
        const u32x4 u = __builtin_bit_cast(u32x4, d);
        pr[0] = u.x;
        pr[1] = u.y;
        pr[2] = u.z;
        pr[3] = u.w;
    };

    for (int t = wave; t < n_tiles; t += kValuWaves) {
        const int key0 = key_begin + t * kTile;
        bool valid;
        const int pid = pt_row[key0 / p.page_size];
        const int64_t rec0 = tile_rec0(p, g, key0, pid, valid);
        const int nvalid = valid ? min(kTile, key_end - key0) : 0;
        // this half's 16 keys (2k + half): word w of each K and V record; norms of keys 2i, 2i + 1
        // in lane i (i < 16)
        uint32_t kw[16], vw[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int64_t rec = rec0 + 2 * k + half;
            kw[k] = p.k_words[rec * kWords + w];
            vw[k] = p.v_words[rec * kWords + w];
        }
        const uint32_t knp = *reinterpret_cast<const uint32_t *>(p.k_norms + rec0 + 2 * (lane & 15));
        const uint32_t vnp = *reinterpret_cast<const uint32_t *>(p.v_norms + rec0 + 2 * (lane & 15));
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const bool live = 2 * k + half < nvalid;
            const uint32_t kpair = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(knp), k));
            const uint32_t vpair = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(vnp), k));
            const float nk = f16_bits_to_f32(static_cast<uint16_t>(half ? (kpair >> 16) : kpair));
            // a key past the length may hold any bits: its value norm must not reach the sums
            const float nv = live ? f16_bits_to_f32(static_cast<uint16_t>(half ? (vpair >> 16) : vpair)) : 0.f;
            // ---- scores
            float x[GG];
            if constexpr (!kLiteral) {
                uint32_t pr[4];
                pairs(kw[k], pr);
#pragma unroll
                for (int h = 0; h < GG; ++h) {
                    float d = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        d = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, qp[h][i]),
                                                   __builtin_bit_cast(f16x2_t, pr[i]), d, false);
                    x[h] = half_wave_sum(d, lane) * nk * fh[h];
                }
            } else {
                float kv[8];
                centroids(kw[k], kv);
                half_wave_fwht(kv, lane);
                const float kscale = nk * (1.0f / 16.0f);
#pragma unroll
                for (int i = 0; i < 8; ++i) kv[i] *= kscale;
#pragma unroll
                for (int h = 0; h < GG; ++h) {
                    float d = 0.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) d = __builtin_fmaf(qv[h][i], kv[i], d);
                    x[h] = half_wave_sum(d, lane) * fh[h];
                }
            }
            bool up = false;
#pragma unroll
            for (int h = 0; h < GG; ++h) {
                if (!live) x[h] = -INFINITY;
                up = up || (x[h] > m_run[h] + kValuSlack);
            }
            if (__any(up)) {
#pragma unroll
                for (int h = 0; h < GG; ++h) {
                    const float m_new = fmaxf(m_run[h], x[h]);
                    const float alpha = (m_new > m_run[h]) ? __builtin_amdgcn_exp2f(m_run[h] - m_new) : 1.0f;
                    l_run[h] *= alpha;
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[h][i] *= alpha;
                    m_run[h] = m_new;
                }
            }
            float pw[GG];
#pragma unroll
            for (int h = 0; h < GG; ++h) {
                const float e = __builtin_amdgcn_exp2f(x[h] - fmaxf(m_run[h], -FLT_MAX));
                l_run[h] += e;
                pw[h] = e;
            }
            // ---- values
            float vv[8];
            if constexpr (!kLiteral) {
                uint32_t pr[4];
                pairs(vw[k], pr);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vv[2 * i] = f16lo(pr[i]);
                    vv[2 * i + 1] = f16hi(pr[i]);
                }
#pragma unroll
                for (int h = 0; h < GG; ++h) pw[h] *= nv;
            } else {
                centroids(vw[k], vv);
                half_wave_fwht(vv, lane);
                const float vscale = nv * (1.0f / 16.0f);
#pragma unroll
                for (int i = 0; i < 8; ++i) vv[i] *= vscale;
            }
#pragma unroll
            for (int h = 0; h < GG; ++h)
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[h][i] = __builtin_fmaf(pw[h], vv[i], acc[h][i]);
        }
    }

    // ---- merge the two halves of the wavefront (lane w and lane w + 32 hold the same dims)
#pragma unroll
    for (int h = 0; h < GG; ++h) {
        float mo, lo;
        {
            float x0, x1;
            lane_pair<32>(m_run[h], x0, x1);
            mo = half ? x0 : x1;
            lane_pair<32>(l_run[h], x0, x1);
            lo = half ? x0 : x1;
        }
        const float M = fmaxf(m_run[h], mo);
        const float fa = (m_run[h] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[h] - M);
        const float fb = (mo == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mo - M);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float x0, x1;
            lane_pair<32>(acc[h][i], x0, x1);
            const float ao = half ? x0 : x1;
            // both halves form the same sum in the same order (the lower half's term first)
            acc[h][i] = half ? (ao * fb + acc[h][i] * fa) : (acc[h][i] * fa + ao * fb);
        }
        l_run[h] = half ? (lo * fb + l_run[h] * fa) : (l_run[h] * fa + lo * fb);
        m_run[h] = M;
    }
    __syncthreads();  // the pair table is no longer needed
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < GG; ++h) {
            stat_m[wave][h] = m_run[h];
            stat_l[wave][h] = l_run[h];
        }
    }
    __syncthreads();
    // ---- merge the 8 wavefronts: each scales its rows to the workgroup maximum and writes them to
    // its LDS slot; thread (row, 4 dims) adds the slots in a fixed order
    float *rows = reinterpret_cast<float *>(lut_mem);  // [wave][GG][256]
#pragma unroll
    for (int h = 0; h < GG; ++h) {
        float M = -INFINITY;
#pragma unroll
        for (int j = 0; j < kValuWaves; ++j) M = fmaxf(M, stat_m[j][h]);
        const float f = (m_run[h] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run[h] - M);
        if (half == 0) {
            float *dst = rows + (wave * GG + h) * kDim + 8 * w;
            *reinterpret_cast<float4v *>(dst) = float4v{acc[h][0] * f, acc[h][1] * f, acc[h][2] * f, acc[h][3] * f};
            *reinterpret_cast<float4v *>(dst + 4) =
                float4v{acc[h][4] * f, acc[h][5] * f, acc[h][6] * f, acc[h][7] * f};
        }
        if (tid == 0) {
            float Ls = 0.f;
            for (int j = 0; j < kValuWaves; ++j)
                Ls += (stat_m[j][h] == -INFINITY) ? 0.f : stat_l[j][h] * __builtin_amdgcn_exp2f(stat_m[j][h] - M);
            resL[h] = Ls;
            if (n_active > 1) {
                float *dstp = reinterpret_cast<float *>(static_cast<char *>(p.workspace) + a.parts_off) +
                              ((static_cast<size_t>(b) * p.n_kv + g) * a.n_splits + s) *
                                  static_cast<size_t>(a.partial_floats);
                dstp[h] = M;
                dstp[kSplitStatPad + h] = Ls;
            }
        }
    }
    __syncthreads();
    float *dst = reinterpret_cast<float *>(static_cast<char *>(p.workspace) + a.parts_off) +
                 ((static_cast<size_t>(b) * p.n_kv + g) * a.n_splits + s) * static_cast<size_t>(a.partial_floats);
    for (int i = tid; i < GG * (kDim / 4); i += kValuThreads) {
        const int h = i / (kDim / 4), d4 = i % (kDim / 4);
        float4v sum = *reinterpret_cast<const float4v *>(rows + h * kDim + 4 * d4);
#pragma unroll
        for (int j = 1; j < kValuWaves; ++j) sum += *reinterpret_cast<const float4v *>(rows + (j * GG + h) * kDim + 4 * d4);
        if (n_active > 1)
            *reinterpret_cast<float4v *>(dst + 2 * kSplitStatPad + h * kDim + 4 * d4) = sum;
        else
            *reinterpret_cast<float4v *>(&qsh[h][4 * d4]) = sum;  // the query rows are no longer needed
    }
    if (n_active > 1) return;
    __syncthreads();
    // ---- single split: the output rows, o = H O / (256 L) (rotated) or O / L (literal)
    for (int h = wave; h < GG; h += kValuWaves) {
        const float4v v = *reinterpret_cast<const float4v *>(&qsh[h][4 * lane]);
        float y[4] = {v[0], v[1], v[2], v[3]};
        const float Lh = resL[h];
        float f = Lh > 0.f ? 1.0f / Lh : 0.f;
        if constexpr (!kLiteral) {
            wave_fwht(y, lane);
            f *= 1.0f / 256.0f;
        }
        u32x2 o;
        o.x = static_cast<uint32_t>(f32_to_bf16(y[0] * f)) | (static_cast<uint32_t>(f32_to_bf16(y[1] * f)) << 16);
        o.y = static_cast<uint32_t>(f32_to_bf16(y[2] * f)) | (static_cast<uint32_t>(f32_to_bf16(y[3] * f)) << 16);
        *reinterpret_cast<u32x2 *>(p.out + row_off(h) + 4 * lane) = o;
    }
}

template <bool kLiteral>
static hipError_t launch_valu_group(const ValuArgs &a, const dim3 &grid, hipStream_t stream) {
    switch (a.group) {
        case 1: hipLaunchKernelGGL((tq4_attn_valu_kernel<kLiteral, 1>), grid, dim3(kValuThreads), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((tq4_attn_valu_kernel<kLiteral, 2>), grid, dim3(kValuThreads), 0, stream, a); break;
        case 4: hipLaunchKernelGGL((tq4_attn_valu_kernel<kLiteral, 4>), grid, dim3(kValuThreads), 0, stream, a); break;
        case 6: hipLaunchKernelGGL((tq4_attn_valu_kernel<kLiteral, 6>), grid, dim3(kValuThreads), 0, stream, a); break;
        case 8: hipLaunchKernelGGL((tq4_attn_valu_kernel<kLiteral, 8>), grid, dim3(kValuThreads), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_valu(const DecodeParams &p, const DecodePlan &plan, bool literal, hipStream_t stream) {
    ValuArgs a;
    a.p = p;
    a.group = plan.group;
    a.n_splits = plan.n_splits;
    a.split_tiles = plan.split_tiles;
    a.partial_floats = static_cast<int32_t>(plan.partial_floats);
    a.parts_off = plan.counters_bytes;
    lut_pairs_from_codebook(a.lut_pairs, codebook().centroid);
    for (int i = 0; i < 16; ++i) a.centroid[i] = codebook().centroid[i];
    const dim3 grid(plan.n_splits, p.n_kv, p.batch);
    const hipError_t e = literal ? launch_valu_group<true>(a, grid, stream) : launch_valu_group<false>(a, grid, stream);
    if (e != hipSuccess) return e;
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
        c.n_queries = 1;
        c.n_q = p.n_q;
        c.n_kv = p.n_kv;
        c.batch = p.batch;
        return launch_split_combine(c, !literal, stream);
    }
    return hipGetLastError();
}

}  // namespace tq4
