// tq4_tile.h -- per-lane machinery shared by the gfx950 attention kernels of this
// library: loading a 32-key TQ4 tile, turning 4-bit indices into fp16 MFMA
// operands through an LDS centroid table, the 8x8 nibble transpose for value
// operands, and a wavefront-wide Hadamard transform.
//
// Lane layout (lane = 16 * gq + n) of a 32-key tile for v_mfma_f32_16x16x32_f16:
//   scores S^T = K Q^T: M-tile mt (keys 16 mt .. 16 mt + 15), K-step ks covers dims of word
//     16 (ks / 4) + 4 gq + (ks % 4); the A operand of lane (gq, n) is that word of key 16 mt + n.
//   S^T results: lane (gq, n) holds column n, keys sigma(j) = j < 4 ? 4 gq + j : 16 + 4 gq + j - 4.
//   values O^T = V^T P^T: the B operand (P^T) of lane (gq, n) holds column n at keys sigma(0..7);
//     the A operand of M-tile (c, i) holds dim 8 (2 n + c) + i of keys sigma(0..7), produced by
//     transposing words 2n + c of those 8 keys.
#pragma once

#include "tq4_device.h"

namespace tq4 {

constexpr int kTile = 32;
constexpr int kLutEntries = 256;
constexpr int kLutWords = kLutEntries * kWave;  // 64 KiB: one table row of 64 copies per entry


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

// Two fp32 -> packed fp16 (lo in the low half) with one v_cvt_pk_f16_f32, round to nearest even:
// the same bits as two f32_to_f16_bits conversions.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){lo, hi}, f16x2_t));
}

// First record of a tile (page `pid`, in-page offset of key0); page IDs outside the pool map to
// page 0 and the tile is masked.
template <class Pool>
__device__ __forceinline__ int64_t tile_rec0(const Pool &p, int g, int key0, int pid, bool &valid) {
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

template <class Pool>
__device__ __forceinline__ void load_k(const Pool &p, int64_t rec0, const LaneOffsets &o, KRegs &t) {
    const char *wb = reinterpret_cast<const char *>(p.k_words) + rec0 * (kWords * 4);
    const char *nb = reinterpret_cast<const char *>(p.k_norms) + rec0 * 2;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h) t.k[mt][h] = *reinterpret_cast<const u32x4 *>(wb + o.k + (2048u * mt + 64u * h));
#pragma unroll
    for (int h = 0; h < 2; ++h) t.kn[h] = *reinterpret_cast<const u32x2 *>(nb + o.nrm + 32u * h);
}

template <class Pool>
__device__ __forceinline__ void load_v(const Pool &p, int64_t rec0, const LaneOffsets &o, VRegs &t) {
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

// One stage h = 4 M of wave_fwht below: lane l pairs with lane l ^ M (DPP moves or the
// lane-swap instructions, no LDS crossbar); the lower lane keeps a + b, the upper a - b.
template <int M>
__device__ __forceinline__ void wave_fwht_stage(float y[4], int lane) {
    const bool upper = (lane & M) != 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if constexpr (M >= 16) {
            float lo, hi;
            lane_pair<M>(y[r], lo, hi);
            y[r] = upper ? (lo - hi) : (lo + hi);
        } else {
            const float o = lane_xor<M>(y[r], lane);
            y[r] = upper ? (o - y[r]) : (y[r] + o);
        }
    }
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
    wave_fwht_stage<1>(y, lane);
    wave_fwht_stage<2>(y, lane);
    wave_fwht_stage<4>(y, lane);
    wave_fwht_stage<8>(y, lane);
    wave_fwht_stage<16>(y, lane);
    wave_fwht_stage<32>(y, lane);
}


// Fill the centroid table: entry e (a nibble pair) -> fp16x2 (16 c[e & 15], 16 c[e >> 4]), one
// copy per lane so each 256-byte row holds one entry; written 16 bytes at a time, 16 per entry.
// With NT threads (256, 512 or 1024), thread t writes entries e = (t >> 4) + (NT >> 4) k, so its
// low nibble (t >> 4) & 15 never changes and its high nibble is (t >> 8) + (NT >> 8) k.  The pair
// words are taken into scalar registers and picked by selects over named values: an indexed
// read of the argument array would be a vector memory load, and waiting for it would also wait
// for every tile load already in flight.
template <int NT>
__device__ __forceinline__ void build_lut(uint32_t *lut_mem, const uint32_t lut_pairs[8], int tid) {
    static_assert(NT == 256 || NT == 512 || NT == 1024, "table fill assumes 256, 512 or 1024 threads");
    uint32_t l[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) l[k] = __builtin_amdgcn_readfirstlane(lut_pairs[k]);
    const uint32_t c_lo = (static_cast<uint32_t>(tid) >> 4) & 15u;
    const uint32_t k0 = c_lo >> 1;  // select tree, once per thread
    const uint32_t a0 = (k0 & 1) ? l[1] : l[0], a1 = (k0 & 1) ? l[3] : l[2];
    const uint32_t a2 = (k0 & 1) ? l[5] : l[4], a3 = (k0 & 1) ? l[7] : l[6];
    const uint32_t b0 = (k0 & 2) ? a1 : a0, b1 = (k0 & 2) ? a3 : a2;
    const uint32_t w_lo = (k0 & 4) ? b1 : b0;
    const uint32_t v_lo = (c_lo & 1) ? (w_lo >> 16) : (w_lo & 0xffffu);
    const uint32_t t8 = static_cast<uint32_t>(tid) >> 8;  // 0 .. NT / 256 - 1
#pragma unroll
    for (int k = 0; k < kLutWords / 4 / NT; ++k) {
        // high nibble c = t8 + (NT / 256) k: word c / 2 of the pair table, half c & 1
        uint32_t w;
        if constexpr (NT == 256) {
            w = l[k >> 1];
        } else {
            const int base = (NT / 256) * k;  // even: t8 picks among words base / 2 ..
            const uint32_t c = t8 + static_cast<uint32_t>(base);
            w = l[base >> 1];
#pragma unroll
            for (int j = 1; j < NT / 512; ++j) w = ((c >> 1) == static_cast<uint32_t>((base >> 1) + j)) ? l[(base >> 1) + j] : w;
        }
        const uint32_t c = (NT == 256) ? static_cast<uint32_t>(k) : t8 + static_cast<uint32_t>((NT / 256) * k);
        const uint32_t v_hi = (c & 1) ? (w >> 16) : (w & 0xffffu);
        const uint32_t v = v_lo | (v_hi << 16);
        reinterpret_cast<u32x4 *>(lut_mem)[tid + NT * k] = u32x4{v, v, v, v};
    }
}

// fp16 bits of 16 * centroid, two per word, from the host codebook.
inline void lut_pairs_from_codebook(uint32_t out[8], const float centroid[16]) {
    for (int k = 0; k < 8; ++k) {
        const _Float16 lo = static_cast<_Float16>(16.0f * centroid[2 * k]);
        const _Float16 hi = static_cast<_Float16>(16.0f * centroid[2 * k + 1]);
        out[k] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                 (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
    }
}

// Wave-uniform power-of-two scale putting max |y| of a rotated query row in [2^13, 2^14) for
// the fp16 operand; returns the exponent e (the scale is 2^e).
__device__ __forceinline__ int q_exponent(float max_abs) {
    int e = 0;
    if (max_abs > 0.f) {
        int E;
        frexpf(max_abs, &E);
        e = 14 - E;
    }
    return e;
}

}  // namespace tq4
