// tq4_encode_wave.h -- one wavefront encodes one 256-dim vector into a TQ4 record.
//
// Record format: "Fitting a 27B-Parameter LLM into 24 GiB of Laptop Memory", section "KVExec:
// Fused Reconstruction with Layer-Scoped Lifetime" (32 u32 words of eight 4-bit indices plus one
// fp16 norm).  The arithmetic is fixed so every implementation produces the same bits: fp32,
// round-to-nearest-even, no contraction into fused multiply-adds;
//   n   = sqrt( stride-halving tree sum of x_d^2 )       (correctly rounded)
//   y   = H x, butterflies (a, b) -> (a + b, a - b) in stages h = 1, 2, ..., 128
//   idx = #{ i : y_d > b_i * (16 n) }, b_i = midpoints of adjacent centroids
//   word k = sum_j idx[8k + j] << 4j,  norm = fp16(n)
// Lane l holds dims 4l .. 4l+3 (one 16-byte load of an fp32 source).  Hadamard stages 1 and 2
// and tree strides 2 and 1 stay in registers; the others pair lane l with lane l ^ (h / 4).
#pragma once

#include "tq4_device.h"

namespace tq4 {

// Lane l's four source values (dims 4l .. 4l+3) of a 256-dim fp32 or bf16 vector.
__device__ __forceinline__ void encode_load(const void *src, bool bf16, int lane, float x[4]) {
    if (bf16) {
        const u32x2 raw = *reinterpret_cast<const u32x2 *>(
            static_cast<const uint16_t *>(src) + 4 * lane);
        x[0] = __uint_as_float(raw.x << 16);
        x[1] = __uint_as_float(raw.x & 0xffff0000u);
        x[2] = __uint_as_float(raw.y << 16);
        x[3] = __uint_as_float(raw.y & 0xffff0000u);
    } else {
        const float4 raw = *reinterpret_cast<const float4 *>(
            static_cast<const float *>(src) + 4 * lane);
        x[0] = raw.x;
        x[1] = raw.y;
        x[2] = raw.z;
        x[3] = raw.w;
    }
}

// Both halves of a butterfly in one add: lanes in the upper half of a pair compute
// other + (-y), which is the same IEEE operation as other - y; lanes in the lower half compute
// other + y, equal to y + other.
__device__ __forceinline__ float flip_if(float y, bool upper) {
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, y) ^ (upper ? 0x80000000u : 0u));
}

template <int M>
__device__ __forceinline__ void enc_stage(float y[4], int lane) {  // Hadamard stage h = 4 M
    const bool upper = (lane & M) != 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if constexpr (M >= 16) {
            // lower lane: lo + hi; upper lane: lo - hi = lo + (-hi)
            float lo, hi;
            lane_pair<M>(y[r], lo, hi);
            y[r] = lo + flip_if(hi, upper);
        } else {
            y[r] = lane_xor<M>(y[r], lane) + flip_if(y[r], upper);
        }
    }
}

template <int M>
__device__ __forceinline__ void norm_stage(float s[4], int lane) {  // tree strides 4 M
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if constexpr (M >= 16) {
            float lo, hi;
            lane_pair<M>(s[r], lo, hi);
            s[r] = lo + hi;  // both lanes of a pair: s[i] + s[i + stride]
        } else {
            s[r] = s[r] + lane_xor<M>(s[r], lane);
        }
    }
}

// Encodes the vector whose lane values encode_load returned: returns the fp32 norm and sets
// word = the packed word (8 indices) that even lane 2k stores as word k.
__device__ __forceinline__ float encode_compute(const float x[4], const float thr[15], int lane, uint32_t &word) {
#pragma clang fp contract(off)
    // ---- squared norm: strides 128 .. 4 are lane strides 32 .. 1, then 2 and 1 in registers.
    // Pairing element e with e ^ stride on every lane reproduces the tree, since fp32 addition
    // is commutative.
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = x[r] * x[r];
    norm_stage<32>(s, lane);
    norm_stage<16>(s, lane);
    norm_stage<8>(s, lane);
    norm_stage<4>(s, lane);
    norm_stage<2>(s, lane);
    norm_stage<1>(s, lane);
    s[0] = s[0] + s[2];
    s[1] = s[1] + s[3];
    s[0] = s[0] + s[1];
    const float n32 = __builtin_sqrtf(s[0]);  // correctly rounded in LLVM's AMDGPU lowering

    // ---- y = H x, ascending stages
    float y[4] = {x[0], x[1], x[2], x[3]};
    {
        float t0 = y[0] + y[1], t1 = y[0] - y[1], t2 = y[2] + y[3], t3 = y[2] - y[3];  // h = 1
        y[0] = t0 + t2;  // h = 2
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

    // ---- thresholds and indices.  idx = #{ i : y > t_i }, t_i = b_i * (16 n).  The thresholds
    // are exact negatives of each other (b_14-i = -b_i, b_7 = 0), so with a = |y|:
    //   y > 0:  idx = 8 + #{ j >= 8 : a > t_j }
    //   y <= 0: idx = #{ j >= 8 : a < t_j } = 7 - #{ j >= 8 : a >= t_j },
    // and a >= t is a' > t for a' the next float above a.
    const float mscale = 16.0f * n32;
    float t[7];
#pragma unroll
    for (int j = 0; j < 7; ++j) t[j] = thr[8 + j] * mscale;
    uint32_t idx[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bool pos = y[r] > 0.0f;
        const uint32_t abits = __builtin_bit_cast(uint32_t, y[r]) & 0x7fffffffu;
        const float a = __builtin_bit_cast(float, pos ? abits : abits + 1u);
        uint32_t c = 0;
#pragma unroll
        for (int j = 0; j < 7; ++j) c += (a > t[j]) ? 1u : 0u;
        idx[r] = pos ? 8u + c : 7u - c;
    }

    // ---- pack: lanes 2k and 2k+1 hold dims 8k .. 8k+7
    const uint32_t half16 = idx[0] | (idx[1] << 4) | (idx[2] << 8) | (idx[3] << 12);
    const uint32_t other16 = lane_xor<1>(half16, lane);
    word = half16 | (other16 << 16);
    return n32;
}

// Encodes the vector whose lane values encode_load returned; writes 32 words and the fp16 norm.
__device__ __forceinline__ void encode_values(const float x[4], const float thr[15], uint32_t *words,
                                              uint16_t *norm, int lane) {
    uint32_t word;
    const float n32 = encode_compute(x, thr, lane, word);
    if ((lane & 1) == 0) words[lane >> 1] = word;
    if (lane == 0) *norm = f32_to_f16_bits(n32);
}

// src: 256 fp32 (bf16 == false) or bf16 values; writes 32 words and the fp16 norm.
__device__ __forceinline__ void encode_vector_wave(const void *src, bool bf16, const float thr[15],
                                                   uint32_t *words, uint16_t *norm, int lane) {
    float x[4];
    encode_load(src, bf16, lane, x);
    encode_values(x, thr, words, norm, lane);
}

}  // namespace tq4
