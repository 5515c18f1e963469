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

__device__ __forceinline__ float enc_xor_lane(float v, int mask) { return __shfl_xor(v, mask, kWave); }

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

// Encodes the vector whose lane values encode_load returned; writes 32 words and the fp16 norm.
__device__ __forceinline__ void encode_values(const float x[4], const float thr[15], uint32_t *words,
                                              uint16_t *norm, int lane) {
#pragma clang fp contract(off)
    // ---- squared norm: strides 128 .. 4 are lane strides 32 .. 1, then 2 and 1 in registers.
    // Pairing element e with e ^ stride on every lane reproduces the tree, since fp32 addition
    // is commutative.
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = x[r] * x[r];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] = s[r] + enc_xor_lane(s[r], m);
    }
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
#pragma unroll
    for (int m = 1; m <= 32; m <<= 1) {  // h = 4 m
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float other = enc_xor_lane(y[r], m);
            y[r] = upper ? (other - y[r]) : (y[r] + other);
        }
    }

    // ---- thresholds and indices
    const float mscale = 16.0f * n32;
    uint32_t idx[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 15; ++i) {
        const float t = thr[i] * mscale;
#pragma unroll
        for (int r = 0; r < 4; ++r) idx[r] += (y[r] > t) ? 1u : 0u;
    }

    // ---- pack: lanes 2k and 2k+1 hold dims 8k .. 8k+7
    const uint32_t half16 = idx[0] | (idx[1] << 4) | (idx[2] << 8) | (idx[3] << 12);
    const uint32_t other16 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(half16), 1, kWave));
    if ((lane & 1) == 0) words[lane >> 1] = half16 | (other16 << 16);
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
