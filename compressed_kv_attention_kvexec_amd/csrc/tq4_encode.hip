// tq4_encode.hip -- TQ4 encoder for gfx950: one wavefront per 256-dim vector.
//
// Record format and the decode steps it must invert: "Fitting a 27B-Parameter
// LLM into 24 GiB of Laptop Memory", section "KVExec: Fused Reconstruction
// with Layer-Scoped Lifetime" (32 u32 words of eight 4-bit indices plus one
// fp16 norm; centroid lookup, inverse Hadamard rotation, norm restore).
//
// The arithmetic is fixed so that every implementation gets the same bits:
// fp32, round-to-nearest-even, no contraction into fused multiply-adds;
//   n   = sqrt( stride-halving tree sum of x_d^2 )       (correctly rounded)
//   y   = H x, butterflies (a, b) -> (a + b, a - b) in stages h = 1, 2, ..., 128
//   idx = #{ i : y_d > b_i * (16 n) }, b_i = midpoints of adjacent centroids
//   word k = sum_j idx[8k + j] << 4j,  norm = fp16(n)
//
// Lane layout: lane l holds dims 4l .. 4l+3 (one 16-byte load of fp32 source).
// Hadamard stages 1 and 2 and tree strides 2 and 1 stay in registers; the
// others pair lane l with lane l ^ (h / 4).
#pragma clang fp contract(off)

#include "tq4_device.h"
#include "tq4_launch.h"

namespace tq4 {

struct EncodeArgs {
    EncodeParams p;
    float thr[15];
};

__device__ __forceinline__ float xor_lane(float v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

__global__ __launch_bounds__(256) void tq4_encode_kernel(EncodeArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t vec = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t per_half = static_cast<int64_t>(a.p.n_tokens) * a.p.n_kv;
    // vectors are ordered [half][token][kv head]; halves with no source are not launched
    int half;
    int64_t rem;
    if (a.p.src[0] != nullptr) {
        half = vec < per_half ? 0 : 1;
        rem = vec - half * per_half;
    } else {
        half = 1;
        rem = vec;
    }
    if (rem >= per_half || a.p.src[half] == nullptr) return;
    const int token = static_cast<int>(rem / a.p.n_kv);
    const int head = static_cast<int>(rem % a.p.n_kv);
    const int slot = a.p.slots[token];
    if (slot < 0 || slot >= a.p.num_slots) return;

    // ---- load 4 consecutive dims
    float x[4];
    const int64_t src_off = rem * kDim + 4 * lane;
    if (a.p.src_bf16) {
        const u32x2 raw = *reinterpret_cast<const u32x2 *>(
            static_cast<const uint16_t *>(a.p.src[half]) + src_off);
        x[0] = __uint_as_float(raw.x << 16);
        x[1] = __uint_as_float(raw.x & 0xffff0000u);
        x[2] = __uint_as_float(raw.y << 16);
        x[3] = __uint_as_float(raw.y & 0xffff0000u);
    } else {
        const float4 raw = *reinterpret_cast<const float4 *>(
            static_cast<const float *>(a.p.src[half]) + src_off);
        x[0] = raw.x;
        x[1] = raw.y;
        x[2] = raw.z;
        x[3] = raw.w;
    }

    // ---- squared norm: strides 128 .. 4 are lane strides 32 .. 1, then 2 and 1 in registers.
    // Pairing element e with e ^ stride on every lane reproduces the tree, since fp32 addition
    // is commutative.
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = x[r] * x[r];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] = s[r] + xor_lane(s[r], m);
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
            const float other = xor_lane(y[r], m);
            y[r] = upper ? (other - y[r]) : (y[r] + other);
        }
    }

    // ---- thresholds and indices
    const float mscale = 16.0f * n32;
    uint32_t idx[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 15; ++i) {
        const float t = a.thr[i] * mscale;
#pragma unroll
        for (int r = 0; r < 4; ++r) idx[r] += (y[r] > t) ? 1u : 0u;
    }

    // ---- pack: lanes 2k and 2k+1 hold dims 8k .. 8k+7
    const uint32_t half16 = idx[0] | (idx[1] << 4) | (idx[2] << 8) | (idx[3] << 12);
    const uint32_t other16 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(half16), 1, kWave));
    const int page = slot / a.p.page_size;
    const int off = slot - page * a.p.page_size;
    const int64_t rec = (static_cast<int64_t>(page) * a.p.n_kv + head) * a.p.page_size + off;
    if ((lane & 1) == 0) a.p.words[half][rec * kWords + (lane >> 1)] = half16 | (other16 << 16);
    if (lane == 0) a.p.norms[half][rec] = f32_to_f16_bits(n32);
}

hipError_t launch_encode(const EncodeParams &p, hipStream_t stream) {
    EncodeArgs a;
    a.p = p;
    const Codebook &cb = codebook();
    for (int i = 0; i < 15; ++i) a.thr[i] = cb.threshold[i];
    const int halves = (p.src[0] != nullptr) + (p.src[1] != nullptr);
    const int64_t vectors = static_cast<int64_t>(halves) * p.n_tokens * p.n_kv;
    if (vectors == 0) return hipSuccess;
    const int64_t blocks = (vectors + 3) / 4;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(tq4_encode_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tq4
