// tq4_encode.hip -- TQ4 encoder for gfx950: four vectors per wavefront, 16 lanes per vector.
//
// Record format and the decode steps it must invert: "Fitting a 27B-Parameter LLM into 24 GiB of
// Laptop Memory", section "KVExec: Fused Reconstruction with Layer-Scoped Lifetime" (32 u32 words
// of eight 4-bit indices plus one fp16 norm; centroid lookup, inverse Hadamard rotation, norm
// restore).  The per-vector arithmetic is the one tq4_encode_wave.h fixes (fp32, round to nearest
// even, no contraction):
//   n   = sqrt( stride-halving tree sum of x_d^2 ),   y = H x in ascending stages h = 1 .. 128,
//   idx = #{ i : y_d > b_i * (16 n) },                 word k = sum_j idx[8k + j] << 4j.
// Here lane g (0 .. 15) of a 16-lane group holds dims 16 g .. 16 g + 15 of its vector, so tree
// strides 8 .. 1 and Hadamard stages 1 .. 8 are register operations, and strides 128 .. 16 and
// stages 16 .. 128 pair lane g with lane g ^ 8 .. g ^ 1 inside one 16-lane row (DPP moves, no
// cross-row swaps).  Every addition pairs the same two values as in the definition, so the
// records are bit-identical to it.
#pragma clang fp contract(off)

#include "tq4_device.h"
#include "tq4_encode_wave.h"
#include "tq4_launch.h"

namespace tq4 {

struct EncodeArgs {
    EncodeParams p;
    float thr[15];
};

constexpr int kEncWaves = 4;                 // wavefronts per workgroup
constexpr int kEncVecsPerWave = 4;           // one vector per 16-lane group
constexpr int64_t kEncMaxWorkgroups = 2048;  // 8 per CU (all resident): each wavefront loops
constexpr int kEncDropOffset = 0x40000000;   // a buffer offset past any record: the store is dropped
constexpr int kBufferFlags = 0x00020000;     // raw 32-bit buffer resource word 3

// Lane g's 16 source values (dims 16 g .. 16 g + 15) of one 256-dim fp32 or bf16 vector.
template <bool BF16>
__device__ __forceinline__ void load16(const char *vec, int g, float x[16]) {
    if constexpr (BF16) {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(vec + 32 * g);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4 r = p[h];
            const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[8 * h + 2 * k] = __uint_as_float(w[k] << 16);
                x[8 * h + 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
            }
        }
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(vec + 64 * g);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const float4 r = p[h];
            x[4 * h] = r.x;
            x[4 * h + 1] = r.y;
            x[4 * h + 2] = r.z;
            x[4 * h + 3] = r.w;
        }
    }
}

// Tree stride 16 M: element e of lane g and of lane g ^ M (commutative, so both lanes of the pair
// get s[i] + s[i + stride]).
template <int M>
__device__ __forceinline__ void norm_cross16(float s[16], int lane) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = s[e] + lane_xor<M>(s[e], lane);
}

// Hadamard stage 16 M: lower lane of the pair lo + hi, upper lane lo - hi = lo + (-hi).
template <int M>
__device__ __forceinline__ void hadamard_cross16(float y[16], int lane) {
    const bool upper = (lane & M) != 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) y[e] = lane_xor<M>(y[e], lane) + flip_if(y[e], upper);
}

// Encodes the vector whose 16-lane group holds x (lane g: dims 16 g ..); returns the fp32 norm and
// the lane's two words (2 g and 2 g + 1).
__device__ __forceinline__ float encode16(const float x[16], const float thr[15], int lane, u32x2 &words) {
#pragma clang fp contract(off)
    const int g = lane & 15;
    // ---- squared norm.  Strides 128, 64, 32, 16 pair lane g with g ^ 8, 4, 2, 1 (element e with
    // itself); both lanes of a pair form s[i] + s[i + stride], as the tree does for i < stride.
    // Then strides 8, 4, 2, 1 inside the lane.
    float s[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = x[e] * x[e];
    norm_cross16<8>(s, lane);
    norm_cross16<4>(s, lane);
    norm_cross16<2>(s, lane);
    norm_cross16<1>(s, lane);
#pragma unroll
    for (int st = 8; st >= 1; st >>= 1)
#pragma unroll
        for (int e = 0; e < st; ++e) s[e] = s[e] + s[e + st];
    const float n32 = __builtin_sqrtf(s[0]);  // correctly rounded in LLVM's AMDGPU lowering

    // ---- y = H x: stages 1, 2, 4, 8 in registers, then 16 .. 128 across lanes (lower lane of a
    // pair: lo + hi; upper lane: lo - hi = lo + (-hi))
    float y[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) y[e] = x[e];
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            if ((e & h) == 0) {
                const float a = y[e], b = y[e + h];
                y[e] = a + b;
                y[e + h] = a - b;
            }
    hadamard_cross16<1>(y, lane);
    hadamard_cross16<2>(y, lane);
    hadamard_cross16<4>(y, lane);
    hadamard_cross16<8>(y, lane);

    // ---- indices.  With a = |y| (or the next float above it for y <= 0) and t_j = b_{8+j}(16 n)
    // ascending, c = #{ j : a > t_j } by a three-level search (sorted thresholds); idx = 8 + c for
    // y > 0, else 7 - c (the thresholds are exact negatives of each other, b_7 = 0).
    const float mscale = 16.0f * n32;
    float t[7];
#pragma unroll
    for (int j = 0; j < 7; ++j) t[j] = thr[8 + j] * mscale;
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const bool pos = y[e] > 0.0f;
        const uint32_t abits = __builtin_bit_cast(uint32_t, y[e]) & 0x7fffffffu;
        const float a = __builtin_bit_cast(float, pos ? abits : abits + 1u);
        const bool c4 = a > t[3];
        const bool c2 = a > (c4 ? t[5] : t[1]);
        const bool c1 = a > (c4 ? (c2 ? t[6] : t[4]) : (c2 ? t[2] : t[0]));
        const uint32_t c = (c4 ? 4u : 0u) + (c2 ? 2u : 0u) + (c1 ? 1u : 0u);
        const uint32_t idx = pos ? 8u + c : 7u - c;
        if (e < 8)
            w0 |= idx << (4 * e);
        else
            w1 |= idx << (4 * (e - 8));
    }
    words = u32x2{w0, w1};
    return n32;
}

// Each wavefront encodes groups of four vectors, group0, group0 + stride, ... (vectors in [half]
// [token][kv head] order, lane group q takes vector 4 G + q).  The next group's sources and slots
// are requested before the current group is encoded.  Records are written through buffer
// resources that cover exactly one record (or nothing for a slot outside the pool or a vector past
// the end): one store per lane group, in which only that group's lanes have an in-range offset.
template <bool BF16>
__global__ __launch_bounds__(kEncWaves * kWave) void tq4_encode_kernel(EncodeArgs a) {
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, g = lane & 15;
    const int group0 = static_cast<int>(blockIdx.x) * kEncWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int stride = static_cast<int>(gridDim.x) * kEncWaves;
    const int per_half = a.p.n_tokens * a.p.n_kv;
    const int first_half = a.p.src[0] != nullptr ? 0 : 1;
    const int total = per_half * ((a.p.src[0] != nullptr) + (a.p.src[1] != nullptr));
    const int n_groups = (total + kEncVecsPerWave - 1) / kEncVecsPerWave;
    if (group0 >= n_groups) return;
    constexpr size_t esize = BF16 ? 2 : 4;
    auto half_of = [&](int vec) { return first_half + static_cast<int>(vec >= per_half); };
    auto rem_of = [&](int vec) { return vec - (vec >= per_half ? per_half : 0); };
    // this lane's vector of group G (clamped to the last vector; past the end it is not stored)
    auto vec_of = [&](int G) { return min(G * kEncVecsPerWave + q, total - 1); };
    auto load = [&](int G, float x[16], int &slot) {
        const int vec = vec_of(G);
        const int rem = rem_of(vec);
        load16<BF16>(static_cast<const char *>(a.p.src[half_of(vec)]) + static_cast<int64_t>(rem) * kDim * esize, g, x);
        slot = a.p.slots[rem / a.p.n_kv];
    };
    auto encode_store = [&](int G, const float x[16], int slot, bool live_group) {
        u32x2 words;
        const float n32 = encode16(x, a.thr, lane, words);
        const uint16_t n16 = f32_to_f16_bits(n32);
#pragma unroll
        for (int qq = 0; qq < kEncVecsPerWave; ++qq) {
            const int vec = G * kEncVecsPerWave + qq;
            const int vq = min(vec, total - 1);
            const int half = half_of(vq);
            const int head = rem_of(vq) % a.p.n_kv;
            const int s_u = __builtin_amdgcn_readlane(slot, 16 * qq);
            const bool valid = live_group && vec < total && s_u >= 0 && s_u < a.p.num_slots;
            const int sl = valid ? s_u : 0;
            const int page = sl / a.p.page_size;
            const int64_t rec =
                (static_cast<int64_t>(page) * a.p.n_kv + head) * a.p.page_size + (sl - page * a.p.page_size);
            const __amdgpu_buffer_rsrc_t wr =
                __builtin_amdgcn_make_buffer_rsrc(a.p.words[half] + rec * kWords, 0, valid ? kWords * 4 : 0, kBufferFlags);
            const __amdgpu_buffer_rsrc_t nr =
                __builtin_amdgcn_make_buffer_rsrc(a.p.norms[half] + rec, 0, valid ? 2 : 0, kBufferFlags);
            const int word_off = q == qq ? 8 * g : kEncDropOffset;
            const int norm_off = (q == qq && g == 0) ? 0 : kEncDropOffset;
            __builtin_amdgcn_raw_buffer_store_b64(words, wr, word_off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b16(n16, nr, norm_off, 0, 0);
        }
    };

    // two register sets used in turn (no copies between iterations)
    float x0[16], x1[16];
    int slot0, slot1;
    load(group0, x0, slot0);
    {   // dropped stores: the loop is entered with the same pending operations as its back edge
        const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(a.p.words[half_of(0)], 0, 0, kBufferFlags);
#pragma unroll
        for (int qq = 0; qq < kEncVecsPerWave; ++qq) {
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, none, kEncDropOffset, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(0), none, kEncDropOffset, 0, 0);
        }
    }
    for (int G = group0; G < n_groups; G += 2 * stride) {
        const bool live1 = G < n_groups - stride;
        const int G1 = live1 ? G + stride : G;
        load(G1, x1, slot1);
        __builtin_amdgcn_sched_barrier(0);  // requested before this group's work
        encode_store(G, x0, slot0, true);
        const int G2 = G < n_groups - 2 * stride ? G + 2 * stride : G;
        load(G2, x0, slot0);
        __builtin_amdgcn_sched_barrier(0);
        encode_store(G1, x1, slot1, live1);
    }
}

hipError_t launch_encode(const EncodeParams &p, hipStream_t stream) {
    EncodeArgs a;
    a.p = p;
    const Codebook &cb = codebook();
    for (int i = 0; i < 15; ++i) a.thr[i] = cb.threshold[i];
    const int halves = (p.src[0] != nullptr) + (p.src[1] != nullptr);
    const int64_t vectors = static_cast<int64_t>(halves) * p.n_tokens * p.n_kv;
    if (vectors == 0) return hipSuccess;
    if (vectors > 0x7fffffff - 2 * kEncMaxWorkgroups * kEncWaves * kEncVecsPerWave) return hipErrorInvalidValue;
    const int64_t groups = (vectors + kEncVecsPerWave - 1) / kEncVecsPerWave;
    int64_t blocks = (groups + kEncWaves - 1) / kEncWaves;
    if (blocks > kEncMaxWorkgroups) blocks = kEncMaxWorkgroups;
    if (p.src_bf16)
        hipLaunchKernelGGL(tq4_encode_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kEncWaves * kWave), 0, stream, a);
    else
        hipLaunchKernelGGL(tq4_encode_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kEncWaves * kWave), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tq4
