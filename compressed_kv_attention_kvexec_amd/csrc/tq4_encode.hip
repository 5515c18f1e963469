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

#include <cfloat>

#include "tq4_device.h"
#include "tq4_encode_wave.h"
#include "tq4_launch.h"

namespace tq4 {

struct EncodeArgs {
    EncodeParams p;
    float thr[15];
    FastDiv by_kv;    // n_kv
    FastDiv by_page;  // page_size
};

constexpr int kEncWaves = 4;                 // wavefronts per workgroup
constexpr int kEncVecsPerWave = 4;           // one vector per 16-lane group
constexpr int64_t kEncMaxWorkgroups = 2048;  // 8 per CU, 6 resident at a time; each wavefront loops

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

// The value of lane (lane ^ M) for M in {1, 2, 4, 8} inside a 16-lane row, as DPP moves whose
// source lane always exists (so no old value has to be kept in the destination).  For M = 4: the
// half-row mirror (lane i of each 8 reads lane 7 - i) and then the quad reversal (lane j of each 4
// reads lane 3 - j).
template <int M>
__device__ __forceinline__ float row_xor(float x, int) {
    const int v = __builtin_bit_cast(int, x);
    int r;
    if constexpr (M == 1) {
        r = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);  // quad_perm 1,0,3,2
    } else if constexpr (M == 2) {
        r = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);  // quad_perm 2,3,0,1
    } else if constexpr (M == 4) {
        r = __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true), 0x1B, 0xF, 0xF, true);
    } else {
        static_assert(M == 8, "row_xor: M is 1, 2, 4 or 8");
        r = __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true);  // row_ror:8
    }
    return __builtin_bit_cast(float, r);
}

// Hadamard stage 16 M: lower lane of the pair lo + hi, upper lane lo - hi = lo + (-hi).  Both are
// one fused multiply-add, own * (+1 or -1) + partner: the product is exact, so the result is the
// rounded sum of the same two values.
template <int M>
__device__ __forceinline__ void hadamard_cross16(float y[16], int lane) {
    const float sgn = (lane & M) != 0 ? -1.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) y[e] = __builtin_fmaf(y[e], sgn, row_xor<M>(y[e], lane));
}

// Row stride (floats) of the squares' transpose area: 17, so the 16 lanes of a row and the four
// vectors of a wavefront fall in different LDS banks.
constexpr int kSqRow = 17;
constexpr int kSqFloats = kEncVecsPerWave * 16 * kSqRow;  // per wavefront

// 2 w + (bit of this lane in mask m), one v_addc_co_u32 with the mask as carry in.  A mask that a
// vector compare has just written needs two wait states before a vector instruction reads it, which
// the compiler does not check inside inline assembly: kFromCompare puts them in front.
template <bool kFromCompare>
__device__ __forceinline__ uint32_t add_twice_carry(uint32_t w, uint64_t m) {
    uint32_t r;
    uint64_t carry_out;
    if constexpr (kFromCompare)
        asm("s_nop 1\n\tv_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(w), "s"(m));
    else
        asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(w), "s"(m));
    return r;
}

// w = 16 w + idx(v): the 4-bit index of coordinate v goes into the word one bit at a time (see the
// index comment in encode16); tb_j = 2 bits(t_j).
__device__ __forceinline__ uint32_t index_bits(uint32_t w, float v, uint32_t tb0, uint32_t tb1, uint32_t tb2,
                                               uint32_t tb3, uint32_t tb4, uint32_t tb5, uint32_t tb6) {
    const uint32_t yb = __builtin_bit_cast(uint32_t, v);
    const uint64_t mp = __builtin_amdgcn_ballot_w64(v > 0.0f);
    const uint32_t key = add_twice_carry<false>(yb, ~mp);  // ~mp: a scalar instruction's result
    const bool c4 = key > tb3;
    const bool c2 = key > (c4 ? tb5 : tb1);
    const uint32_t hi = c2 ? tb6 : tb4, lo = c2 ? tb2 : tb0;
    const bool c1 = key > (c4 ? hi : lo);
    const uint64_t m4 = __builtin_amdgcn_ballot_w64(c4);
    const uint64_t m2 = __builtin_amdgcn_ballot_w64(c2);
    const uint64_t m1 = __builtin_amdgcn_ballot_w64(c1);
    w = add_twice_carry<true>(w, mp);
    w = add_twice_carry<false>(w, ~(m4 ^ mp));
    w = add_twice_carry<false>(w, ~(m2 ^ mp));
    return add_twice_carry<false>(w, ~(m1 ^ mp));
}

// Encodes the vector whose 16-lane group holds x (lane g: dims 16 g ..); returns the fp32 norm and
// the lane's two words (2 g and 2 g + 1).  sq: this lane group's 16 x 17 floats of LDS.
__device__ __forceinline__ float encode16(const float x[16], const float thr[15], int lane, float *sq, u32x2 &words) {
#pragma clang fp contract(off)
    const int g = lane & 15;
    // ---- squared norm.  The tree's strides 128, 64, 32, 16 pair dim 16 g + e with the same e in
    // lanes g ^ 8, 4, 2, 1, and strides 8 .. 1 pair elements inside a lane.  The squares go through
    // LDS transposed (lane g then holds the squares of element g from all 16 lanes, in lane order),
    // so strides 128 .. 16 become additions inside the lane and strides 8 .. 1 four exchanges of one
    // value: the same pairs in the same order as the tree.
    {
        float s[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = x[e] * x[e];
#pragma unroll
        for (int e = 0; e < 16; ++e) sq[g * kSqRow + e] = s[e];
    }
    __builtin_amdgcn_wave_barrier();
    float ts[16];
#pragma unroll
    for (int l = 0; l < 16; ++l) ts[l] = sq[l * kSqRow + g];  // square of dim 16 l + g
#pragma unroll
    for (int st = 8; st >= 1; st >>= 1)
#pragma unroll
        for (int l = 0; l < st; ++l) ts[l] = ts[l] + ts[l + st];
    float s0 = ts[0];  // strides 128 .. 16 done for element g; strides 8 .. 1 pair lanes
    s0 = s0 + row_xor<8>(s0, lane);
    s0 = s0 + row_xor<4>(s0, lane);
    s0 = s0 + row_xor<2>(s0, lane);
    s0 = s0 + row_xor<1>(s0, lane);
    const float n32 = __builtin_sqrtf(s0);  // correctly rounded in LLVM's AMDGPU lowering

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

    // ---- indices: idx = #{ i : y > b_i (16 n) } over the 15 ascending thresholds.
    const float mscale = 16.0f * n32;
    uint32_t w0 = 0, w1 = 0;
    if (__all(n32 <= FLT_MAX)) {
        // Every norm of the wavefront is finite, so n < 2^64 (its square did not overflow) and y and
        // the thresholds are finite (|y| <= 16 n).  The
        // thresholds are exact negatives of each other (b_7 = 0), so with c = #{ j : t_j < |y| } for
        // y > 0 and c = #{ j : t_j <= |y| } otherwise (t_j = b_{8+j} (16 n), j = 0 .. 6), idx is
        // 8 + c or 7 - c, i.e. bit 3 = [y > 0] and bits 2 .. 0 those of c, each flipped for y <= 0.
        // Compared as integers: key = 2 bits(y) + [y <= 0] (the doubling drops the sign) against
        // 2 bits(t_j) orders both cases at once.  c comes from a three-level search; the nibble
        // goes into the word one bit at a time, w = 2 w + bit, highest element first.
        const uint32_t tb0 = 2u * __builtin_bit_cast(uint32_t, thr[8] * mscale);
        const uint32_t tb1 = 2u * __builtin_bit_cast(uint32_t, thr[9] * mscale);
        const uint32_t tb2 = 2u * __builtin_bit_cast(uint32_t, thr[10] * mscale);
        const uint32_t tb3 = 2u * __builtin_bit_cast(uint32_t, thr[11] * mscale);
        const uint32_t tb4 = 2u * __builtin_bit_cast(uint32_t, thr[12] * mscale);
        const uint32_t tb5 = 2u * __builtin_bit_cast(uint32_t, thr[13] * mscale);
        const uint32_t tb6 = 2u * __builtin_bit_cast(uint32_t, thr[14] * mscale);
#pragma unroll
        for (int e = 7; e >= 0; --e) {
            w0 = index_bits(w0, y[e], tb0, tb1, tb2, tb3, tb4, tb5, tb6);
            w1 = index_bits(w1, y[e + 8], tb0, tb1, tb2, tb3, tb4, tb5, tb6);
        }
    } else {
        // an infinite or NaN norm in the wavefront: the count itself, over all 15 thresholds
        float t[15];
#pragma unroll
        for (int i = 0; i < 15; ++i) t[i] = thr[i] * mscale;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            uint32_t idx = 0;
#pragma unroll
            for (int i = 0; i < 15; ++i) idx += y[e] > t[i] ? 1u : 0u;
            if (e < 8)
                w0 |= idx << (4 * e);
            else
                w1 |= idx << (4 * (e - 8));
        }
    }
    words = u32x2{w0, w1};
    return n32;
}

// Each wavefront encodes groups of four vectors, group0, group0 + stride, ... (vectors in [half]
// [token][kv head] order, lane group q takes vector 4 G + q).  The next group's sources and slots
// are requested before the current group is encoded.  Each lane computes its vector's record
// address itself and the wavefront writes the four records with one 8-byte store per lane and one
// norm store (lanes with g = 0); a slot outside the pool or a vector past the end is not written.
// Six wavefronts per SIMD (at most 85 registers each, none spilled): measured faster than five.
// Divisions by n_kv and page_size are multiplications by host-computed constants.
template <bool BF16>
__global__ __launch_bounds__(kEncWaves * kWave) __attribute__((amdgpu_waves_per_eu(6, 6))) void tq4_encode_kernel(EncodeArgs a) {
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, g = lane & 15;
    const int group0 = static_cast<int>(blockIdx.x) * kEncWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int stride = static_cast<int>(gridDim.x) * kEncWaves;
    const int per_half = a.p.n_tokens * a.p.n_kv;
    const int first_half = a.p.src[0] != nullptr ? 0 : 1;
    // the two halves' pointers, read once (an index into the argument array would be a scalar
    // load and wait at every use)
    const char *const src0 = static_cast<const char *>(a.p.src[0]), *const src1 = static_cast<const char *>(a.p.src[1]);
    uint32_t *const words0 = a.p.words[0], *const words1 = a.p.words[1];
    uint16_t *const norms0 = a.p.norms[0], *const norms1 = a.p.norms[1];
    const int total = per_half * ((a.p.src[0] != nullptr) + (a.p.src[1] != nullptr));
    const int n_groups = (total + kEncVecsPerWave - 1) / kEncVecsPerWave;
    if (group0 >= n_groups) return;
    __shared__ float sq_all[kEncWaves * kSqFloats];
    float *const sq = sq_all + (threadIdx.x >> 6) * kSqFloats + q * 16 * kSqRow;
    constexpr size_t esize = BF16 ? 2 : 4;
    auto half_of = [&](int vec) { return first_half + static_cast<int>(vec >= per_half); };
    auto rem_of = [&](int vec) { return vec - (vec >= per_half ? per_half : 0); };
    // this lane's vector of group G (clamped to the last vector; past the end it is not stored)
    auto vec_of = [&](int G) { return min(G * kEncVecsPerWave + q, total - 1); };
    auto load = [&](int G, float x[16], int &slot) {
        const int vec = vec_of(G);
        const int rem = rem_of(vec);
        load16<BF16>((half_of(vec) ? src1 : src0) + static_cast<int64_t>(rem) * kDim * esize, g, x);
        slot = a.p.slots[fast_div(rem, a.by_kv)];
    };
    auto encode_store = [&](int G, const float x[16], int slot, bool live_group) {
        u32x2 words;
        const float n32 = encode16(x, a.thr, lane, sq, words);
        const uint16_t n16 = f32_to_f16_bits(n32);
        // each lane group stores its own vector's record: lane g writes words 2 g, 2 g + 1 (< 2^31
        // records, so the record index is a 32-bit value)
        const int vec = G * kEncVecsPerWave + q;
        const int vq = min(vec, total - 1);
        const int half = half_of(vq);
        const int rq = rem_of(vq);
        const int head = rq - fast_div(rq, a.by_kv) * a.p.n_kv;
        const bool valid = live_group && vec < total && slot >= 0 && slot < a.p.num_slots;
        if (valid) {
            const int page = fast_div(slot, a.by_page);
            const uint32_t rec = static_cast<uint32_t>((page * a.p.n_kv + head) * a.p.page_size + (slot - page * a.p.page_size));
            *reinterpret_cast<u32x2 *>((half ? words1 : words0) + static_cast<uint64_t>(rec) * kWords + 2 * g) = words;
            if (g == 0) (half ? norms1 : norms0)[rec] = n16;
        }
    };

    // two register sets used in turn (no copies between iterations)
    float x0[16], x1[16];
    int slot0, slot1;
    load(group0, x0, slot0);
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
    a.by_kv = make_fast_div(static_cast<uint32_t>(p.n_kv));
    a.by_page = make_fast_div(static_cast<uint32_t>(p.page_size));
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
