// tq4_device.h -- small device helpers shared by the gfx950 kernels of this
// library (not by its test oracle).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq4 {

constexpr int kDim = 256;
constexpr int kWords = 32;
constexpr int kLevels = 16;
constexpr int kWave = 64;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Division by a fixed d in [1, 2^31) of x in [0, 2^31): q = (umulhi(x, m) + x) >> l with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1 (Granlund and Montgomery, "Division by
// Invariant Integers using Multiplication", unsigned division); umulhi(x, m) + x stays below 2^32.
struct FastDiv {
    uint32_t m;
    uint32_t l;
};

inline FastDiv make_fast_div(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t{1} << l) < d) ++l;
    const uint64_t m = ((uint64_t{1} << 32) * ((uint64_t{1} << l) - d)) / d + 1;
    return FastDiv{static_cast<uint32_t>(m), l};
}

__device__ __forceinline__ int fast_div(int x, FastDiv f) {
    const uint32_t ux = static_cast<uint32_t>(x);
    return static_cast<int>((__umulhi(ux, f.m) + ux) >> f.l);
}

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Two fp32 -> packed bf16 (a in the low half) with one v_cvt_pk_bf16_f32, round to nearest even:
// the same bits as f32_to_bf16 for every finite input.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){a, b}, bf16x2_t));
}

// fp32 -> fp16 bits using the hardware conversion (round to nearest even).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
    _Float16 h = static_cast<_Float16>(f);
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// v_perm_b32: result byte k = byte sel.byte_k of the 8-byte value {hi, lo}
// (selectors 0..3 pick lo's bytes, 4..7 hi's bytes, 0x0c gives 0x00).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Value of lane (lane ^ M) of a wavefront, M in {1, 2, 4, 8, 16, 32}, without the LDS crossbar:
// DPP quad permutes for 1 and 2, DPP row rotates by 4 / 12 and 8 inside each 16-lane row for 4
// and 8, and the lane-swap instructions between 16-lane rows and between 32-lane halves for 16
// and 32.  (Both swap results are kept: each holds the partner's value in half of the lanes.)
template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x, int lane) {
    const int v = static_cast<int>(x);
    if constexpr (M == 1) {
        return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
    } else if constexpr (M == 2) {
        return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
    } else if constexpr (M == 4) {
        // banks 0 and 2 of each row (lanes 0-3, 8-11) read lane + 4 (row_ror:12), banks 1 and 3
        // read lane - 4 (row_ror:4); the bank masks make the two moves write disjoint lanes
        const int down = __builtin_amdgcn_update_dpp(0, v, 0x12C, 0xF, 0x5, false);
        return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(down, v, 0x124, 0xF, 0xA, false));
    } else if constexpr (M == 8) {
        return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));  // row_ror:8
    } else if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return static_cast<uint32_t>((lane & 16) ? r[0] : r[1]);
    } else {
        static_assert(M == 32, "lane_xor: M must be a power of two below 64");
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return static_cast<uint32_t>((lane & 32) ? r[0] : r[1]);
    }
}

template <int M>
__device__ __forceinline__ float lane_xor(float x, int lane) {
    return __builtin_bit_cast(float, lane_xor<M>(__builtin_bit_cast(uint32_t, x), lane));
}

// Maximum and sum of x over the whole wavefront, in every lane: partners lane ^ 32, ^ 16, ..., ^ 1
// in that order (the sum pairs the same values as a butterfly over __shfl_xor would).
__device__ __forceinline__ float wave_max_f32(float x, int lane) {
    x = fmaxf(x, lane_xor<32>(x, lane));
    x = fmaxf(x, lane_xor<16>(x, lane));
    x = fmaxf(x, lane_xor<8>(x, lane));
    x = fmaxf(x, lane_xor<4>(x, lane));
    x = fmaxf(x, lane_xor<2>(x, lane));
    return fmaxf(x, lane_xor<1>(x, lane));
}
__device__ __forceinline__ float wave_sum_f32(float x, int lane) {
    x += lane_xor<32>(x, lane);
    x += lane_xor<16>(x, lane);
    x += lane_xor<8>(x, lane);
    x += lane_xor<4>(x, lane);
    x += lane_xor<2>(x, lane);
    return x + lane_xor<1>(x, lane);
}

// For M = 16 or 32: the pair (lo, hi) with lo = the value of the lower lane of each (l, l ^ M)
// pair and hi = the value of the upper lane, in every lane (one swap instruction, no select).
template <int M>
__device__ __forceinline__ void lane_pair(float x, float &lo, float &hi) {
    static_assert(M == 16 || M == 32, "lane_pair: M is 16 or 32");
    // The elements are copied to plain ints before the bit casts: this compiler lowers
    // __builtin_bit_cast of an element of a vector-typed value as a load from the vector's first
    // element, which would make hi a copy of lo.
    const int v = __builtin_bit_cast(int, x);
    int r0, r1;
    if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        r0 = r[0];
        r1 = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        r0 = r[0];
        r1 = r[1];
    }
    lo = __builtin_bit_cast(float, r0);
    hi = __builtin_bit_cast(float, r1);
}

// Maximum of x over the whole wavefront, as a wave-uniform value (lane swaps and DPP, no LDS).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x, int lane) {
    x = max(x, lane_xor<32>(x, lane));
    x = max(x, lane_xor<16>(x, lane));
    x = max(x, lane_xor<8>(x, lane));
    x = max(x, lane_xor<4>(x, lane));
    x = max(x, lane_xor<2>(x, lane));
    x = max(x, lane_xor<1>(x, lane));
    return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(x)));
}

}  // namespace tq4
