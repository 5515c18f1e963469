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

}  // namespace tq4
