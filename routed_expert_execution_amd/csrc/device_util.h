// Device helpers shared by the libmoe kernels (wave64, gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

__device__ inline float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Round to the nearest bfloat16, ties to even (v_cvt_pk_bf16_f32 on gfx950), returned as float.
__device__ inline float round_bf16(float v) {
    __bf16 b = (__bf16)v;
    return __uint_as_float((uint32_t)__builtin_bit_cast(unsigned short, b) << 16);
}

// IEEE binary16 bits -> float (exact).
__device__ inline float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
}

// Sum over aligned groups of SEG lanes (SEG a power of two <= 64); every lane
// of a group ends with the group's sum, combined in one fixed order.
template <int SEG>
__device__ inline float seg_sum(float v) {
#pragma unroll
    for (int m = SEG / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__device__ inline uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

// int8 lane j of a 32-bit word -> float
__device__ inline float i8(uint32_t w, int j) { return (float)(int8_t)(w >> (8 * j)); }

}  // namespace moe
