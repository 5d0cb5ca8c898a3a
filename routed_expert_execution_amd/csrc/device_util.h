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

// Lane permutation through DPP (no LDS traffic, folded into the consuming VALU op).
template <int CTRL>
__device__ inline float dpp_f(float v) {
    return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of SEG lanes (SEG a power of two <= 64).  Every lane
// of a group ends with the same bits (each step adds a lane and its partner,
// and a + b == b + a exactly), in one fixed order: lane ^ 1, lane ^ 2, the other
// quad of the 8 (row_half_mirror), the other 8 of the row (row_mirror), the
// other row of the 32 (permlane16_swap), the other 32 (permlane32_swap).
template <int SEG>
__device__ inline float seg_sum(float v) {
    if constexpr (SEG >= 2) v += dpp_f<0xB1>(v);
    if constexpr (SEG >= 4) v += dpp_f<0x4E>(v);
    if constexpr (SEG >= 8) v += dpp_f<0x141>(v);
    if constexpr (SEG >= 16) v += dpp_f<0x140>(v);
    if constexpr (SEG >= 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    if constexpr (SEG >= 64) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return v;
}

// Sum over the four 16-lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48): the last two
// steps of seg_sum<64>, same fixed order.
__device__ inline float cross_row_sum(float v) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// seg_sum with a wave-uniform group size.
__device__ inline float seg_sum_rt(float v, int seg) {
    switch (seg) {
        case 1: return v;
        case 2: return seg_sum<2>(v);
        case 4: return seg_sum<4>(v);
        case 8: return seg_sum<8>(v);
        case 16: return seg_sum<16>(v);
        case 32: return seg_sum<32>(v);
        default: return seg_sum<64>(v);
    }
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS writes but
// leaves its global loads in flight.
__device__ inline void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Maximum over the wave of an unsigned 64-bit value, returned to every lane:
// the partner exchanges of seg_sum<64> (DPP within rows, then the row and
// half-wave swaps), each keeping the larger value.
template <int CTRL>
__device__ inline uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}
__device__ inline uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ inline uint64_t wave_max_u64(uint64_t v) {
    v = max_u64(v, dpp_u64<0xB1>(v));
    v = max_u64(v, dpp_u64<0x4E>(v));
    v = max_u64(v, dpp_u64<0x141>(v));
    v = max_u64(v, dpp_u64<0x140>(v));
    auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    v = max_u64(((uint64_t)hi[0] << 32) | lo[0], ((uint64_t)hi[1] << 32) | lo[1]);
    lo = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    hi = __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
    return max_u64(((uint64_t)hi[0] << 32) | lo[0], ((uint64_t)hi[1] << 32) | lo[1]);
}

// Maximum over the wave of an unsigned 32-bit value, returned to every lane:
// the same partner exchanges, one max each.
__device__ inline uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0u, v, 0x140, 0xF, 0xF, false));
    auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max((uint32_t)r[0], (uint32_t)r[1]);
    r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max((uint32_t)r[0], (uint32_t)r[1]);
}

// Minimum over the wave of an unsigned 32-bit value, returned to every lane.
__device__ inline uint32_t wave_min_u32(uint32_t v) {
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, v, 0xB1, 0xF, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, v, 0x4E, 0xF, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, v, 0x141, 0xF, 0xF, false));
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0xFFFFFFFFu, v, 0x140, 0xF, 0xF, false));
    auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = min((uint32_t)r[0], (uint32_t)r[1]);
    r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return min((uint32_t)r[0], (uint32_t)r[1]);
}

// Bits of the lanes below this one in a 64-lane mask.
__device__ inline int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

// int8 lane j of a 32-bit word -> float
__device__ inline float i8(uint32_t w, int j) { return (float)(int8_t)(w >> (8 * j)); }

}  // namespace moe
