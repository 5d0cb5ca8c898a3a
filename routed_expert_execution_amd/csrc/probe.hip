// Measurement helpers for the peak references next to the path's own numbers:
// the HBM rate a plain streaming read reaches from one launch, and the rate of
// back-to-back bf16 matrix-core products.  Neither is part of the routed path.
#include <algorithm>

#include "internal.h"

namespace moe {
namespace {

constexpr int kReadThreads = 512;
constexpr int kReadUnroll = 8;  // 16-byte loads in flight per thread

// Workgroup b reads its own contiguous chunk of src, every 16-byte word once,
// kReadUnroll loads issued before any is used, folded with xor; a word is
// stored only if the fold hits a value the caller cannot expect, which keeps
// the loads live.
__global__ __launch_bounds__(kReadThreads) void read_kernel(const uint4* __restrict__ src, int64_t n, int64_t per_wg,
                                                            uint32_t* __restrict__ sink) {
    const int64_t b0 = (int64_t)blockIdx.x * per_wg, e = min(b0 + per_wg, n);
    uint32_t acc = 0;
    for (int64_t i = b0 + threadIdx.x; i < e; i += kReadThreads * kReadUnroll) {
        uint4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; u++) {
            const int64_t j = i + (int64_t)kReadThreads * u;
            v[u] = j < e ? src[j] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Each wave runs `iters` rounds of CH independent bf16 matrix-core products,
// 16x16x32 (16,384 flops each) or 32x32x16 (32,768 flops); the sums are
// stored only under a condition no finite input meets.
template <int SHAPE, int CH>
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* __restrict__ sink) {
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; j++) {
        a[j] = (__bf16)(0.001f * (float)((threadIdx.x + j) & 7));
        b[j] = (__bf16)(0.002f * (float)((threadIdx.x * 3 + j) & 7));
    }
    float s = 0.f;
    if constexpr (SHAPE == 0) {
        f32x4 acc[CH];
#pragma unroll
        for (int c = 0; c < CH; c++) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; it++) {
#pragma unroll
            for (int c = 0; c < CH; c++) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < CH; c++) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    } else {
        f32x16 acc[CH];
#pragma unroll
        for (int c = 0; c < CH; c++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[c][r] = 0.f;
        for (int it = 0; it < iters; it++) {
#pragma unroll
            for (int c = 0; c < CH; c++) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < CH; c++) s += acc[c][0] + acc[c][5] + acc[c][10] + acc[c][15];
    }
    if (s == -1.0f) sink[0] = s;
}

// LDS read rate: each of 4 waves reads 16 bytes per lane per instruction
// (consecutive lanes, consecutive 16-byte words: no bank conflicts) from a
// 32 KiB buffer, `iters` rounds of 8 reads, folded with xor.
__global__ __launch_bounds__(256) void lds_kernel(int iters, uint32_t* __restrict__ sink) {
    __shared__ uint4 buf[2048];
    for (int i = threadIdx.x; i < 2048; i += 256) buf[i] = make_uint4(i, i * 3, i * 5, i * 7);
    __syncthreads();
    uint32_t acc = 0;
    const int base = (threadIdx.x & 63) + (threadIdx.x >> 6) * 512;
    for (int it = 0; it < iters; it++) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) v[u] = buf[(base + 64 * u + it) & 2047];
#pragma unroll
        for (int u = 0; u < 8; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

// variant v: instruction v % 2 (0: 16x16x32, 1: 32x32x16), independent
// accumulators per wave 4 << (v / 2) (4, 8 or 16)
int probe_chains(int v) { return 4 << (v / 2); }

}  // namespace

hipError_t launch_probe_read(const void* src, int64_t bytes, int wgs, uint32_t* sink, hipStream_t s) {
    const int64_t n = bytes / 16;
    if (wgs < 1) wgs = 512;
    const int64_t per = (n + wgs - 1) / wgs;
    hipLaunchKernelGGL(read_kernel, dim3(wgs), dim3(kReadThreads), 0, s, (const uint4*)src, n, per, sink);
    return hipGetLastError();
}

hipError_t launch_probe_mfma(int iters, int grid, int shape, float* sink, hipStream_t s) {
    switch (shape) {
        case 0: hipLaunchKernelGGL((mfma_kernel<0, 4>), dim3(grid), dim3(256), 0, s, iters, sink); break;
        case 1: hipLaunchKernelGGL((mfma_kernel<1, 4>), dim3(grid), dim3(256), 0, s, iters, sink); break;
        case 2: hipLaunchKernelGGL((mfma_kernel<0, 8>), dim3(grid), dim3(256), 0, s, iters, sink); break;
        case 3: hipLaunchKernelGGL((mfma_kernel<1, 8>), dim3(grid), dim3(256), 0, s, iters, sink); break;
        case 4: hipLaunchKernelGGL((mfma_kernel<0, 16>), dim3(grid), dim3(256), 0, s, iters, sink); break;
        default: hipLaunchKernelGGL((mfma_kernel<1, 16>), dim3(grid), dim3(256), 0, s, iters, sink); break;
    }
    return hipGetLastError();
}

hipError_t launch_probe_lds(int iters, int grid, uint32_t* sink, hipStream_t s) {
    hipLaunchKernelGGL(lds_kernel, dim3(grid), dim3(256), 0, s, iters, sink);
    return hipGetLastError();
}

int64_t probe_mfma_flops(int iters, int grid, int shape) {
    return (int64_t)grid * 4 * probe_chains(shape) * (shape % 2 == 0 ? 16384LL : 32768LL) * iters;
}

}  // namespace moe
