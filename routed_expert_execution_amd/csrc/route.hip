// Router logits and top-k routing ("Nanite for Experts", §3.1: the router's
// decisions pick the experts; "Nanite for Experts", §1 and "Paging the
// Experts", §3.1: top-8 of 256 routed experts per token).
//
// router_gemv: one wave per (expert row, group of tokens).  Each lane reads
//   float4 slices of the row at a 1 KiB stride (coalesced), accumulates its
//   slice in order, then the wave sums lanes with a fixed xor butterfly, so
//   the logits are reproducible bit for bit.
// topk: one wave per token.  Each lane keeps its logits as 64-bit keys
//   (order-preserving float bits << 32 | ~expert), so one unsigned max picks
//   the larger logit and, on ties, the lower expert index; k rounds of a wave
//   max select the experts.  Weights are the softmax over the selected logits
//   (or over all, norm == 0), in fp32.
#include "device_util.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kTokensPerWave = 4;

__global__ __launch_bounds__(256) void router_gemv_kernel(const void* __restrict__ x, int x_bf16,
                                                          const float* __restrict__ w_r, int T, int E,
                                                          int d, float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    const int t0 = blockIdx.y * kTokensPerWave;
    const float* row = w_r + (int64_t)e * d;
    for (int t = t0; t < min(T, t0 + kTokensPerWave); t++) {
        float acc = 0.f;
        for (int c = lane * 4; c < d; c += 256) {
            const float4 w = *(const float4*)(row + c);
            float xv[4];
            if (x_bf16) {
                const uint2 b = *(const uint2*)((const uint16_t*)x + (int64_t)t * d + c);
                xv[0] = bf16_bits_to_f32(b.x & 0xFFFF);
                xv[1] = bf16_bits_to_f32(b.x >> 16);
                xv[2] = bf16_bits_to_f32(b.y & 0xFFFF);
                xv[3] = bf16_bits_to_f32(b.y >> 16);
            } else {
                const float4 f = *(const float4*)((const float*)x + (int64_t)t * d + c);
                xv[0] = f.x; xv[1] = f.y; xv[2] = f.z; xv[3] = f.w;
            }
            acc = fmaf(w.x, xv[0], acc);
            acc = fmaf(w.y, xv[1], acc);
            acc = fmaf(w.z, xv[2], acc);
            acc = fmaf(w.w, xv[3], acc);
        }
        acc = seg_sum<64>(acc);
        if (lane == 0) logits[(int64_t)t * E + e] = acc;
    }
}

__device__ inline uint32_t order_bits(float v) {
    uint32_t b = __float_as_uint(v);
    if (b == 0x80000000u) b = 0;  // -0 ranks with +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ inline float unorder_bits(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int KPL>  // keys per lane: ceil(E / 64)
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   int norm, int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* l = logits + (int64_t)t * E;
    uint64_t key[KPL];
#pragma unroll
    for (int m = 0; m < KPL; m++) {
        const int e = lane + 64 * m;
        key[m] = e < E ? ((uint64_t)order_bits(l[e]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e) : 0;
    }
    float my_logit = 0.f;  // lane j keeps the j-th selected logit
    int my_id = 0;
    for (int j = 0; j < k; j++) {
        uint64_t best = 0;
#pragma unroll
        for (int m = 0; m < KPL; m++) best = key[m] > best ? key[m] : best;
        const uint64_t top = wave_max_u64(best);
#pragma unroll
        for (int m = 0; m < KPL; m++) if (key[m] == top) key[m] = 0;  // keys are unique
        if (lane == j) {
            my_id = (int)(0xFFFFFFFFu - (uint32_t)top);
            my_logit = unorder_bits((uint32_t)(top >> 32));
        }
    }
    const float lmax = __shfl(my_logit, 0, 64);
    float z;
    if (norm) {
        float ex = lane < k ? expf(my_logit - lmax) : 0.f;
        z = seg_sum<64>(ex);
    } else {
        float part = 0.f;
#pragma unroll
        for (int m = 0; m < KPL; m++) {
            const int e = lane + 64 * m;
            if (e < E) part += expf(l[e] - lmax);
        }
        z = seg_sum<64>(part);
    }
    if (lane < k) {
        ids[(int64_t)t * k + lane] = my_id;
        w[(int64_t)t * k + lane] = expf(my_logit - lmax) / z;
    }
}

}  // namespace

hipError_t launch_router_gemv(const void* x, int x_bf16, const float* w_r, int64_t T, int E, int d,
                              float* logits, hipStream_t s) {
    dim3 grid((E + 3) / 4, (unsigned)((T + kTokensPerWave - 1) / kTokensPerWave));
    hipLaunchKernelGGL(router_gemv_kernel, grid, dim3(256), 0, s, x, x_bf16, w_r, (int)T, E, d, logits);
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int64_t T, int E, int k, int norm, int32_t* ids, float* w,
                       hipStream_t s) {
    dim3 grid((unsigned)((T + 3) / 4));
    const int kpl = (E + 63) / 64;
    if (kpl <= 1) hipLaunchKernelGGL(topk_kernel<1>, grid, dim3(256), 0, s, logits, (int)T, E, k, norm, ids, w);
    else if (kpl <= 2) hipLaunchKernelGGL(topk_kernel<2>, grid, dim3(256), 0, s, logits, (int)T, E, k, norm, ids, w);
    else if (kpl <= 4) hipLaunchKernelGGL(topk_kernel<4>, grid, dim3(256), 0, s, logits, (int)T, E, k, norm, ids, w);
    else if (kpl <= 8) hipLaunchKernelGGL(topk_kernel<8>, grid, dim3(256), 0, s, logits, (int)T, E, k, norm, ids, w);
    else hipLaunchKernelGGL(topk_kernel<16>, grid, dim3(256), 0, s, logits, (int)T, E, k, norm, ids, w);
    return hipGetLastError();
}

}  // namespace moe
