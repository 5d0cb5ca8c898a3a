// Router logits and top-k routing ("Nanite for Experts", §3.1: the router's
// decisions pick the experts; "Nanite for Experts", §1 and "Paging the
// Experts", §3.1: top-8 of 256 routed experts per token).
//
// router_gemv: one wave per (expert row, group of tokens).  Each lane reads
//   float4 slices of the row at a 1 KiB stride (coalesced), accumulates its
//   slice in order, then the wave sums lanes with a fixed xor butterfly, so
//   the logits are reproducible bit for bit.
// route_union (T <= kFusedMaxT): the same logits, then top-k and the union in
//   one single-workgroup launch (see below).
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

// Lane's share of row . x[t] (float4 slices at a 1 KiB stride, in order), then
// the fixed lane butterfly: every lane returns the same bits.
__device__ inline float row_dot(const float* row, const void* x, int x_bf16, int t, int d, int lane) {
    constexpr int U = 8;  // slices in flight per lane (d_model 2048 is 8 slices)
    float acc = 0.f;
    for (int c0 = lane * 4; c0 < d; c0 += 256 * U) {
        float4 wv[U], xv[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int c = c0 + 256 * u;
            if (c < d) {
                wv[u] = *(const float4*)(row + c);
                if (x_bf16) {
                    const uint2 b = *(const uint2*)((const uint16_t*)x + (int64_t)t * d + c);
                    xv[u] = make_float4(bf16_bits_to_f32(b.x & 0xFFFF), bf16_bits_to_f32(b.x >> 16),
                                        bf16_bits_to_f32(b.y & 0xFFFF), bf16_bits_to_f32(b.y >> 16));
                } else {
                    xv[u] = *(const float4*)((const float*)x + (int64_t)t * d + c);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (c0 + 256 * u < d) {
                acc = fmaf(wv[u].x, xv[u].x, acc);
                acc = fmaf(wv[u].y, xv[u].y, acc);
                acc = fmaf(wv[u].z, xv[u].z, acc);
                acc = fmaf(wv[u].w, xv[u].w, acc);
            }
        }
    }
    return seg_sum<64>(acc);
}

__global__ __launch_bounds__(256) void router_gemv_kernel(const void* __restrict__ x, int x_bf16,
                                                          const float* __restrict__ w_r, int T, int E,
                                                          int d, float* __restrict__ logits) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    const int t0 = blockIdx.y * kTokensPerWave;
    const float* row = w_r + (int64_t)e * d;
    for (int t = t0; t < min(T, t0 + kTokensPerWave); t++) {
        const float acc = row_dot(row, x, x_bf16, t, d, lane);
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

// One wave: top-k of one token's E logits (KPL = ceil(E / 64) keys per lane).
template <int KPL>
__device__ inline void topk_wave(const float* l, int E, int k, int norm, int32_t* ids, float* w) {
    const int lane = threadIdx.x & 63;
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
        ids[lane] = my_id;
        w[lane] = expf(my_logit - lmax) / z;
    }
}

template <int KPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   int norm, int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_wave<KPL>(logits + (int64_t)t * E, E, k, norm, ids + (int64_t)t * k, w + (int64_t)t * k);
}

// ---- route + union of a few tokens in one launch ------------------------------
//
// For T <= kFusedMaxT: the union of at most kFusedMaxT * 32 assignments is
// computed by one workgroup from the ids it has just selected.  Entry i goes
// to place |{j : e_j < e_i or (e_j == e_i and j < i)}| (its place in the stable
// order by expert), which is the same unique result the counting sort gives.

__device__ void union_small(const int32_t* s_ids, int N, int* s_sorted, int32_t* n_active, int32_t* experts,
                            int32_t* offsets, int32_t* entries) {
    const int i = threadIdx.x;
    if (i < N) {
        const int e = s_ids[i];
        int pos = 0;
        for (int j = 0; j < N; j++) {
            const int f = s_ids[j];
            pos += (f < e || (f == e && j < i)) ? 1 : 0;
        }
        s_sorted[pos] = e;
        entries[pos] = i;
    }
    __syncthreads();
    if (i < N) {
        const int e = s_sorted[i];
        if (i == 0 || s_sorted[i - 1] != e) {
            int rank = 0;  // buckets before this one
            for (int p = 1; p <= i; p++) rank += s_sorted[p] != s_sorted[p - 1] ? 1 : 0;
            experts[rank] = e;
            offsets[rank] = i;
        }
    }
    if (i == 0) {
        int nb = N > 0 ? 1 : 0;
        for (int p = 1; p < N; p++) nb += s_sorted[p] != s_sorted[p - 1] ? 1 : 0;
        *n_active = nb;
        offsets[nb] = N;
    }
}

struct RouteUnion {
    int T, E, k, norm;
    int32_t* ids;
    float* w;
    int32_t* n_active;
    int32_t* experts;
    int32_t* offsets;
    int32_t* entries;
};

// Top-k of the T tokens (one wave each), then the union; one workgroup of 256.
template <int KPL>
__device__ void topk_union_wg(const float* logits, const RouteUnion& r) {
    __shared__ int32_t s_ids[kFusedMaxT * 32];
    __shared__ int s_sorted[kFusedMaxT * 32];
    const int t = threadIdx.x >> 6;
    if (t < r.T) topk_wave<KPL>(logits + (int64_t)t * r.E, r.E, r.k, r.norm, r.ids + t * r.k, r.w + t * r.k);
    __syncthreads();  // the ids just written are this workgroup's own
    const int N = r.T * r.k;
    if ((int)threadIdx.x < N) s_ids[threadIdx.x] = r.ids[threadIdx.x];
    __syncthreads();
    union_small(s_ids, N, s_sorted, r.n_active, r.experts, r.offsets, r.entries);
}

template <int KPL>
__global__ __launch_bounds__(256) void topk_union_kernel(const float* __restrict__ logits, RouteUnion r) {
    topk_union_wg<KPL>(logits, r);
}

}  // namespace

hipError_t launch_route_union(const void* x, int x_bf16, const float* w_r, const float* logits_in, int64_t T,
                              int E, int d, int k, int norm, float* logits, int32_t* ids, float* w,
                              const moe_plan& plan, hipStream_t s) {
    RouteUnion r{(int)T, E, k, norm, ids, w, plan.n_active, plan.experts, plan.offsets, plan.entries};
    if (!logits_in) {
        hipLaunchKernelGGL(router_gemv_kernel, dim3((E + 3) / 4, 1), dim3(256), 0, s, x, x_bf16, w_r, (int)T, E, d,
                           logits);
        logits_in = logits;
    }
    const int kpl = (E + 63) / 64;
#define MOE_TU(K) hipLaunchKernelGGL(topk_union_kernel<K>, dim3(1), dim3(256), 0, s, logits_in, r)
    if (kpl <= 1) MOE_TU(1); else if (kpl <= 2) MOE_TU(2); else if (kpl <= 4) MOE_TU(4);
    else if (kpl <= 8) MOE_TU(8); else MOE_TU(16);
#undef MOE_TU
    return hipGetLastError();
}

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
