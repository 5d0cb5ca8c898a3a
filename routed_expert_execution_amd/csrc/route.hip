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
// topk: one wave per token, on order-preserving 32-bit keys (-0 ranked with
//   +0), ties to the lower index.  Up to 256 experts and top-32: a lower bound
//   of the k-th largest key (the smallest of 8 group maxima) leaves a few
//   candidates, which rank themselves by counting; otherwise (or with more
//   than 64 candidates) k rounds, each a DPP/permlane max of the keys and a
//   min of the indices holding it.  Weights are the softmax over the selected
//   logits (or over all, norm == 0), in fp32.
#include "internal.h"
#include "route_device.h"

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
        const float acc = row_dot(row, x, x_bf16, t, d, lane);
        if (lane == 0) logits[(int64_t)t * E + e] = acc;
    }
}

template <int KPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   int norm, int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
    __shared__ uint64_t sc[4][128];
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_wave<KPL>(logits + (int64_t)t * E, E, k, norm, ids + (int64_t)t * k, w + (int64_t)t * k,
                   sc[threadIdx.x >> 6]);
}

struct RouteUnion {
    int T, E, k, norm;
    int32_t* ids;
    float* w;
    int32_t* n_active;
    int32_t* experts;
    int32_t* offsets;
    int32_t* entries;
    int32_t* mirror;  // or null (pinned host memory): [0] n_active, [1, 1 + E) the experts, then
                      // the T k selected ids and the T k weights (float bits), entry t k + j
};

// Top-k of the T tokens (one wave each), then the union; one workgroup of 256.
template <int KPL>
__device__ void topk_union_wg(const float* logits, const RouteUnion& r) {
    static_assert(kFusedMaxT * 32 <= 128, "union_small holds two entries per lane of one wave");
    __shared__ int32_t s_ids[kFusedMaxT * 32];
    __shared__ float s_w[kFusedMaxT * 32];
    __shared__ uint64_t sc[4][128];
    const int t = threadIdx.x >> 6;
    if (t < r.T)
        topk_wave<KPL>(logits + (int64_t)t * r.E, r.E, r.k, r.norm, s_ids + t * r.k, s_w + t * r.k, sc[t]);
    __syncthreads();
    const int N = r.T * r.k;
    if ((int)threadIdx.x < N) {
        r.ids[threadIdx.x] = s_ids[threadIdx.x];
        r.w[threadIdx.x] = s_w[threadIdx.x];
    }
    union_small(s_ids, N, r.n_active, r.experts, r.offsets, r.entries);
    if (r.mirror) {  // the units, for a host that maps them (written after the union is complete)
        __syncthreads();
        const int na = *r.n_active;
        for (int i = threadIdx.x; i < na; i += blockDim.x) r.mirror[1 + i] = r.experts[i];
        for (int i = threadIdx.x; i < N; i += blockDim.x) {
            r.mirror[1 + r.E + i] = s_ids[i];
            r.mirror[1 + r.E + N + i] = __float_as_int(s_w[i]);
        }
        // The host polls the count: every word above reaches host memory
        // first (each thread's own stores, then the barrier), then the count.
        __threadfence_system();
        __syncthreads();
        if (threadIdx.x == 0) __hip_atomic_store(r.mirror, na, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

template <int KPL>
__global__ __launch_bounds__(256) void topk_union_kernel(const float* __restrict__ logits, RouteUnion r) {
    topk_union_wg<KPL>(logits, r);
}

}  // namespace

hipError_t launch_route_union(const void* x, int x_bf16, const float* w_r, const float* logits_in, int64_t T,
                              int E, int d, int k, int norm, float* logits, int32_t* ids, float* w,
                              const moe_plan& plan, hipStream_t s, int32_t* mirror) {
    RouteUnion r{(int)T, E, k, norm, ids, w, plan.n_active, plan.experts, plan.offsets, plan.entries, mirror};
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
