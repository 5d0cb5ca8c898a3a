// Expert-major union of the routed tokens ("Nanite for Experts", §5.3: the
// expert ids of a multi-token window are unioned and each distinct expert is
// scheduled once; §11.3: the union removes redundant work before any kernel).
//
// Up to kPlanOneWgMax assignments, one workgroup of 1024 threads does a stable
// counting sort of the T*k assignments by expert id, entirely in LDS:
//   1. W waves each own a contiguous segment of the assignments and count it
//      into their own LDS histogram row (integer LDS atomics; counts only).
//   2. Per expert, the rows are turned into exclusive per-segment offsets.
//   3. A block-wide prefix scan gives each expert's bucket start and its rank
//      among the experts present; experts[], offsets[] and n_active are written.
//   4. Each wave walks its segment 64 entries at a time; an entry's place is
//      bucket start + its segment offset + the number of earlier lanes of the
//      same 64 holding the same expert (one wave ballot per bit of the expert
//      id finds them).  Segments are in entry order and lanes in entry order,
//      so buckets list entries ascending: the result is unique and
//      bit-reproducible.
#include "device_util.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kHistInts = 8192;  // LDS ints for the per-wave histograms
constexpr int kIdsPerLane = 4;   // ids each lane loads at once

__device__ inline int block_exclusive_scan(int v, int* wave_tot, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int n = __shfl_up(incl, o, 64);
        if (lane >= o) incl += n;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int t = lane < kThreads / 64 ? wave_tot[lane] : 0;
        int ti = t;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            int n = __shfl_up(ti, o, 64);
            if (lane >= o) ti += n;
        }
        if (lane < kThreads / 64) wave_tot[lane] = ti - t;  // exclusive wave offsets
        if (lane == kThreads / 64 - 1) *total = ti;
    }
    __syncthreads();
    int r = wave_tot[wave] + incl - v;
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kThreads) void plan_kernel(const int32_t* __restrict__ ids, int N, int E,
                                                        int32_t* __restrict__ n_active,
                                                        int32_t* __restrict__ experts,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ entries, int* err) {
    __shared__ int hist[kHistInts];  // [W][E]
    __shared__ int start[1024];      // bucket start per expert
    __shared__ int wave_tot[kThreads / 64];
    __shared__ int total_n, total_a;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int W = kHistInts / E;
    if (W > kThreads / 64) W = kThreads / 64;
    const int seg = (N + W - 1) / W;

    for (int i = threadIdx.x; i < W * E; i += kThreads) hist[i] = 0;
    __syncthreads();
    if (wave < W) {
        const int lo = wave * seg, hi = min(N, lo + seg);
        for (int i0 = lo; i0 < hi; i0 += 64 * kIdsPerLane) {
            int e[kIdsPerLane];
#pragma unroll
            for (int u = 0; u < kIdsPerLane; u++) {
                const int i = i0 + 64 * u + lane;
                e[u] = i < hi ? ids[i] : 0;
            }
#pragma unroll
            for (int u = 0; u < kIdsPerLane; u++) {
                if (i0 + 64 * u + lane >= hi) continue;
                if (e[u] >= 0 && e[u] < E) atomicAdd(&hist[wave * E + e[u]], 1);
                else atomicOr(err, kErrBadId);
            }
        }
    }
    __syncthreads();
    // per expert (E <= 1024 = one thread each): exclusive offsets of each segment inside the bucket
    {
        const int e = threadIdx.x;
        int cnt = 0;
        if (e < E) {
            for (int w = 0; w < W; w++) {
                const int c = hist[w * E + e];
                hist[w * E + e] = cnt;
                cnt += c;
            }
        }
        const int first = block_exclusive_scan(cnt, wave_tot, &total_n);
        const int rank = block_exclusive_scan(cnt > 0 ? 1 : 0, wave_tot, &total_a);
        if (e < E) {
            start[e] = first;
            if (cnt > 0) {
                experts[rank] = e;
                offsets[rank] = first;
            }
        }
    }
    if (threadIdx.x == 0) {
        *n_active = total_a;
        offsets[total_a] = total_n;
    }
    __syncthreads();
    // stable scatter
    if (wave < W) {
        const int lo = wave * seg, hi = min(N, lo + seg);
        const uint64_t lt = (1ull << lane) - 1ull;
        int nbits = 0;
        while ((1 << nbits) < E) nbits++;
        for (int i00 = lo; i00 < hi; i00 += 64 * kIdsPerLane) {
            int ev[kIdsPerLane];
#pragma unroll
            for (int u = 0; u < kIdsPerLane; u++) {
                const int i = i00 + 64 * u + lane;
                ev[u] = i < hi ? ids[i] : -1;
            }
#pragma unroll
            for (int u = 0; u < kIdsPerLane; u++) {
                const int i = i00 + 64 * u + lane;
                int e = ev[u];
                const bool ok = i < hi && e >= 0 && e < E;
                if (!ok) e = 0;
                // lanes holding the same expert: agree on every bit of the id
                uint64_t mine = __ballot(ok);
                for (int b = 0; b < nbits; b++) {
                    const bool bit = (e >> b) & 1;
                    const uint64_t m = __ballot(ok && bit);
                    mine &= bit ? m : ~m;
                }
                if (ok) {
                    entries[start[e] + hist[wave * E + e] + __popcll(mine & lt)] = i;
                    if ((mine >> lane) == 1ull)  // highest lane holding this expert
                        hist[wave * E + e] += __popcll(mine);
                }
            }
        }
    }
}

// ---- several workgroups (large T) -------------------------------------------------
//
// The same stable counting sort over kSegEntries-entry segments, one workgroup
// each, in three launches:
//   1. each workgroup counts its segment per expert (LDS atomics) into its
//      row of a global table cnt[segment][E];
//   2. one workgroup turns every expert's column into exclusive per-segment
//      offsets, scans the totals into bucket starts (experts[], offsets[],
//      n_active, as above) and adds each bucket's start to its column, so
//      that cnt[b][e] becomes the first place of segment b's entries of e;
//   3. each workgroup scatters its segment exactly as the one-workgroup
//      kernel does, from those places.
// The result is the unique stable order, bit for bit that of plan_kernel.

constexpr int kSegEntries = kThreads * kIdsPerLane;  // entries per workgroup

__global__ __launch_bounds__(kThreads) void plan_count_kernel(const int32_t* __restrict__ ids, int N, int E,
                                                              int* __restrict__ cnt, int* err) {
    __shared__ int h[1024];
    for (int e = threadIdx.x; e < E; e += kThreads) h[e] = 0;
    __syncthreads();
    const int lo = blockIdx.x * kSegEntries, hi = min(N, lo + kSegEntries);
    int e[kIdsPerLane];
#pragma unroll
    for (int u = 0; u < kIdsPerLane; u++) {
        const int i = lo + u * kThreads + threadIdx.x;
        e[u] = i < hi ? ids[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < kIdsPerLane; u++) {
        if (lo + u * kThreads + (int)threadIdx.x >= hi) continue;
        if (e[u] >= 0 && e[u] < E) atomicAdd(&h[e[u]], 1);
        else atomicOr(err, kErrBadId);
    }
    __syncthreads();
    for (int x = threadIdx.x; x < E; x += kThreads) cnt[(int64_t)blockIdx.x * E + x] = h[x];
}

__global__ __launch_bounds__(kThreads) void plan_scan_kernel(int B, int E, int* __restrict__ cnt,
                                                             int32_t* __restrict__ n_active,
                                                             int32_t* __restrict__ experts,
                                                             int32_t* __restrict__ offsets) {
    __shared__ int wave_tot[kThreads / 64];
    __shared__ int total_n, total_a;
    const int e = threadIdx.x;
    int tot = 0;
    if (e < E)
        for (int b = 0; b < B; b++) {
            const int c = cnt[(int64_t)b * E + e];
            cnt[(int64_t)b * E + e] = tot;
            tot += c;
        }
    const int first = block_exclusive_scan(tot, wave_tot, &total_n);
    const int rank = block_exclusive_scan(tot > 0 ? 1 : 0, wave_tot, &total_a);
    if (e < E) {
        for (int b = 0; b < B; b++) cnt[(int64_t)b * E + e] += first;
        if (tot > 0) {
            experts[rank] = e;
            offsets[rank] = first;
        }
    }
    if (threadIdx.x == 0) {
        *n_active = total_a;
        offsets[total_a] = total_n;
    }
}

__global__ __launch_bounds__(kThreads) void plan_scatter_kernel(const int32_t* __restrict__ ids, int N, int E,
                                                                const int* __restrict__ cnt,
                                                                int32_t* __restrict__ entries) {
    __shared__ int hist[kHistInts];  // [W][E]: per wave, the next place of each expert
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int W = kHistInts / E;
    if (W > kThreads / 64) W = kThreads / 64;
    const int lo0 = blockIdx.x * kSegEntries, hi0 = min(N, lo0 + kSegEntries);
    const int seg = (hi0 - lo0 + W - 1) / W;
    for (int i = threadIdx.x; i < W * E; i += kThreads) hist[i] = 0;
    __syncthreads();
    if (wave < W) {  // per wave counts of its sub-segment
        const int lo = lo0 + wave * seg, hi = min(hi0, lo + seg);
        for (int i0 = lo; i0 < hi; i0 += 64) {
            const int i = i0 + lane;
            const int e = i < hi ? ids[i] : -1;
            if (e >= 0 && e < E) atomicAdd(&hist[wave * E + e], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kThreads) {  // waves in order from the segment's first place
        int p = cnt[(int64_t)blockIdx.x * E + e];
        for (int w = 0; w < W; w++) {
            const int c = hist[w * E + e];
            hist[w * E + e] = p;
            p += c;
        }
    }
    __syncthreads();
    if (wave < W) {
        const int lo = lo0 + wave * seg, hi = min(hi0, lo + seg);
        const uint64_t lt = (1ull << lane) - 1ull;
        int nbits = 0;
        while ((1 << nbits) < E) nbits++;
        for (int i0 = lo; i0 < hi; i0 += 64) {
            const int i = i0 + lane;
            int e = i < hi ? ids[i] : -1;
            const bool ok = i < hi && e >= 0 && e < E;
            if (!ok) e = 0;
            uint64_t mine = __ballot(ok);
            for (int b = 0; b < nbits; b++) {
                const bool bit = (e >> b) & 1;
                const uint64_t m = __ballot(ok && bit);
                mine &= bit ? m : ~m;
            }
            if (ok) {
                entries[hist[wave * E + e] + __popcll(mine & lt)] = i;
                if ((mine >> lane) == 1ull) hist[wave * E + e] += __popcll(mine);
            }
        }
    }
}

}  // namespace

int64_t plan_workspace_ints(int64_t T, int k, int E) {
    const int64_t N = T * k;
    return N > kPlanOneWgMax ? (N + kSegEntries - 1) / kSegEntries * E : 0;
}

hipError_t launch_plan(const int32_t* ids, int64_t T, int k, int E, const moe_plan& plan, int* err,
                       hipStream_t s, int* ws) {
    const int N = (int)(T * k);
    if (N <= kPlanOneWgMax || !ws) {
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, s, ids, N, E, plan.n_active, plan.experts,
                           plan.offsets, plan.entries, err);
        return hipGetLastError();
    }
    const int B = (N + kSegEntries - 1) / kSegEntries;
    hipLaunchKernelGGL(plan_count_kernel, dim3(B), dim3(kThreads), 0, s, ids, N, E, ws, err);
    hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(kThreads), 0, s, B, E, ws, plan.n_active, plan.experts,
                       plan.offsets);
    hipLaunchKernelGGL(plan_scatter_kernel, dim3(B), dim3(kThreads), 0, s, ids, N, E, ws, plan.entries);
    return hipGetLastError();
}

}  // namespace moe
