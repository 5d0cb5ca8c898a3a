// Page-table writes of one staging call: the entries of the experts whose
// payloads it copied (their slots) and of the experts those slots evicted
// (absent), written by one launch after the copies instead of one fill per
// entry.
#include "internal.h"

namespace moe {
namespace {

// The writes of one batch touch distinct entries (an evicted expert is never
// one the same call maps), so their order inside the launch does not matter.
__global__ __launch_bounds__(kPtBatch) void pt_write_kernel(int32_t* __restrict__ pt, PtWrites w) {
    const int i = threadIdx.x;
    if (i < w.n) pt[w.idx[i]] = w.val[i];
}

}  // namespace

hipError_t launch_pt_write(int32_t* pt, const PtWrites& w, hipStream_t s) {
    if (w.n <= 0) return hipSuccess;
    if (w.n > kPtBatch) return hipErrorInvalidValue;
    pt_write_kernel<<<1, kPtBatch, 0, s>>>(pt, w);
    return hipGetLastError();
}

}  // namespace moe

namespace moe {
namespace {

constexpr int kPullThreads = 512;
constexpr int kPullUnroll = 8;  // 16-byte loads in flight per thread

// Copies a.n payloads of a.words 16-byte words each from a.src[i] (pinned host
// memory read over the bus, or device memory) to a.dst[i] (a slot); each
// workgroup takes one contiguous stretch of the payloads laid end to end, with
// kPullUnroll loads issued before the first store.  Workgroup 0 also writes the
// page-table entries in w, which later work on the stream reads.
__global__ __launch_bounds__(kPullThreads) void pull_kernel(PullArgs a, int32_t* __restrict__ pt, PtWrites w) {
    if (blockIdx.x == 0 && threadIdx.x < w.n) pt[w.idx[threadIdx.x]] = w.val[threadIdx.x];
    const uint32_t total = (uint32_t)a.n * a.words;
    const uint32_t per = (total + gridDim.x - 1) / gridDim.x;
    const uint32_t b0 = blockIdx.x * per, e = min(b0 + per, total);
    for (uint32_t i = b0 + threadIdx.x; i < e; i += kPullThreads * kPullUnroll) {
        uint4 v[kPullUnroll];
#pragma unroll
        for (int u = 0; u < kPullUnroll; u++) {
            const uint32_t j = i + kPullThreads * u;
            if (j < e) {
                const uint32_t p = j / a.words;
                v[u] = a.src[p][j - p * a.words];
            }
        }
#pragma unroll
        for (int u = 0; u < kPullUnroll; u++) {
            const uint32_t j = i + kPullThreads * u;
            if (j < e) {
                const uint32_t p = j / a.words;
                a.dst[p][j - p * a.words] = v[u];
            }
        }
    }
}

}  // namespace

hipError_t launch_pull(const PullArgs& a, int32_t* pt, const PtWrites& w, hipStream_t s) {
    if (a.n < 1 || a.n > kPullMax || a.words < 1 || w.n < 0 || w.n > kPtBatch ||
        (uint64_t)a.n * a.words > 0x7FFFFFFFull)
        return hipErrorInvalidValue;
    pull_kernel<<<kPullWorkgroups, kPullThreads, 0, s>>>(a, pt, w);
    return hipGetLastError();
}

}  // namespace moe
