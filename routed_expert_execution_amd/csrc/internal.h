// Internal declarations of libmoe: payload geometry and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kQK = 32;         // elements per quant block
constexpr int kTileBlocks = 64; // blocks per tile: one block per lane of a wave64
constexpr int kWave = 64;

inline int block_bytes(int qtype) { return qtype == MOE_Q8_0 ? 34 : 18; }

// Geometry of one expert payload (device tile layout; see moe_payload_bytes in moe.h).
struct Geom {
    int d = 0, f = 0, qtype = 0;
    int nb_d = 0, nb_f = 0;      // blocks per gate/up row, per down row
    int64_t tile_bytes = 0;      // 64 blocks
    int64_t gu_tiles = 0;        // tiles per gate matrix (= per up matrix)
    int64_t d_tiles = 0;         // tiles of the down matrix
    int64_t payload = 0;

    bool init(int d_, int f_, int qt) {
        d = d_; f = f_; qtype = qt;
        if (qt != MOE_Q8_0 && qt != MOE_Q4_0) return false;
        if (d <= 0 || f <= 0 || d % kQK || f % kQK) return false;
        nb_d = d / kQK; nb_f = f / kQK;
        // gate/up rows: 4..64 blocks, a power of two (whole 4-block column groups);
        // down rows: whole 4-block column groups, at most 64 blocks
        if (nb_d < 4 || nb_d > 64 || (nb_d & (nb_d - 1))) return false;
        if (nb_f % 4 || nb_f > 64) return false;
        tile_bytes = (int64_t)kTileBlocks * block_bytes(qt);
        gu_tiles = (int64_t)f * nb_d / kTileBlocks;
        d_tiles = (int64_t)d * nb_f / kTileBlocks;
        payload = (2 * gu_tiles + d_tiles) * tile_bytes;
        return true;
    }
    __host__ __device__ int64_t gate_tile(int64_t t) const { return 2 * t * tile_bytes; }
    __host__ __device__ int64_t up_tile(int64_t t) const { return (2 * t + 1) * tile_bytes; }
    __host__ __device__ int64_t down_tile(int64_t t) const { return (2 * gu_tiles + t) * tile_bytes; }
    // Block (row r, column block cb) of each matrix -> (tile, lane).  Every
    // matrix uses one tile shape: 16 rows x 4 column blocks, lane = 16 * (cb % 4)
    // + r % 16, tiles ordered by row group then column group, so the tiles of
    // 16 consecutive rows are consecutive: one MFMA step of 16 rows x 128
    // columns reads one whole tile, and 16 rows of a GEMV one contiguous run.
    __host__ __device__ void gu_block(int64_t r, int cb, int64_t* tile, int* lane) const {
        *tile = (r / 16) * (nb_d / 4) + cb / 4;
        *lane = 16 * (cb % 4) + (int)(r % 16);
    }
    __host__ __device__ void down_block(int64_t r, int cb, int64_t* tile, int* lane) const {
        *tile = (r / 16) * (nb_f / 4) + cb / 4;
        *lane = 16 * (cb % 4) + (int)(r % 16);
    }
};

// Byte offsets inside one tile for block i (0..63).
__host__ __device__ inline int q8_lo(int i) { return 16 * i; }
__host__ __device__ inline int q8_hi(int i) { return 16 * kTileBlocks + 16 * i; }
__host__ __device__ inline int q8_scale(int i) { return 32 * kTileBlocks + 2 * i; }
__host__ __device__ inline int q4_nib(int i) { return 16 * i; }
__host__ __device__ inline int q4_scale(int i) { return 16 * kTileBlocks + 2 * i; }

// Device error word bits.
constexpr int kErrMiss = 1;     // unmapped expert met by a kernel
constexpr int kErrBadId = 4;    // expert id out of range in a plan input
constexpr int kErrSync = 8;     // a decode workgroup's bounded wait for the hidden rows ran out

// ---- launchers (return hipError_t of the launch) ----

hipError_t launch_router_gemv(const void* x, int x_bf16, const float* w_r, int64_t T, int E, int d,
                              float* logits, hipStream_t s);
hipError_t launch_topk(const float* logits, int64_t T, int E, int k, int norm, int32_t* ids,
                       float* w, hipStream_t s);
// Up to kPlanOneWgMax assignments one workgroup sorts them; more take three
// launches over segments of 4096, with a workspace of plan_workspace_ints()
// ints (without one, the one-workgroup kernel, however large).  Measured
// (event time): 16,384 assignments 25.7 us in one workgroup, 21.5 us in
// segments; 524,288 in segments 63 us.
constexpr int64_t kPlanOneWgMax = 8192;
int64_t plan_workspace_ints(int64_t T, int k, int E);
hipError_t launch_plan(const int32_t* ids, int64_t T, int k, int E, const moe_plan& plan, int* err,
                       hipStream_t s, int* ws = nullptr);
hipError_t launch_dequant(const Geom& g, const uint8_t* payload, int prec, float* out, hipStream_t s);
// Route and union of at most kFusedMaxT tokens: router logits (unless
// logits_in), then top-k and the union in one single-workgroup launch.  Same
// results as launch_router_gemv + launch_topk + launch_plan.
constexpr int kFusedMaxT = 4;
hipError_t launch_route_union(const void* x, int x_bf16, const float* w_r, const float* logits_in, int64_t T,
                              int E, int d, int k, int norm, float* logits, int32_t* ids, float* w,
                              const moe_plan& plan, hipStream_t s, int32_t* mirror = nullptr);

struct FfnArgs {
    // experts
    const uint8_t* pool;
    int64_t payload_bytes;
    const int32_t* pt;      // page table [L x E]
    int layer, E, n_slots;
    const uint8_t* shared;  // shared expert payload or null
    // plan
    const int32_t* n_active;
    const int32_t* experts;
    const int32_t* offsets;
    const int32_t* entries;
    const float* topk_w;
    int k;
    // activations
    const void* x;
    int x_bf16;
    int T;
    // routing inside the decode launch (route != kRoutePlan): the plan above is
    // then an output, computed from logits_in [T, E] (kRouteLogits) or from
    // x . w_router^T (kRouteRouter, w_router [E, d] fp32)
    int route, norm;
    const float* logits_in;
    const float* w_router;
    int32_t* ids_out;       // [T, k]
    float* w_out;           // [T, k]
    int32_t *o_n_active, *o_experts, *o_offsets, *o_entries;
    // outputs and workspace
    float* hbuf;            // two halves, each kDecodeCopies copies of [T*k + T, d_ff] hidden rows
                            // (plan positions, then the shared rows) and [T, E] logits; every
                            // word 0xFFFFFFFF at creation
    uint32_t* sync;         // [kSyncInts], zero at creation: [kSyncCount] finished down workgroups,
                            // [kSyncArrive + p] gate/up workgroups arrived in a launch of parity p
    int64_t wait_ticks;     // bound of a workgroup's wait (100 MHz wall-clock ticks); negative:
                            // every wait gives up at its first check (tests of the time-out path)
    float* y;               // [T, d]
    int* err;
};

enum { kRoutePlan = 0, kRouteLogits = 1, kRouteRouter = 2 };

// Largest step the decode kernel takes.
constexpr int kDecodeMaxT = 4;
constexpr int kSyncInts = 32, kSyncCount = 0, kSyncArrive = 16;  // one 128-byte line

// A workspace half holds kDecodeCopies copies of the same words, each starting
// on its own 4 KiB: every value is stored into all of them and each reader reads
// one, so that hundreds of workgroups reading the same few KiB spread over
// several memory channels instead of queueing on one (8 measured best of 4, 8
// and 16 for the one- and four-token steps, once the four-token step split its
// down work over twice the workgroups; 4 before).
constexpr int kDecodeCopies = 8;
// Floats of one copy: hidden rows for top_k and d_ff, then the logits of E experts.
__host__ __device__ inline int64_t decode_h_rows_floats(int k, int f) { return (int64_t)kDecodeMaxT * (k + 1) * f; }
__host__ __device__ inline int64_t decode_copy_floats(int k, int f, int E) {
    return (decode_h_rows_floats(k, f) + (int64_t)kDecodeMaxT * E + 1023) / 1024 * 1024;
}
// A half: the copies, then one copy of partial output rows (T x d) that the
// first down workgroup of a split row group hands to the second.
__host__ __device__ inline int64_t decode_half_floats(int k, int f, int E, int d) {
    return kDecodeCopies * decode_copy_floats(k, f, E) + ((int64_t)kDecodeMaxT * d + 1023) / 1024 * 1024;
}
// Floats of the whole decode workspace (both halves).
__host__ __device__ inline int64_t decode_h_floats(int k, int f, int E, int d) {
    return 2 * decode_half_floats(k, f, E, d);
}

hipError_t launch_ffn_decode(const Geom& g, const FfnArgs& a, int prec, hipStream_t s);

// Hit/miss split of a one-token step ("Nanite for Experts", §5.5: the experts
// already resident run while the missing ones are still being copied in; the
// results are merged into the token's row).  Two launches of the decode
// kernel's split variant: the resident units first, the copied ones after
// their copies.  Each unit's term w (W_d h) comes from the same code in either
// launch, and the merge adds the terms in plan order with the shared expert
// last, so y does not depend on which units were resident.
enum { kSplitAll = 0, kSplitHits = 1, kSplitMisses = 2 };
constexpr int kSplitMaskWords = 1024 / 32;  // one bit per expert id (E <= 1024)
struct SplitSel {
    uint32_t miss[kSplitMaskWords];  // bit e: expert e is copied in by the step
    int which;     // kSplitAll: every unit, y written;
                   // kSplitHits: the units whose bit is clear and the shared expert, their terms
                   //   written to part, y untouched;
                   // kSplitMisses: the units whose bit is set; the other terms read from part; y written
    float* part;   // [top_k + 1, d] terms by hidden row (plan position; the shared expert's last)
};
inline int64_t split_part_floats(int k, int d) { return (int64_t)(k + 1) * d; }
// The split variant holds every W_d tile of the step in registers: (units) x
// (d_ff / 128) tiles at most kSplitMaxTiles.
constexpr int kSplitMaxTiles = 40;
hipError_t launch_ffn_split(const Geom& g, const FfnArgs& a, int prec, const SplitSel& sel, hipStream_t s);

// Prefill (T > kDecodeMaxT): bucket tiles on the matrix cores; see ffn_prefill.hip.
constexpr int kPrefillBM = 64;     // tokens per large tile
constexpr int kPrefillWide = 128;  // tokens per wide tile (buckets of at least wide_min tokens)
constexpr int kWideMinDefault = 1024;

struct PrefillArgs {
    Geom g;
    const uint8_t* pool;
    int64_t payload_bytes;
    const int32_t* pt;
    int layer, E, n_slots;
    const uint8_t* shared;
    const int32_t* n_active;
    const int32_t* experts;
    const int32_t* offsets;
    const int32_t* entries;
    const float* topk_w;
    int k;
    const void* x;
    int x_bf16;
    int T, d, f;
    int gemm_min;          // bf16 mode: buckets with at least this many tokens use 64-token tiles
    void* h;               // [T*k + T, f] hidden rows per bucket entry (+ shared per token):
                           // bf16 in bf16 mode, fp32 otherwise
    float* part;           // [T*k + T, d] partial output rows
    int32_t* inv;          // [T*k] plan position of entry t*k + j
    int32_t* sched_big;    // [4 * cap_big] tile records (16-byte aligned), 64-token tiles
    int32_t* sched_small;  // [4 * cap_small] tile records (16-byte aligned), 16-token tiles
    int32_t* sched_wide;   // [4 * cap_wide] tile records (16-byte aligned), 128-token tiles
    int32_t* n_tiles;      // [4]: 64-token tiles, 16-token tiles, the plan positions the units
                           // cover, 128-token tiles
    int cap_big, cap_small, cap_wide;  // records the three arrays hold
    int wide_min;          // bf16 mode: buckets with at least this many tokens use 128-token tiles
    float* y;
    int* err;
};

// Upper bounds on the tiles of each size a call of T tokens can need.
void prefill_max_tiles(int64_t T, int k, int E, bool shared, int* big_tiles, int* small_tiles, int* wide_tiles);

// The chunk path's workspace carved out of one buffer (256-byte aligned
// sections): hidden rows, partial rows, entry inverse, the two tile-record
// arrays and the counts.  Returns the bytes needed for T tokens.
struct PrefillLayout {
    size_t h, part, inv, sched_big, sched_small, sched_wide, n_tiles, total;
    int cap_big, cap_small, cap_wide;
};
PrefillLayout prefill_layout(int64_t T, int k, int E, int d, int f, bool bf16_hidden);

// The fixed device array behind moe_expert_ffn_static, and its address on the
// current device (taken once per device).
constexpr size_t kStaticScratchBytes = MOE_STATIC_SCRATCH_BYTES;
hipError_t static_scratch(void** out);
// Streams of a prefill call: the caller's, and an auxiliary one (null: all on
// s) on which the 64-token tile chain runs beside the 16-token one, forked
// from and joined back into s with the two events.
struct PrefillStreams {
    hipStream_t s;
    hipStream_t aux;
    hipEvent_t fork, join;
};
hipError_t launch_ffn_prefill(const PrefillArgs& a, int prec, const PrefillStreams& st);

// Peak references (probe.hip): a streaming read of `bytes` (a multiple of 16)
// by `wgs` workgroups, and `iters` rounds of bf16 matrix-core products (shape 0:
// 16x16x32, 1: 32x32x16) over `grid` workgroups of 4 waves, with the flops the
// latter performs.
// Page-table writes (entry index, value) applied by one launch.
constexpr int kPtBatch = 128;
struct PtWrites {
    int32_t n;
    int32_t idx[kPtBatch];
    int32_t val[kPtBatch];
};
hipError_t launch_pt_write(int32_t* pt, const PtWrites& w, hipStream_t s);

// Payload copies of one pull launch: src[i] (pinned host or device memory, as
// the kernel addresses it) -> dst[i] (a slot), `words` 16-byte words each.
constexpr int kPullMax = 32;
constexpr int kPullWorkgroups = 64;  // measured best for reads over the host bus
struct PullArgs {
    const uint4* src[kPullMax];
    uint4* dst[kPullMax];
    int32_t n;
    uint32_t words;
};
static_assert(2 * kPullMax <= kPtBatch, "a pull launch writes up to two entries per copy");
hipError_t launch_pull(const PullArgs& a, int32_t* pt, const PtWrites& w, hipStream_t s);

hipError_t launch_probe_read(const void* src, int64_t bytes, int wgs, uint32_t* sink, hipStream_t s);
hipError_t launch_probe_mfma(int iters, int grid, int shape, float* sink, hipStream_t s);
hipError_t launch_probe_lds(int iters, int grid, uint32_t* sink, hipStream_t s);
int64_t probe_mfma_flops(int iters, int grid, int shape);

}  // namespace moe
