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
        auto pow2_le64 = [](int v) { return v >= 1 && v <= 64 && (v & (v - 1)) == 0; };
        if (!pow2_le64(nb_d) || !pow2_le64(nb_f)) return false;
        // whole tiles only: rows per tile = 64 / blocks per row
        if (f % (kTileBlocks / nb_d) || d % (kTileBlocks / nb_f)) return false;
        tile_bytes = (int64_t)kTileBlocks * block_bytes(qt);
        gu_tiles = (int64_t)f * nb_d / kTileBlocks;
        d_tiles = (int64_t)d * nb_f / kTileBlocks;
        payload = (2 * gu_tiles + d_tiles) * tile_bytes;
        return true;
    }
    int64_t gate_tile(int64_t t) const { return 2 * t * tile_bytes; }
    int64_t up_tile(int64_t t) const { return (2 * t + 1) * tile_bytes; }
    int64_t down_tile(int64_t t) const { return (2 * gu_tiles + t) * tile_bytes; }
};

// Byte offsets inside one tile for block i (0..63).
__host__ __device__ inline int q8_lo(int i) { return 16 * i; }
__host__ __device__ inline int q8_hi(int i) { return 16 * kTileBlocks + 16 * i; }
__host__ __device__ inline int q8_scale(int i) { return 32 * kTileBlocks + 2 * i; }
__host__ __device__ inline int q4_nib(int i) { return 16 * i; }
__host__ __device__ inline int q4_scale(int i) { return 16 * kTileBlocks + 2 * i; }

// Device error word bits.
constexpr int kErrMiss = 1;     // unmapped expert met by a kernel
constexpr int kErrTimeout = 2;  // bounded wait gave up
constexpr int kErrBadId = 4;    // expert id out of range in a plan input

// ---- launchers (return hipError_t of the launch) ----

hipError_t launch_router_gemv(const void* x, int x_bf16, const float* w_r, int64_t T, int E, int d,
                              float* logits, hipStream_t s);
hipError_t launch_topk(const float* logits, int64_t T, int E, int k, int norm, int32_t* ids,
                       float* w, hipStream_t s);
hipError_t launch_plan(const int32_t* ids, int64_t T, int k, int E, const moe_plan& plan, int* err,
                       hipStream_t s);
hipError_t launch_dequant(const Geom& g, const uint8_t* payload, int prec, float* out, hipStream_t s);

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
    // outputs and workspace
    float* h;               // [T*k + T, f] hidden states
    float* y;               // [T, d]
    unsigned* sync;         // [2] inter-workgroup counters, zero between launches
    int* err;
    int spin_limit;
};

// Largest step the fused single-launch decode kernel takes.
constexpr int kDecodeMaxT = 4;

hipError_t launch_ffn_decode(const Geom& g, const FfnArgs& a, int prec, hipStream_t s);

}  // namespace moe
