// Decode step of the routed experts (T <= 4 tokens): every expert of the step
// in one launch — the expert-major operator that consumes routed positions and
// page-table entries for several resident experts at once ("Nanite for
// Experts", §12, milestone 1; §11.5: the unit of execution should be
// expert-major, not many separately orchestrated fragments) — followed by a
// small fixed-order combine launch.
//
// ffn_partial: one workgroup per (unit, chunk).  A unit is a routed expert of
//   the plan (ascending expert id) or the shared expert (last); a chunk is
//   ROWS consecutive hidden rows: 16 for Q8_0 (one code half of a 32-column
//   block of W_d, which the tile layout stores contiguously) and 32 for Q4_0
//   (whose nibble bytes hold both halves).  The workgroup
//     1. resolves the unit's slot through the page table ("Nanite for
//        Experts", §5.4; a -1 entry fails closed: NaN partials, error word),
//     2. issues every weight load of the chunk at once — its gate and up rows
//        and the matching columns of W_d (all d rows), one 16-byte load per
//        lane per tile piece — plus the bucket's activations (into LDS),
//     3. computes h_c = silu(W_g[c] x) * (W_u[c] x) for each token of the bucket
//        (each lane's blocks summed over its tiles, then the four lanes of a
//        row and the waves, in fixed order), into LDS,
//     4. after one workgroup barrier, each lane owns one output row of W_d's
//        columns: ROWS codes times h_c broadcast from LDS, no cross-lane sum,
//        and writes the partial row P[entry][chunk][row].
//   No workgroup ever waits for another.
// combine: y[t, i] = sum over t's entries in plan order (ascending expert) of
//   w * (sum over chunks of P) + the shared expert's chunks, in one fixed
//   order that depends only on expert ids and ranks, never on slots.
#include "device_util.h"
#include "internal.h"

namespace moe {
namespace {

// Workgroup shape: ROWS hidden rows per chunk, 8 waves.  With up to 4 tokens
// per bucket the down tiles are loaded after the gate/up products, so that the
// activations of four tokens and all tiles are not live at once.
template <int QT> constexpr int chunk_rows() { return QT == MOE_Q8_0 ? 16 : 32; }
constexpr int kMaxD = 2048;  // largest d_model
template <int TG> constexpr int wg_waves() { return 8; }
template <int TG> constexpr bool down_early() { return TG < 4; }
// PPW gate/up tile pairs and DPW down tiles per wave are compile-time, so each
// wave holds exactly its tiles in registers: (1,1) for small d_model, (2,4)
// for Q8_0 at d_model 2048 (16-row chunks), (4,4) otherwise.

template <int QT> struct Tile;
template <> struct Tile<MOE_Q8_0> {
    uint4 lo, hi;
    uint32_t s;
    __device__ void load(const uint8_t* t, int i) {
        lo = *(const uint4*)(t + q8_lo(i));
        hi = *(const uint4*)(t + q8_hi(i));
        s = *(const uint16_t*)(t + q8_scale(i));
    }
    __device__ void clear() { lo = hi = make_uint4(0, 0, 0, 0); s = 0; }
    // one code half (codes 0..15 or 16..31 of the lane's block) into lo
    __device__ void load_half(const uint8_t* t, int i, int half) {
        lo = *(const uint4*)(t + (half ? q8_hi(i) : q8_lo(i)));
        s = *(const uint16_t*)(t + q8_scale(i));
    }
};
template <> struct Tile<MOE_Q4_0> {
    uint4 nib;
    uint32_t s;
    __device__ void load(const uint8_t* t, int i) {
        nib = *(const uint4*)(t + q4_nib(i));
        s = *(const uint16_t*)(t + q4_scale(i));
    }
    __device__ void clear() { nib = make_uint4(0, 0, 0, 0); s = 0; }
};

// Weight as multiplied: PREC_F32 keeps the code (the scale is applied once after
// the dot product, so each product is the exact dequantised weight times v up
// to rounding); PREC_BF16 rounds each exact d*q to bf16.
template <int PREC>
__device__ inline float wq(float code, float s) { return PREC == MOE_PREC_BF16 ? round_bf16(code * s) : code; }

// Dot products of the lane's block with N 32-float vectors v[n].
template <int QT, int PREC, int N>
__device__ inline void tile_dots(const Tile<QT>& t, const float (&v)[N][32], float (&acc)[N]) {
    const float s = f16_bits_to_f32(t.s);
#pragma unroll
    for (int n = 0; n < N; n++) acc[n] = 0.f;
    if constexpr (QT == MOE_Q8_0) {
        const uint32_t w[8] = {t.lo.x, t.lo.y, t.lo.z, t.lo.w, t.hi.x, t.hi.y, t.hi.z, t.hi.w};
#pragma unroll
        for (int m = 0; m < 8; m++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float c = wq<PREC>(i8(w[m], j), s);
#pragma unroll
                for (int n = 0; n < N; n++) acc[n] = fmaf(c, v[n][4 * m + j], acc[n]);
            }
    } else {
        const uint32_t w[4] = {t.nib.x, t.nib.y, t.nib.z, t.nib.w};
#pragma unroll
        for (int m = 0; m < 4; m++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t b = (w[m] >> (8 * j)) & 0xFF;
                const float clo = wq<PREC>((float)((int)(b & 15) - 8), s);
                const float chi = wq<PREC>((float)((int)(b >> 4) - 8), s);
#pragma unroll
                for (int n = 0; n < N; n++) {
                    acc[n] = fmaf(clo, v[n][4 * m + j], acc[n]);
                    acc[n] = fmaf(chi, v[n][16 + 4 * m + j], acc[n]);
                }
            }
    }
    if (PREC == MOE_PREC_F32) {
#pragma unroll
        for (int n = 0; n < N; n++) acc[n] *= s;
    }
}

// Dot products of the 16 codes held in t.lo (a Q8_0 half block) with N
// 16-float vectors.
template <int PREC, int N>
__device__ inline void half_dots(const Tile<MOE_Q8_0>& t, const float (&v)[N][16], float (&acc)[N]) {
    const float s = f16_bits_to_f32(t.s);
#pragma unroll
    for (int n = 0; n < N; n++) acc[n] = 0.f;
    const uint32_t w[4] = {t.lo.x, t.lo.y, t.lo.z, t.lo.w};
#pragma unroll
    for (int m = 0; m < 4; m++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float c = wq<PREC>(i8(w[m], j), s);
#pragma unroll
            for (int n = 0; n < N; n++) acc[n] = fmaf(c, v[n][4 * m + j], acc[n]);
        }
    if (PREC == MOE_PREC_F32) {
#pragma unroll
        for (int n = 0; n < N; n++) acc[n] *= s;
    }
}

struct Grid {
    int units_max;  // routed units allotted (the plan may use fewer) + shared
    int n_chunks;   // d_ff / ROWS
    int pairs;      // gate/up tile pairs per chunk = ROWS * (d_model/32) / 64
    int dtiles;     // down tiles per W_d column block = d_model / 64
    int nbd, d, d_ff;
    int64_t tile_bytes, down_off;
};

template <int QT, int PREC, int TG, int PPW, int DPW>
__global__ __launch_bounds__(wg_waves<TG>() * 64, TG == 1 ? 4 : 2) void ffn_partial_kernel(FfnArgs a, Grid g) {
    constexpr int ROWS = chunk_rows<QT>();
    constexpr int WAVES = wg_waves<TG>();
    __shared__ float h_c[TG][ROWS];
    __shared__ __attribute__((aligned(16))) float xl[TG][kMaxD];
    __shared__ float red[2][WAVES][ROWS / 16][TG][16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int u = blockIdx.x / g.n_chunks, c = blockIdx.x - u * g.n_chunks;

    // Level 1: small-table loads that do not depend on each other (indices
    // clamped into range so all can be in flight together).
    const int na = *a.n_active;
    const int e = a.experts[min(u, a.E - 1)];
    const int o0 = a.offsets[min(u, a.E)];
    const int o1 = a.offsets[min(u + 1, a.E)];
    const bool has_shared = a.shared != nullptr;
    if (u >= na + (has_shared ? 1 : 0)) return;  // uniform over the workgroup
    const bool routed = u < na;
    // Level 2: the page-table entry and the bucket's token ids.
    const bool e_ok = e >= 0 && e < a.E;
    const int slot = a.pt[(int64_t)a.layer * a.E + (e_ok ? e : 0)];
    const int b0 = routed ? o0 : 0;
    const int nb = routed ? o1 - o0 : a.T;  // tokens in the bucket, <= T <= TG
    int tok[TG], prow[TG];
#pragma unroll
    for (int gi = 0; gi < TG; gi++) {
        const bool in = gi < nb;
        tok[gi] = !in ? -1 : !routed ? gi : a.T == 1 ? 0 : a.entries[b0 + gi] / a.k;
        prow[gi] = !in ? -1 : routed ? b0 + gi : a.T * a.k + gi;
    }
    const uint8_t* base = !routed ? a.shared
                        : (e_ok && slot >= 0 && slot < a.n_slots) ? a.pool + (int64_t)slot * a.payload_bytes
                                                                  : nullptr;
    if (!base && threadIdx.x == 0) atomicOr(a.err, kErrMiss);
    const float qnan = __uint_as_float(0x7FC00000u);

    // Level 3: every weight load of the chunk, then the activations.  The
    // chunk's gate/up rows are tiles [c*pairs, (c+1)*pairs) of each matrix.
    // Its W_d columns: Q8_0 chunk c is code half c%2 of column block c/2;
    // Q4_0 chunk c is column block c.  A column block is dtiles tiles.
    const int colblk = QT == MOE_Q8_0 ? c >> 1 : c;
    Tile<QT> tg[PPW], tu[PPW], td[DPW];
#pragma unroll
    for (int q = 0; q < PPW; q++) {
        const int pi = wave + q * WAVES;
        if (base && pi < g.pairs) {
            const int64_t t = (int64_t)c * g.pairs + pi;
            tg[q].load(base + 2 * t * g.tile_bytes, lane);
            tu[q].load(base + (2 * t + 1) * g.tile_bytes, lane);
        } else {
            tg[q].clear();
            tu[q].clear();
        }
    }
    auto load_down = [&]() {
#pragma unroll
        for (int q = 0; q < DPW; q++) {
            const int pi = wave + q * WAVES;
            if (base && pi < g.dtiles) {
                const uint8_t* tp = base + g.down_off + ((int64_t)colblk * g.dtiles + pi) * g.tile_bytes;
                if constexpr (QT == MOE_Q8_0) td[q].load_half(tp, lane, c & 1);
                else td[q].load(tp, lane);
            } else {
                td[q].clear();
            }
        }
    };
    if constexpr (down_early<TG>()) load_down();
    // The bucket's activations into LDS, fp32 (bf16-rounded in bf16 mode).
    for (int gi = 0; gi < TG; gi++)
        for (int i = threadIdx.x * 4; i < g.d; i += WAVES * 64 * 4) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (tok[gi] >= 0) {
                if (a.x_bf16) {
                    const uint2 w = *(const uint2*)((const uint16_t*)a.x + (int64_t)tok[gi] * g.d + i);
                    v = make_float4(bf16_bits_to_f32(w.x & 0xFFFF), bf16_bits_to_f32(w.x >> 16),
                                    bf16_bits_to_f32(w.y & 0xFFFF), bf16_bits_to_f32(w.y >> 16));
                } else {
                    v = *(const float4*)((const float*)a.x + (int64_t)tok[gi] * g.d + i);
                    if (PREC == MOE_PREC_BF16)
                        v = make_float4(round_bf16(v.x), round_bf16(v.y), round_bf16(v.z), round_bf16(v.w));
                }
            }
            *(float4*)&xl[gi][i] = v;
        }
    lds_barrier();

    // gate/up.  Pair pi of the chunk is tile (row group pi / K4, column group
    // pi % K4); lane (n, j) = (lane % 16, lane / 16) holds column block
    // 4 (pi % K4) + j of row n.  Each lane sums its blocks' dot products over the
    // wave's pairs; the four lanes of a row, then the waves (through LDS), are
    // added in fixed order.
    constexpr int RG = ROWS / 16;
    const int K4 = g.nbd >> 2;
    const int nrow = lane & 15, jb = lane >> 4;
    float accg[RG][TG], accu[RG][TG];
#pragma unroll
    for (int r = 0; r < RG; r++)
#pragma unroll
        for (int gi = 0; gi < TG; gi++) accg[r][gi] = accu[r][gi] = 0.f;
#pragma unroll
    for (int q = 0; q < PPW; q++) {
        const int pi = wave + q * WAVES;
        if (pi >= g.pairs) break;
        const int rgl = pi / K4, cb = 4 * (pi - rgl * K4) + jb;
        float xs[TG][32];
#pragma unroll
        for (int gi = 0; gi < TG; gi++)
#pragma unroll
            for (int m = 0; m < 8; m++) {
                const float4 v = *(const float4*)&xl[gi][cb * kQK + 4 * m];
                xs[gi][4 * m] = v.x; xs[gi][4 * m + 1] = v.y; xs[gi][4 * m + 2] = v.z; xs[gi][4 * m + 3] = v.w;
            }
        float dg[TG], du[TG];
        tile_dots<QT, PREC, TG>(tg[q], xs, dg);
        tile_dots<QT, PREC, TG>(tu[q], xs, du);
#pragma unroll
        for (int r = 0; r < RG; r++)
            if (r == rgl)
#pragma unroll
                for (int gi = 0; gi < TG; gi++) {
                    accg[r][gi] += dg[gi];
                    accu[r][gi] += du[gi];
                }
    }
#pragma unroll
    for (int r = 0; r < RG; r++)
#pragma unroll
        for (int gi = 0; gi < TG; gi++) {
            const float gs = cross_row_sum(accg[r][gi]), us = cross_row_sum(accu[r][gi]);
            if (jb == 0) {
                red[0][wave][r][gi][nrow] = gs;
                red[1][wave][r][gi][nrow] = us;
            }
        }
    if constexpr (!down_early<TG>()) load_down();
    lds_barrier();
    if (threadIdx.x < ROWS * TG) {
        const int gi = threadIdx.x / ROWS, rr = threadIdx.x - gi * ROWS, r = rr >> 4, n = rr & 15;
        float gs = 0.f, us = 0.f;
        for (int w = 0; w < WAVES; w++) {
            gs += red[0][w][r][gi][n];
            us += red[1][w][r][gi][n];
        }
        float hv = silu(gs) * us;
        if (PREC == MOE_PREC_BF16) hv = round_bf16(hv);
        h_c[gi][rr] = base ? hv : qnan;
    }
    __syncthreads();

    // down: the lane owns output row (pi * 64 + lane)
    float hv[TG][ROWS];
#pragma unroll
    for (int gi = 0; gi < TG; gi++)
#pragma unroll
        for (int j = 0; j < ROWS; j++) hv[gi][j] = h_c[gi][j];
#pragma unroll
    for (int q = 0; q < DPW; q++) {
        const int pi = wave + q * WAVES;
        if (pi >= g.dtiles) break;
        float acc[TG];
        if constexpr (QT == MOE_Q8_0) half_dots<PREC, TG>(td[q], hv, acc);
        else tile_dots<QT, PREC, TG>(td[q], hv, acc);
        const int row = pi * kTileBlocks + lane;
#pragma unroll
        for (int gi = 0; gi < TG; gi++)
            if (prow[gi] >= 0) a.part[((int64_t)prow[gi] * g.n_chunks + c) * g.d + row] = base ? acc[gi] : qnan;
    }
}

// combine: a workgroup of 256 threads covers 64 outputs of one token as 16
// float4 quads x 16 entry slots.  Token t's entries are found in plan order
// (ascending expert) with one ballot; each thread sums every chunk of its
// (quad, entry) with all loads in flight, and the per-entry sums are then
// weighted and added per output in plan order, shared expert last.
constexpr int kCombineQuads = 16;
constexpr int kCombineSlots = 16;
constexpr int kMaxCombine = 33;  // top_k <= 32 entries + shared
constexpr int kChunkBatch = 16;

__global__ __launch_bounds__(kCombineQuads * kCombineSlots) void combine_kernel(FfnArgs a, int n_chunks, int d) {
    __shared__ int s_q[kMaxCombine];
    __shared__ float s_w[kMaxCombine];
    __shared__ int s_cnt;
    __shared__ float4 red[kMaxCombine][kCombineQuads];
    const int t = blockIdx.y;
    const int qd = threadIdx.x % kCombineQuads, slot = threadIdx.x / kCombineQuads;
    const int i4 = blockIdx.x * kCombineQuads + qd;  // output quad
    const int n_ent = a.T * a.k;
    if (threadIdx.x < 64) {
        int base = 0;
        for (int q0 = 0; q0 < n_ent; q0 += 64) {
            const int q = q0 + threadIdx.x;
            const int ent = q < n_ent ? a.entries[q] : -1;
            const bool mine = q < n_ent && ent / a.k == t;
            const uint64_t m = __ballot(mine);
            if (mine) {
                const int r = base + __popcll(m & ((1ull << threadIdx.x) - 1ull));
                s_q[r] = q;
                s_w[r] = a.topk_w[ent];
            }
            base += __popcll(m);
        }
        if (threadIdx.x == 0) {
            int cnt = base;
            if (a.shared) {
                s_q[cnt] = n_ent + t;
                s_w[cnt] = 1.0f;
                cnt++;
            }
            s_cnt = cnt;
        }
    }
    __syncthreads();
    const int cnt = s_cnt;
    const bool in = i4 * 4 < d;
    for (int j = slot; j < cnt; j += kCombineSlots) {
        const float4* p = (const float4*)(a.part + (int64_t)s_q[j] * n_chunks * d) + i4;
        float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int c0 = 0; c0 < n_chunks; c0 += kChunkBatch) {
            float4 v[kChunkBatch];
#pragma unroll
            for (int b = 0; b < kChunkBatch; b++)
                v[b] = (in && c0 + b < n_chunks) ? p[(int64_t)(c0 + b) * (d / 4)] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int b = 0; b < kChunkBatch; b++) {
                sum.x += v[b].x; sum.y += v[b].y; sum.z += v[b].z; sum.w += v[b].w;
            }
        }
        red[j][qd] = sum;
    }
    __syncthreads();
    if (slot == 0 && in) {
        const int n_routed = a.shared ? cnt - 1 : cnt;
        float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < cnt; j++) {
            const float4 s4 = red[j][qd];
            const float wj = j < n_routed ? s_w[j] : 1.0f;
            if (j < n_routed) {
                y.x = fmaf(wj, s4.x, y.x); y.y = fmaf(wj, s4.y, y.y);
                y.z = fmaf(wj, s4.z, y.z); y.w = fmaf(wj, s4.w, y.w);
            } else {
                y.x += s4.x; y.y += s4.y; y.z += s4.z; y.w += s4.w;
            }
        }
        *(float4*)(a.y + (int64_t)t * d + i4 * 4) = y;
    }
}

template <int QT, int PREC, int TG, int PPW, int DPW>
hipError_t launch_t(const Grid& g, const FfnArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((ffn_partial_kernel<QT, PREC, TG, PPW, DPW>), dim3(g.units_max * g.n_chunks),
                       dim3(wg_waves<TG>() * 64), 0, s, a, g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(combine_kernel, dim3((g.d / 4 + kCombineQuads - 1) / kCombineQuads, a.T),
                       dim3(kCombineQuads * kCombineSlots), 0, s, a, g.n_chunks, g.d);
    return hipGetLastError();
}

template <int QT, int PREC, int TG>
hipError_t launch_w(Grid g, const FfnArgs& a, hipStream_t s) {
    constexpr int ROWS = chunk_rows<QT>();
    constexpr int W = wg_waves<TG>();
    g.n_chunks = g.d_ff / ROWS;
    g.pairs = ROWS * g.nbd / kTileBlocks;
    if (g.pairs < 1) return hipErrorInvalidValue;
    if (g.pairs <= W && g.dtiles <= W) return launch_t<QT, PREC, TG, 1, 1>(g, a, s);
    if (g.pairs <= 2 * W && g.dtiles <= 4 * W) return launch_t<QT, PREC, TG, 2, 4>(g, a, s);
    if (g.pairs <= 4 * W && g.dtiles <= 4 * W) return launch_t<QT, PREC, TG, 4, 4>(g, a, s);
    return hipErrorInvalidValue;
}

template <int QT, int PREC>
hipError_t launch_tg(const Grid& g, const FfnArgs& a, hipStream_t s) {
    if (a.T <= 1) return launch_w<QT, PREC, 1>(g, a, s);
    if (a.T <= 2) return launch_w<QT, PREC, 2>(g, a, s);
    return launch_w<QT, PREC, 4>(g, a, s);
}

}  // namespace

hipError_t launch_ffn_decode(const Geom& g, const FfnArgs& a, int prec, hipStream_t s) {
    Grid gr{};
    gr.units_max = min(a.T * a.k, a.E) + (a.shared ? 1 : 0);
    gr.dtiles = g.d / kTileBlocks;
    gr.nbd = g.nb_d;
    gr.d = g.d;
    gr.d_ff = g.f;
    gr.tile_bytes = g.tile_bytes;
    gr.down_off = 2 * g.gu_tiles * g.tile_bytes;
    if (g.qtype == MOE_Q8_0)
        return prec == MOE_PREC_BF16 ? launch_tg<MOE_Q8_0, MOE_PREC_BF16>(gr, a, s)
                                     : launch_tg<MOE_Q8_0, MOE_PREC_F32>(gr, a, s);
    return prec == MOE_PREC_BF16 ? launch_tg<MOE_Q4_0, MOE_PREC_BF16>(gr, a, s)
                                 : launch_tg<MOE_Q4_0, MOE_PREC_F32>(gr, a, s);
}

}  // namespace moe
