// Routed experts for a chunk of T > 4 tokens (prefill): per bucket, the gate/up
// and down products on the matrix cores.  The expert union ("Nanite for
// Experts", §5.3) means each tile of a bucket's tokens reads its expert's
// weights once.
//
//   schedule  one workgroup: the tiles of every bucket and of the shared expert
//             (all T tokens): 64-token tiles for buckets of at least gemm_min
//             tokens in bf16 mode, 16-token tiles otherwise; and the inverse of
//             the plan's entries for the combine
//   gate/up   one wave per (tile, 16 features).  Per step of 4 weight blocks
//             (128 columns), lane (n, g) = (lane % 16, lane / 16) reads block
//             g of feature n's row (the 4 blocks are 64 contiguous bytes of the
//             row per code half) and dequantises it straight into the B operand;
//             lane (m, g) reads the same 32 activation columns of token m for
//             the A operand.  bf16 mode: v_mfma_f32_16x16x32_bf16, the operand
//             slot (g, i) of MFMA s holding element 8s + i of block g; fp32 mode:
//             exact weights on v_mfma_f32_16x16x4_f32, slot g of MFMA j holding
//             element j of block g.  h = silu(g) * u, bf16-rounded in bf16 mode,
//             to one workspace row per bucket entry (the shared expert: per token)
//   down      the same over d_ff, one wave per (tile, 16 output rows); the
//             payload keeps a column block's rows together, so the 16 lanes of
//             a block group read 16 consecutive rows (256 contiguous bytes);
//             partial rows to the workspace
//   combine   y[t] = sum_j w[t,j] * partial(t,j) + shared partial(t), in rank
//             order j, shared last: fixed, slot-independent.
// No wave waits on another: the kernels have no barriers besides the schedule's.
#include <algorithm>

#include "device_util.h"
#include "internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BIG = kPrefillBM;  // tokens per large tile (4 row groups of 16)
constexpr int SMALL = 16;        // tokens per small tile
constexpr int WAVES = 4;         // waves per workgroup, 16 features / rows each
constexpr int COLS = WAVES * 16; // features / output rows per workgroup item

__device__ inline const uint8_t* unit_base(const PrefillArgs& a, int u, int na) {
    if (u == na) return a.shared;
    const int e = a.experts[u];
    if (e < 0 || e >= a.E) return nullptr;
    const int s = a.pt[(int64_t)a.layer * a.E + e];
    return (s >= 0 && s < a.n_slots) ? a.pool + (int64_t)s * a.payload_bytes : nullptr;
}

// Bucket geometry of unit u: first plan position and size.
__device__ inline void unit_rows(const PrefillArgs& a, int u, int na, int* p0, int* M) {
    if (u == na) { *p0 = 0; *M = a.T; }
    else { *p0 = a.offsets[u]; *M = a.offsets[u + 1] - a.offsets[u]; }
}

// Token and workspace row of bucket row m.
__device__ inline int row_token(const PrefillArgs& a, int u, int na, int p0, int m) {
    return u == na ? m : a.entries[p0 + m] / a.k;
}
__device__ inline int row_slot(const PrefillArgs& a, int u, int na, int p0, int m) {
    return u == na ? a.T * a.k + m : p0 + m;
}

// ---- schedule --------------------------------------------------------------

__device__ int block_prefix(int v, int* wave_tot, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int n = __shfl_up(incl, o, 64);
        if (lane >= o) incl += n;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        int s = 0;
        for (int w = 0; w < (int)(blockDim.x >> 6); w++) { const int t = wave_tot[w]; wave_tot[w] = s; s += t; }
        *total = s;
    }
    __syncthreads();
    const int r = wave_tot[wave] + incl - v;
    __syncthreads();
    return r;
}

// sched_big / sched_small: (unit, first row) per tile; n_tiles = {big, small}.
__global__ __launch_bounds__(1024) void schedule_kernel(PrefillArgs a, int prec) {
    __shared__ int wave_tot[16];
    __shared__ int tot_b, tot_s;
    const int na = *a.n_active;
    const int n_units = na + (a.shared ? 1 : 0);
    int base_b = 0, base_s = 0;
    for (int u0 = 0; u0 < n_units; u0 += 1024) {
        const int u = u0 + threadIdx.x;
        int tb = 0, ts = 0;
        if (u < n_units) {
            int p0, M;
            unit_rows(a, u, na, &p0, &M);
            if (prec == MOE_PREC_BF16 && M >= a.gemm_min) tb = (M + BIG - 1) / BIG;
            else ts = (M + SMALL - 1) / SMALL;
        }
        const int fb = base_b + block_prefix(tb, wave_tot, &tot_b);
        const int fs = base_s + block_prefix(ts, wave_tot, &tot_s);
        for (int i = 0; i < tb; i++) {
            a.sched_big[2 * (fb + i)] = u;
            a.sched_big[2 * (fb + i) + 1] = i * BIG;
        }
        for (int i = 0; i < ts; i++) {
            a.sched_small[2 * (fs + i)] = u;
            a.sched_small[2 * (fs + i) + 1] = i * SMALL;
        }
        base_b += tot_b;
        base_s += tot_s;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        a.n_tiles[0] = base_b;
        a.n_tiles[1] = base_s;
    }
    const int n_ent = a.T * a.k;
    for (int p = threadIdx.x; p < n_ent; p += blockDim.x) {
        const int ent = a.entries[p];
        if (ent >= 0 && ent < n_ent) a.inv[ent] = p;
    }
}

// ---- weights ------------------------------------------------------------------

// One lane's block: its codes and scale, as stored in a tile.
template <int QT> struct Raw;
template <> struct Raw<MOE_Q8_0> {
    uint4 lo, hi;
    uint32_t s;
    __device__ void load(const uint8_t* t, int i) {
        lo = *(const uint4*)(t + q8_lo(i));
        hi = *(const uint4*)(t + q8_hi(i));
        s = *(const uint16_t*)(t + q8_scale(i));
    }
    __device__ void zero() { lo = hi = make_uint4(0, 0, 0, 0); s = 0; }
    // The 32 weights d*q, exact in fp32 (an fp16 scale times an 8-bit code needs
    // 19 significant bits).  Codes are biased to unsigned bytes (q + 128) so each
    // converts in one step; fma(d, q + 128, -128 d) rounds once, to d*q itself.
    __device__ void values(float (&v)[32]) const {
        const float d = f16_bits_to_f32(s), o = -128.f * d;
        const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int p = 0; p < 8; p++) {
            const uint32_t b = w[p] ^ 0x80808080u;
#pragma unroll
            for (int i = 0; i < 4; i++) v[4 * p + i] = fmaf(d, (float)((b >> (8 * i)) & 0xFF), o);
        }
    }
};
template <> struct Raw<MOE_Q4_0> {
    uint4 nib;
    uint32_t s;
    __device__ void load(const uint8_t* t, int i) {
        nib = *(const uint4*)(t + q4_nib(i));
        s = *(const uint16_t*)(t + q4_scale(i));
    }
    __device__ void zero() { nib = make_uint4(0, 0, 0, 0); s = 0; }
    // Byte b holds element b (low nibble) and element b + 16 (high nibble),
    // each as q + 8.
    __device__ void values(float (&v)[32]) const {
        const float d = f16_bits_to_f32(s), o = -8.f * d;
        const uint32_t w[4] = {nib.x, nib.y, nib.z, nib.w};
#pragma unroll
        for (int p = 0; p < 4; p++) {
            const uint32_t lo4 = w[p] & 0x0F0F0F0Fu, hi4 = (w[p] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                v[4 * p + i] = fmaf(d, (float)((lo4 >> (8 * i)) & 0xFF), o);
                v[16 + 4 * p + i] = fmaf(d, (float)((hi4 >> (8 * i)) & 0xFF), o);
            }
        }
    }
};

__device__ inline uint32_t pack_bf16(float a, float b) {
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// B operands of the 4 bf16 MFMAs of a block: weights rounded to bf16, MFMA s
// taking elements 8s..8s+7.
template <int QT>
__device__ inline void b_operands(const Raw<QT>& r, bf16x8 (&b)[4]) {
    float v[32];
    r.values(v);
#pragma unroll
    for (int s = 0; s < 4; s++) {
        const uint4 q = make_uint4(pack_bf16(v[8 * s], v[8 * s + 1]), pack_bf16(v[8 * s + 2], v[8 * s + 3]),
                                   pack_bf16(v[8 * s + 4], v[8 * s + 5]), pack_bf16(v[8 * s + 6], v[8 * s + 7]));
        b[s] = __builtin_bit_cast(bf16x8, q);
    }
}

// ---- activation rows ------------------------------------------------------------

// 8 consecutive values of a row starting at column c, as bf16 (fp32 rows are
// rounded to nearest even); zero for a padding row (row < 0).
__device__ inline bf16x8 row8_bf16(const void* base, bool is_bf16, int64_t pitch, int row, int c) {
    uint4 q = make_uint4(0, 0, 0, 0);
    if (row >= 0) {
        if (is_bf16) {
            q = *(const uint4*)((const uint16_t*)base + row * pitch + c);
        } else {
            const float* p = (const float*)base + row * pitch + c;
            const float4 f0 = *(const float4*)p, f1 = *(const float4*)(p + 4);
            q = make_uint4(pack_bf16(f0.x, f0.y), pack_bf16(f0.z, f0.w), pack_bf16(f1.x, f1.y),
                           pack_bf16(f1.z, f1.w));
        }
    }
    return __builtin_bit_cast(bf16x8, q);
}

// 32 consecutive values of a row starting at column c, as fp32 (bf16 widened
// exactly); zero for a padding row.
__device__ inline void row32_f32(const void* base, bool is_bf16, int64_t pitch, int row, int c, float (&v)[32]) {
    if (row < 0) {
#pragma unroll
        for (int j = 0; j < 32; j++) v[j] = 0.f;
        return;
    }
    if (is_bf16) {
        const uint4* p = (const uint4*)((const uint16_t*)base + row * pitch + c);
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const uint4 w = p[q];
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                v[8 * q + 2 * i] = __uint_as_float(ww[i] << 16);
                v[8 * q + 2 * i + 1] = __uint_as_float(ww[i] & 0xFFFF0000u);
            }
        }
    } else {
        const float4* p = (const float4*)((const float*)base + row * pitch + c);
#pragma unroll
        for (int q = 0; q < 8; q++) {
            const float4 f = p[q];
            v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
        }
    }
}

// ---- the tile product ------------------------------------------------------------
//
// One wave: C[16 R tokens][16 columns] for MATS weight matrices sharing the
// A operand (gate and up: 2; down: 1), over nkb K blocks.  Lane (n, g) owns
// block g of each step for column n; lane (m, g) the same block of token rows
// m, m + 16, ...  blk(mat, col, kb, &tile_ptr, &lane_in_tile) locates a block.

template <int QT, int PREC, int R, int MATS, class BlockAt>
__device__ void tile_product(const void* A, bool a_bf16, int64_t a_pitch, const int (&arow)[R], int nkb,
                             BlockAt blk, f32x4 (&acc)[MATS][R]) {
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < MATS; mt++)
#pragma unroll
        for (int r = 0; r < R; r++) acc[mt][r] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int kb0 = 0; kb0 < nkb; kb0 += 4) {
        const int kb = kb0 + g;
        const bool live = kb < nkb;
        Raw<QT> raw[MATS];
#pragma unroll
        for (int mt = 0; mt < MATS; mt++) {
            if (live) {
                const uint8_t* t;
                int i;
                blk(mt, n, kb, &t, &i);
                raw[mt].load(t, i);
            } else {
                raw[mt].zero();
            }
        }
        const int c = (live ? kb : 0) * kQK;
        if constexpr (PREC == MOE_PREC_BF16) {
            bf16x8 b[MATS][4];
#pragma unroll
            for (int mt = 0; mt < MATS; mt++) b_operands<QT>(raw[mt], b[mt]);
#pragma unroll
            for (int r = 0; r < R; r++) {
                const int row = live ? arow[r] : -1;
#pragma unroll
                for (int s = 0; s < 4; s++) {
                    const bf16x8 av = row8_bf16(A, a_bf16, a_pitch, row, c + 8 * s);
#pragma unroll
                    for (int mt = 0; mt < MATS; mt++)
                        acc[mt][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[mt][s], acc[mt][r], 0, 0, 0);
                }
            }
        } else {
            static_assert(R == 1, "fp32 tiles are 16 tokens");
            float w[MATS][32], x[32];
#pragma unroll
            for (int mt = 0; mt < MATS; mt++) raw[mt].values(w[mt]);
            row32_f32(A, a_bf16, a_pitch, live ? arow[0] : -1, c, x);
#pragma unroll
            for (int j = 0; j < 32; j++)
#pragma unroll
                for (int mt = 0; mt < MATS; mt++)
                    acc[mt][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(x[j], w[mt][j], acc[mt][0], 0, 0, 0);
        }
    }
}

// Work item i of a launch: (tile, column group of COLS).  Big tiles first.
struct Item {
    int u, m0, M, p0;
    bool big;
};

__device__ inline bool item_at(const PrefillArgs& a, int na, int i, int ngroups, Item* it, int* col0) {
    const int nb = a.n_tiles[0] * ngroups;
    int ti, rows;
    const int32_t* sched;
    if (i < nb) {
        ti = i / ngroups; sched = a.sched_big; rows = BIG; it->big = true;
    } else {
        i -= nb;
        ti = i / ngroups;
        if (ti >= a.n_tiles[1]) return false;
        sched = a.sched_small; rows = SMALL; it->big = false;
    }
    *col0 = (i % ngroups) * COLS;
    it->u = sched[2 * ti];
    it->m0 = sched[2 * ti + 1];
    int Mu;
    unit_rows(a, it->u, na, &it->p0, &Mu);
    it->M = min(rows, Mu - it->m0);
    return true;
}

// ---- gate/up ------------------------------------------------------------------------

template <int QT, int PREC, int R>
__device__ void gate_up_item(const PrefillArgs& a, int na, const Item& it, const uint8_t* base, int n0) {
    const int lane = threadIdx.x & 63, n = lane & 15;
    int arow[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int m = 16 * r + n;
        arow[r] = m < it.M ? row_token(a, it.u, na, it.p0, it.m0 + m) : -1;
    }
    const Geom& G = a.g;
    auto blk = [&](int mt, int col, int kb, const uint8_t** t, int* i) {
        int64_t tile;
        G.gu_block(n0 + col, kb, &tile, i);
        *t = base + (mt == 0 ? G.gate_tile(tile) : G.up_tile(tile));
    };
    f32x4 acc[2][R];
    tile_product<QT, PREC, R, 2>(a.x, a.x_bf16 != 0, a.d, arow, G.nb_d, blk, acc);
    // C register e of row group r: token row 16 r + 4 (lane / 16) + e, feature lane % 16
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int m = 16 * r + 4 * (lane >> 4) + e;
            if (m < it.M) {
                const int64_t idx = (int64_t)row_slot(a, it.u, na, it.p0, it.m0 + m) * a.f + n0 + n;
                const float hv = silu(acc[0][r][e]) * acc[1][r][e];
                if (PREC == MOE_PREC_BF16) ((__bf16*)a.h)[idx] = (__bf16)hv;
                else ((float*)a.h)[idx] = hv;
            }
        }
}

template <int QT, int PREC>
__global__ __launch_bounds__(256) void prefill_gate_up_kernel(PrefillArgs a) {
    const int na = *a.n_active;
    const int ngroups = (a.f + COLS - 1) / COLS;
    const int wave = threadIdx.x >> 6;
    for (int i = blockIdx.x;; i += gridDim.x) {
        Item it;
        int c0;
        if (!item_at(a, na, i, ngroups, &it, &c0)) return;
        const int n0 = c0 + 16 * wave;
        if (n0 >= a.f) continue;
        const uint8_t* base = unit_base(a, it.u, na);
        if (!base) {  // fail closed: NaN hidden rows, error word
            if ((threadIdx.x & 63) == 0) atomicOr(a.err, kErrMiss);
            for (int j = threadIdx.x & 63; j < it.M * 16; j += 64) {
                const int64_t idx = (int64_t)row_slot(a, it.u, na, it.p0, it.m0 + j / 16) * a.f + n0 + j % 16;
                if (PREC == MOE_PREC_BF16) ((uint16_t*)a.h)[idx] = 0x7FC0;
                else ((float*)a.h)[idx] = __uint_as_float(0x7FC00000u);
            }
            continue;
        }
        if constexpr (PREC == MOE_PREC_BF16) {
            if (it.big) {
                gate_up_item<QT, PREC, BIG / 16>(a, na, it, base, n0);
                continue;
            }
        }
        gate_up_item<QT, PREC, 1>(a, na, it, base, n0);
    }
}

// ---- down ---------------------------------------------------------------------------

template <int QT, int PREC, int R>
__device__ void down_item(const PrefillArgs& a, int na, const Item& it, const uint8_t* base, int r0) {
    const int lane = threadIdx.x & 63, n = lane & 15;
    int arow[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int m = 16 * r + n;
        arow[r] = m < it.M ? row_slot(a, it.u, na, it.p0, it.m0 + m) : -1;
    }
    const Geom& G = a.g;
    auto blk = [&](int, int col, int kb, const uint8_t** t, int* i) {
        int64_t tile;
        G.down_block(r0 + col, kb, &tile, i);
        *t = base + G.down_tile(tile);
    };
    f32x4 acc[1][R];
    tile_product<QT, PREC, R, 1>(a.h, PREC == MOE_PREC_BF16, a.f, arow, G.nb_f, blk, acc);
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int m = 16 * r + 4 * (lane >> 4) + e;
            if (m < it.M)
                a.part[(int64_t)row_slot(a, it.u, na, it.p0, it.m0 + m) * a.d + r0 + n] = acc[0][r][e];
        }
}

template <int QT, int PREC>
__global__ __launch_bounds__(256) void prefill_down_kernel(PrefillArgs a) {
    const int na = *a.n_active;
    const int ngroups = a.d / COLS;
    const int wave = threadIdx.x >> 6;
    for (int i = blockIdx.x;; i += gridDim.x) {
        Item it;
        int c0;
        if (!item_at(a, na, i, ngroups, &it, &c0)) return;
        const int r0 = c0 + 16 * wave;
        const uint8_t* base = unit_base(a, it.u, na);
        if (!base) {
            for (int j = threadIdx.x & 63; j < it.M * 16; j += 64)
                a.part[(int64_t)row_slot(a, it.u, na, it.p0, it.m0 + j / 16) * a.d + r0 + j % 16] =
                    __uint_as_float(0x7FC00000u);
            continue;
        }
        if constexpr (PREC == MOE_PREC_BF16) {
            if (it.big) {
                down_item<QT, PREC, BIG / 16>(a, na, it, base, r0);
                continue;
            }
        }
        down_item<QT, PREC, 1>(a, na, it, base, r0);
    }
}

// ---- combine ---------------------------------------------------------------------

__global__ __launch_bounds__(256) void prefill_combine_kernel(PrefillArgs a) {
    const int t = blockIdx.y;
    const int i4 = blockIdx.x * blockDim.x + threadIdx.x;  // output quad
    if (i4 * 4 >= a.d) return;
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < a.k; j++) {
        const int p = a.inv[t * a.k + j];
        const float w = a.topk_w[t * a.k + j];
        const float4 v = *(const float4*)(a.part + (int64_t)p * a.d + i4 * 4);
        y.x = fmaf(w, v.x, y.x); y.y = fmaf(w, v.y, y.y); y.z = fmaf(w, v.z, y.z); y.w = fmaf(w, v.w, y.w);
    }
    if (a.shared) {
        const float4 v = *(const float4*)(a.part + (int64_t)(a.T * a.k + t) * a.d + i4 * 4);
        y.x += v.x; y.y += v.y; y.z += v.z; y.w += v.w;
    }
    *(float4*)(a.y + (int64_t)t * a.d + i4 * 4) = y;
}

// Workgroups per product launch: several per CU; each loops over the items.
constexpr int kGrid = 2048;

template <int QT, int PREC>
hipError_t launch_qp(const PrefillArgs& a, int big_tiles, int small_tiles, hipStream_t s) {
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, s, a, PREC);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int bt = PREC == MOE_PREC_BF16 ? big_tiles : 0;
    const int64_t gu_items = (int64_t)(bt + small_tiles) * ((a.f + COLS - 1) / COLS);
    const int64_t dn_items = (int64_t)(bt + small_tiles) * (a.d / COLS);
    hipLaunchKernelGGL((prefill_gate_up_kernel<QT, PREC>), dim3((unsigned)std::min<int64_t>(gu_items, kGrid)),
                       dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_down_kernel<QT, PREC>), dim3((unsigned)std::min<int64_t>(dn_items, kGrid)),
                       dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_combine_kernel, dim3((a.d / 4 + 255) / 256, a.T), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

void prefill_max_tiles(int64_t T, int k, int E, bool shared, int* big_tiles, int* small_tiles) {
    const int64_t units = (T * k < E ? T * k : E) + (shared ? 1 : 0);
    const int64_t rows = T * k + (shared ? T : 0);
    *big_tiles = (int)((rows + BIG - 1) / BIG + units);
    *small_tiles = (int)((rows + SMALL - 1) / SMALL + units);
}

hipError_t launch_ffn_prefill(const PrefillArgs& a, int prec, hipStream_t s) {
    if (a.d % COLS || a.f % 16) return hipErrorInvalidValue;
    int bt, st;
    prefill_max_tiles(a.T, a.k, a.E, a.shared != nullptr, &bt, &st);
    if (a.g.qtype == MOE_Q8_0)
        return prec == MOE_PREC_BF16 ? launch_qp<MOE_Q8_0, MOE_PREC_BF16>(a, bt, st, s)
                                     : launch_qp<MOE_Q8_0, MOE_PREC_F32>(a, bt, st, s);
    return prec == MOE_PREC_BF16 ? launch_qp<MOE_Q4_0, MOE_PREC_BF16>(a, bt, st, s)
                                 : launch_qp<MOE_Q4_0, MOE_PREC_F32>(a, bt, st, s);
}

}  // namespace moe
