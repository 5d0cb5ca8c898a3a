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
constexpr int WIDE = kPrefillWide;  // tokens per wide tile
constexpr int SMALL = 16;        // tokens per small tile
constexpr int WAVES = 4;         // waves per workgroup, 16 features / rows each
constexpr int COLS = WAVES * 16; // features / output rows per workgroup item

// A tile: up to 16 or 64 rows of one bucket (or of the shared expert), as the
// schedule resolves it, so that a tile kernel reads one record before streaming.
//   slot  >= 0: the expert's pool slot; kUnmapped: not resident (fail closed);
//         kShared: the shared expert
//   first plan position of the tile's first row (routed), or its first token
//   M     rows in the tile
struct TileRec {
    int slot, first, M, pad;
};
constexpr int kUnmapped = -1, kShared = -2;

__device__ inline TileRec load_rec(const int32_t* recs, int i) {
    const int4 v = ((const int4*)recs)[i];
    return TileRec{v.x, v.y, v.z, v.w};
}

__device__ inline const uint8_t* tile_base(const PrefillArgs& a, const TileRec& t) {
    if (t.slot == kShared) return a.shared;
    return t.slot >= 0 ? a.pool + (int64_t)t.slot * a.payload_bytes : nullptr;
}

// Token and workspace row of tile row m.
__device__ inline int row_token(const PrefillArgs& a, const TileRec& t, int m) {
    return t.slot == kShared ? t.first + m : min(max(a.entries[t.first + m], 0), a.T * a.k - 1) / a.k;
}
__device__ inline int row_slot(const PrefillArgs& a, const TileRec& t, int m) {
    return t.slot == kShared ? a.T * a.k + t.first + m : t.first + m;
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

// Tile records of each size (sched_big, sched_small) and their counts (n_tiles);
// the page table is read here, once per bucket.
// The entry -> plan position inverse (for the combine) is written here too:
// the first 4 blockDim.x entries are loaded before the schedule's own chain of
// dependent loads (n_active, then offsets and experts, then the page table),
// so that their round trips overlap.
//
// The plan is an input of the C ABI, so the schedule checks it rather than
// trusting it: n_active is clamped to [0, min(E, T k)], each unit's offsets to
// [0, T k] with offsets[u] <= offsets[u + 1], and records beyond the arrays'
// capacity are dropped; any of these sets kErrBadId.  Only the plan positions
// the units cover, [0, offsets[n_active]), enter the inverse map, and
// n_tiles[2] tells the combine where that range ends, so an entry the plan
// dropped (an out-of-range expert id) or a stale word past the range never
// stands for another entry.
constexpr int kSchedInvAhead = 4;

__global__ __launch_bounds__(1024) void schedule_kernel(PrefillArgs a, int prec) {
    __shared__ int wave_tot[16];
    __shared__ int tot_b, tot_s, tot_w;
    __shared__ int s_bad, s_nvalid;
    const int n_ent = a.T * a.k;
    int ent_ahead[kSchedInvAhead];
#pragma unroll
    for (int q = 0; q < kSchedInvAhead; q++) {
        const int p = threadIdx.x + q * (int)blockDim.x;
        ent_ahead[q] = p < n_ent ? a.entries[p] : -1;
    }
    // A unit's plan words and page-table entry, read at a clamped index (the
    // plan arrays hold E units) so that the first pass's loads need not wait
    // for n_active: one level of plan loads, then one of page-table loads.
    struct UnitIn {
        int p0, p1, e, sl;
    };
    auto unit_in = [&](int u) {
        const int uc = min(u, a.E - 1);
        UnitIn r{a.offsets[uc], a.offsets[uc + 1], a.experts[uc], -1};
        if (r.e >= 0 && r.e < a.E) r.sl = a.pt[(int64_t)a.layer * a.E + r.e];
        return r;
    };
    const UnitIn first = unit_in(threadIdx.x);
    const int na_raw = *a.n_active;
    const int na = min(max(na_raw, 0), min(a.E, n_ent));
    if (threadIdx.x == 0) {
        s_bad = na != na_raw;
        s_nvalid = 0;
    }
    __syncthreads();
    const int n_units = na + (a.shared ? 1 : 0);
    int base_b = 0, base_s = 0, base_w = 0;
    for (int u0 = 0; u0 < n_units; u0 += 1024) {
        const int u = u0 + threadIdx.x;
        int tb = 0, ts = 0, tw = 0, slot = kShared, p0 = 0, M = 0;
        if (u < n_units) {
            if (u == na) {
                M = a.T;
            } else {
                const UnitIn in = u0 == 0 ? first : unit_in(u);
                p0 = min(max(in.p0, 0), n_ent);
                const int p1 = min(max(in.p1, 0), n_ent);
                if (p0 != in.p0 || p1 != in.p1 || p1 < p0) s_bad = 1;
                M = max(p1 - p0, 0);
                if (u == na - 1) s_nvalid = p1;
                slot = kUnmapped;
                if (in.e >= 0 && in.e < a.E && in.sl >= 0 && in.sl < a.n_slots) slot = in.sl;
                if (slot == kUnmapped) atomicOr(a.err, kErrMiss);
            }
            // (a call of fewer than wide_min tokens launches no 128-token tiles)
            if (prec == MOE_PREC_BF16 && M >= a.wide_min && a.T >= a.wide_min) tw = (M + WIDE - 1) / WIDE;
            else if (prec == MOE_PREC_BF16 && M >= a.gemm_min) tb = (M + BIG - 1) / BIG;
            else ts = (M + SMALL - 1) / SMALL;
        }
        const int fb = base_b + block_prefix(tb, wave_tot, &tot_b);
        const int fs = base_s + block_prefix(ts, wave_tot, &tot_s);
        const int fw = base_w + block_prefix(tw, wave_tot, &tot_w);
        for (int i = 0; i < tw; i++) {
            if (fw + i >= a.cap_wide) { s_bad = 1; break; }
            ((int4*)a.sched_wide)[fw + i] = make_int4(slot, p0 + i * WIDE, min(WIDE, M - i * WIDE), 0);
        }
        for (int i = 0; i < tb; i++) {
            if (fb + i >= a.cap_big) { s_bad = 1; break; }
            ((int4*)a.sched_big)[fb + i] = make_int4(slot, p0 + i * BIG, min(BIG, M - i * BIG), 0);
        }
        for (int i = 0; i < ts; i++) {
            if (fs + i >= a.cap_small) { s_bad = 1; break; }
            ((int4*)a.sched_small)[fs + i] = make_int4(slot, p0 + i * SMALL, min(SMALL, M - i * SMALL), 0);
        }
        base_b += tot_b;
        base_s += tot_s;
        base_w += tot_w;
        __syncthreads();
    }
    const int n_valid = s_nvalid;
    if (threadIdx.x == 0) {
        a.n_tiles[0] = min(base_b, a.cap_big);
        a.n_tiles[1] = min(base_s, a.cap_small);
        a.n_tiles[2] = n_valid;
        a.n_tiles[3] = min(base_w, a.cap_wide);
        if (s_bad) atomicOr(a.err, kErrBadId);
    }
#pragma unroll
    for (int q = 0; q < kSchedInvAhead; q++) {
        const int p = threadIdx.x + q * (int)blockDim.x;
        const int ent = ent_ahead[q];
        if (p < n_valid && ent >= 0 && ent < n_ent) a.inv[ent] = p;
    }
    for (int p = threadIdx.x + kSchedInvAhead * (int)blockDim.x; p < n_valid; p += blockDim.x) {
        const int ent = a.entries[p];
        if (ent >= 0 && ent < n_ent) a.inv[ent] = p;
    }
}

// ---- weights ------------------------------------------------------------------

// Raw buffer loads (gfx9 buffer resource word 3: untyped 32-bit data).  A load
// past the resource's size returns zeros.
constexpr int kBufWord3 = 0x00020000;
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 as_float4(uint4 v) {
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

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
    // the same block through a buffer resource: codes at voff + so, scale at vs + ss
    __device__ void load_buf(__amdgpu_buffer_rsrc_t r, int voff, int vs, int so, int ss) {
        lo = buf_load16(r, voff + q8_lo(0), so);
        hi = buf_load16(r, voff + q8_hi(0), so);
        s = __builtin_amdgcn_raw_buffer_load_b16(r, vs, ss, 0);
    }
    __device__ void zero() { lo = hi = make_uint4(0, 0, 0, 0); s = 0; }
    // Elements 8j..8j+7 as biased bytes (q + 128), 4 per word.
    __device__ void biased8(int j, uint32_t& w0, uint32_t& w1) const {
        const uint4 h = j < 2 ? lo : hi;
        w0 = ((j & 1) ? h.z : h.x) ^ 0x80808080u;
        w1 = ((j & 1) ? h.w : h.y) ^ 0x80808080u;
    }
    static constexpr float kBias = 128.f;
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
    __device__ void load_buf(__amdgpu_buffer_rsrc_t r, int voff, int vs, int so, int ss) {
        nib = buf_load16(r, voff, so);
        s = __builtin_amdgcn_raw_buffer_load_b16(r, vs, ss, 0);
    }
    __device__ void zero() { nib = make_uint4(0, 0, 0, 0); s = 0; }
    // Elements 8j..8j+7 as biased bytes (q + 8), 4 per word: low nibbles of
    // bytes 8j.. for j < 2, high nibbles of bytes 8(j - 2).. otherwise.
    __device__ void biased8(int j, uint32_t& w0, uint32_t& w1) const {
        const uint32_t a = (j & 1) ? nib.z : nib.x, b = (j & 1) ? nib.w : nib.y;
        const int sh = j < 2 ? 0 : 4;
        w0 = (a >> sh) & 0x0F0F0F0Fu;
        w1 = (b >> sh) & 0x0F0F0F0Fu;
    }
    static constexpr float kBias = 8.f;
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

// B operand of bf16 MFMA j of a block: elements 8j..8j+7, each d*q (exact in
// fp32: fma(d, q + bias, -bias d) rounds once) rounded to bf16.
template <int QT>
__device__ inline bf16x8 b_operand(const Raw<QT>& r, int j) {
    const float d = f16_bits_to_f32(r.s), o = -Raw<QT>::kBias * d;
    uint32_t w0, w1;
    r.biased8(j, w0, w1);
    auto v = [&](uint32_t w, int i) { return fmaf(d, (float)((w >> (8 * i)) & 0xFF), o); };
    const uint4 q = make_uint4(pack_bf16(v(w0, 0), v(w0, 1)), pack_bf16(v(w0, 2), v(w0, 3)),
                               pack_bf16(v(w1, 0), v(w1, 1)), pack_bf16(v(w1, 2), v(w1, 3)));
    return __builtin_bit_cast(bf16x8, q);
}

// ---- activation rows ------------------------------------------------------------
//
// The 32 values of one row in one K block, as loaded (bf16 pairs or fp32), and
// converted only when used.  Loads are unconditional (a padding row reads a
// valid row and is zeroed at conversion) so that a step's loads issue back to
// back.
template <bool XB> struct ARaw;
template <> struct ARaw<true> {
    uint4 q[4];
    __device__ void load(const void* base, int64_t pitch, int row, int c) {
        const uint4* p = (const uint4*)((const uint16_t*)base + row * pitch + c);
#pragma unroll
        for (int i = 0; i < 4; i++) q[i] = p[i];
    }
    // values 8s..8s+7 as bf16
    __device__ bf16x8 bf16(int s, bool keep) const {
        return __builtin_bit_cast(bf16x8, keep ? q[s] : make_uint4(0, 0, 0, 0));
    }
    __device__ void f32(float (&v)[32], bool keep) const {
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const uint32_t w[4] = {q[s].x, q[s].y, q[s].z, q[s].w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                v[8 * s + 2 * i] = keep ? __uint_as_float(w[i] << 16) : 0.f;
                v[8 * s + 2 * i + 1] = keep ? __uint_as_float(w[i] & 0xFFFF0000u) : 0.f;
            }
        }
    }
};
template <> struct ARaw<false> {
    float4 f[8];
    __device__ void load(const void* base, int64_t pitch, int row, int c) {
        const float4* p = (const float4*)((const float*)base + row * pitch + c);
#pragma unroll
        for (int i = 0; i < 8; i++) f[i] = p[i];
    }
    // values 8s..8s+7 rounded to bf16 (nearest even)
    __device__ bf16x8 bf16(int s, bool keep) const {
        const float4 a = f[2 * s], b = f[2 * s + 1];
        const uint4 q = make_uint4(pack_bf16(a.x, a.y), pack_bf16(a.z, a.w), pack_bf16(b.x, b.y), pack_bf16(b.z, b.w));
        return __builtin_bit_cast(bf16x8, keep ? q : make_uint4(0, 0, 0, 0));
    }
    __device__ void f32(float (&v)[32], bool keep) const {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            v[4 * i] = keep ? f[i].x : 0.f;
            v[4 * i + 1] = keep ? f[i].y : 0.f;
            v[4 * i + 2] = keep ? f[i].z : 0.f;
            v[4 * i + 3] = keep ? f[i].w : 0.f;
        }
    }
};

// ---- the tile product ------------------------------------------------------------
//
// One wave: C[16 R tokens][16 columns] for MATS weight matrices sharing the
// A operand (gate and up: 2; down: 1), over nkb K blocks.  Lane (n, g) owns
// block g of each step for column n; lane (m, g) the same block of token rows
// m, m + 16, ... (arow[r]: a valid row; alive[r]: whether it is a real one).
// blk(mat, col, kb, &tile_ptr, &lane_in_tile) locates a block.
//
// Pipelining: loads complete in order, so a step's compute waits for every load
// issued before its last operand.  With one row group, a step's weights and
// activations are both fetched one step ahead; with four (whose activations
// would need 64 more registers per buffer), the step's activations are issued
// before the next step's weights.

template <int QT, int PREC, bool XB, int R, int MATS, class BlockAt>
__device__ void tile_product(const void* A, int64_t a_pitch, const int (&arow)[R], const bool (&alive)[R], int nkb,
                             BlockAt blk, f32x4 (&acc)[MATS][R]) {
    constexpr bool AHEAD = R == 1;  // activations fetched a step ahead
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < MATS; mt++)
#pragma unroll
        for (int r = 0; r < R; r++) acc[mt][r] = f32x4{0.f, 0.f, 0.f, 0.f};
    struct Stage {
        Raw<QT> w[MATS];
        ARaw<XB> x[AHEAD ? R : 1];
    };
    // kb0 + g clamped: a fetch past the end re-reads the last block.
    auto fetch_w = [&](int kb0, Stage& st) {
        const int kb = min(kb0 + g, nkb - 1);
#pragma unroll
        for (int mt = 0; mt < MATS; mt++) {
            const uint8_t* t;
            int i;
            blk(mt, n, kb, &t, &i);
            st.w[mt].load(t, i);
        }
    };
    auto fetch_x = [&](int kb0, ARaw<XB>(&x)[R]) {
        const int c = min(kb0 + g, nkb - 1) * kQK;
#pragma unroll
        for (int r = 0; r < R; r++) x[r].load(A, a_pitch, arow[r], c);
    };
    auto compute = [&](int kb0, const Raw<QT>(&w)[MATS], const ARaw<XB>(&x)[R]) {
        const bool live = kb0 + g < nkb;
        if constexpr (PREC == MOE_PREC_BF16) {
#pragma unroll
            for (int s = 0; s < 4; s++) {
                bf16x8 b[MATS];
#pragma unroll
                for (int mt = 0; mt < MATS; mt++) b[mt] = b_operand<QT>(w[mt], s);
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const bf16x8 av = x[r].bf16(s, live && alive[r]);
#pragma unroll
                    for (int mt = 0; mt < MATS; mt++)
                        acc[mt][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[mt], acc[mt][r], 0, 0, 0);
                }
            }
        } else {
            static_assert(R == 1, "fp32 tiles are 16 tokens");
            float xv[32];
            x[0].f32(xv, live && alive[0]);
#pragma unroll
            for (int mt = 0; mt < MATS; mt++) {
                float wv[32];
                w[mt].values(wv);
#pragma unroll
                for (int j = 0; j < 32; j++)
                    acc[mt][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[j], wv[j], acc[mt][0], 0, 0, 0);
            }
        }
    };
    // One step: operands of step kb0 in cur; next step's loads into nxt.
    auto one = [&](int kb0, Stage& cur, Stage& nxt) {
        if constexpr (AHEAD) {
            fetch_w(kb0 + 4, nxt);
            fetch_x(kb0 + 4, nxt.x);
            compute(kb0, cur.w, cur.x);
        } else {
            ARaw<XB> x[R];
            fetch_x(kb0, x);
            fetch_w(kb0 + 4, nxt);
            compute(kb0, cur.w, x);
        }
    };
    // Two stages, alternating; the loop body has no exit between a fetch and
    // its use, so the compiler keeps the loads where they are issued.
    Stage sa, sb;
    fetch_w(0, sa);
    if constexpr (AHEAD) fetch_x(0, sa.x);
    const int n_steps = (nkb + 3) / 4;
    int kb0 = 0;
    for (int i = 0; i < n_steps / 2; i++, kb0 += 8) {
        one(kb0, sa, sb);
        one(kb0 + 4, sb, sa);
    }
    if (n_steps & 1) one(kb0, sa, sb);
}

// ---- the bf16 tile product: activations staged through LDS -------------------------
//
// The four waves of a workgroup share the tile's token rows, so each step's
// activation block (16 R rows x 128 columns, bf16) is loaded once per workgroup,
// 256 contiguous bytes per row, into one of two LDS buffers, and each wave reads
// its A fragments from there.  One barrier per step: the buffer written during
// step k was last read during step k - 1.  The barrier orders LDS only, so the
// next step's weight loads stay in flight across it.
//
// NW weight stages: with 2, a step's weights are fetched one step ahead; with 3,
// two steps ahead.  Loads complete in order, and each step waits for the next
// step's activations (issued after the weights of the step after it), so with
// 3 stages a weight fetch has two steps to arrive instead of one, for 9 (Q8_0)
// or 5 (Q4_0) more registers per matrix.

constexpr int APITCH = 128 + 8;  // bf16 per LDS row: 272 bytes, conflict-free 16-byte reads

// srow[q]: source row of tile row (threadIdx.x % 256) / 16 + 16 q (a valid row;
// skeep[q] false for padding rows, staged as zeros).  Waves with wlive false
// take part in the staging and barriers only.
//
// KH = 2: a workgroup of 8 waves splits K in two halves, waves w and w + 4
// taking the same 16 columns over the first and the second half (threads 256
// and up stage the second half's activations); at the end the second half's
// sums are added to the first's (first + second, a fixed order) and only
// waves 0-3 hold the result.  It doubles the waves of a launch that has few
// items, each with half the K steps.
template <int QT, bool XB, int R, int MATS, int NW, int KH, class BlockAt>
__device__ void tile_product_lds(const void* A, int64_t a_pitch, const int (&srow)[R], const bool (&skeep)[R],
                                 int nkb, bool wlive, BlockAt blk, f32x4 (&acc)[MATS][R]) {
    static_assert(KH == 1 || KH == 2, "K in one or two halves");
    __shared__ __attribute__((aligned(16))) __bf16 abuf[2][KH][16 * R][APITCH];
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    const int tt = threadIdx.x & 255, th = KH == 1 ? 0 : threadIdx.x >> 8;  // staging thread, its half
    const int wh = th;                                                       // this wave's half
    const int srow_t = tt >> 4, scol = (tt & 15) * 8;  // staging: 8 columns per thread
    // K blocks [kbeg, kend) of a half
    const int nkh = (nkb + KH - 1) / KH;
    const int kbeg_w = wh * nkh, kend_w = min(kbeg_w + nkh, nkb);
    const int kbeg_t = th * nkh, kend_t = min(kbeg_t + nkh, nkb);
#pragma unroll
    for (int mt = 0; mt < MATS; mt++)
#pragma unroll
        for (int r = 0; r < R; r++) acc[mt][r] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto fetch_w = [&](int kb0, Raw<QT>(&w)[MATS]) {
        const int kb = min(kbeg_w + kb0 + g, kend_w - 1);
#pragma unroll
        for (int mt = 0; mt < MATS; mt++) {
            const uint8_t* t;
            int i;
            blk(mt, n, kb, &t, &i);
            w[mt].load(t, i);
        }
    };
    // columns [kb0 * 32, kb0 * 32 + 128) of the half of this thread's staging
    // rows; blocks past the half (a ragged last step) are zeros
    struct AStage {
        uint4 q[R];
    };
    auto fetch_a = [&](int kb0, AStage& st) {
        const int c = (kbeg_t + kb0) * kQK + scol;
        const bool in = (kbeg_t + kb0 + scol / kQK) < kend_t;
        const int cc = in ? c : 0;
#pragma unroll
        for (int q = 0; q < R; q++) {
            uint4 v;
            if constexpr (XB) {
                v = *(const uint4*)((const uint16_t*)A + srow[q] * a_pitch + cc);
            } else {
                const float* p = (const float*)A + srow[q] * a_pitch + cc;
                const float4 f0 = *(const float4*)p, f1 = *(const float4*)(p + 4);
                v = make_uint4(pack_bf16(f0.x, f0.y), pack_bf16(f0.z, f0.w), pack_bf16(f1.x, f1.y),
                               pack_bf16(f1.z, f1.w));
            }
            st.q[q] = (skeep[q] && in) ? v : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_a = [&](int buf, const AStage& st) {
#pragma unroll
        for (int q = 0; q < R; q++) *(uint4*)&abuf[buf][th][srow_t + 16 * q][scol] = st.q[q];
    };
    auto compute = [&](int buf, const Raw<QT>(&w)[MATS]) {
#pragma unroll
        for (int s = 0; s < 4; s++) {
            bf16x8 b[MATS];
#pragma unroll
            for (int mt = 0; mt < MATS; mt++) b[mt] = b_operand<QT>(w[mt], s);
#pragma unroll
            for (int r = 0; r < R; r++) {
                const bf16x8 av = *(const bf16x8*)&abuf[buf][wh][16 * r + n][kQK * g + 8 * s];
#pragma unroll
                for (int mt = 0; mt < MATS; mt++)
                    acc[mt][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[mt], acc[mt][r], 0, 0, 0);
            }
        }
    };
    // step k: weights of k in wc, activations of k in LDS buffer k & 1; the
    // activations of k + 1 and the weights of k + NW - 1 (into wn) issued first
    auto one = [&](int kb0, int buf, Raw<QT>(&wc)[MATS], Raw<QT>(&wn)[MATS]) {
        AStage st;
        fetch_a(kb0 + 4, st);
        if (wlive) fetch_w(kb0 + 4 * (NW - 1), wn);
        if (wlive) compute(buf, wc);
        store_a(buf ^ 1, st);
        lds_barrier();
    };
    const int n_steps = (nkh + 3) / 4;
    int kb0 = 0;
    if constexpr (NW == 2) {
        Raw<QT> wa[MATS], wb[MATS];
        {
            AStage st;
            fetch_a(0, st);
            if (wlive) fetch_w(0, wa);
            store_a(0, st);
            lds_barrier();
        }
        for (int i = 0; i < n_steps / 2; i++, kb0 += 8) {
            one(kb0, 0, wa, wb);
            one(kb0 + 4, 1, wb, wa);
        }
        if (n_steps & 1) one(kb0, 0, wa, wb);
    } else {
        static_assert(NW == 3, "two or three weight stages");
        Raw<QT> wa[MATS], wb[MATS], wc[MATS];
        {
            AStage st;
            fetch_a(0, st);
            if (wlive) fetch_w(0, wa);
            if (wlive) fetch_w(4, wb);
            store_a(0, st);
            lds_barrier();
        }
        // stage of step k: wa, wb, wc for k % 3 = 0, 1, 2; LDS buffer k & 1
        int step = 0;
        for (; step + 3 <= n_steps; step += 3, kb0 += 12) {
            one(kb0, step & 1, wa, wc);
            one(kb0 + 4, (step + 1) & 1, wb, wa);
            one(kb0 + 8, step & 1, wc, wb);
        }
        if (step < n_steps) one(kb0, step & 1, wa, wc);
        if (step + 1 < n_steps) one(kb0 + 4, (step + 1) & 1, wb, wa);
    }
    if constexpr (KH == 2) {
        // the second half's sums through LDS (no wave reads the activations
        // any more after the last step's barrier), added to the first's
        float* red = (float*)&abuf[0][0][0][0];
        static_assert(sizeof(abuf) >= sizeof(float) * 4 * 64 * MATS * R * 4, "the sums fit the buffers");
        const int w4 = (threadIdx.x >> 6) & 3;
        if (wh == 1)
#pragma unroll
            for (int mt = 0; mt < MATS; mt++)
#pragma unroll
                for (int r = 0; r < R; r++)
#pragma unroll
                    for (int e = 0; e < 4; e++) red[((mt * R + r) * 4 + e) * 256 + w4 * 64 + lane] = acc[mt][r][e];
        lds_barrier();
        if (wh == 0)
#pragma unroll
            for (int mt = 0; mt < MATS; mt++)
#pragma unroll
                for (int r = 0; r < R; r++)
#pragma unroll
                    for (int e = 0; e < 4; e++) acc[mt][r][e] += red[((mt * R + r) * 4 + e) * 256 + w4 * 64 + lane];
        lds_barrier();  // (the LDS is the next item's staging)
    }
}

// ---- gate/up ------------------------------------------------------------------------

template <int QT, int PREC, bool XB, int R, int KH>
__device__ void gate_up_item(const PrefillArgs& a, const TileRec& t, const uint8_t* base, int n0, bool wlive) {
    const int lane = threadIdx.x & 63, n = lane & 15;
    const Geom& G = a.g;
    auto blk = [&](int mt, int col, int kb, const uint8_t** t, int* i) {
        int64_t tile;
        G.gu_block(n0 + col, kb, &tile, i);
        *t = base + (mt == 0 ? G.gate_tile(tile) : G.up_tile(tile));
    };
    f32x4 acc[2][R];
    if constexpr (PREC == MOE_PREC_BF16) {
        int srow[R];
        bool skeep[R];
#pragma unroll
        for (int q = 0; q < R; q++) {
            const int m = ((threadIdx.x & 255) >> 4) + 16 * q;
            skeep[q] = m < t.M;
            srow[q] = row_token(a, t, skeep[q] ? m : 0);
        }
        tile_product_lds<QT, XB, R, 2, 2, KH>(a.x, a.d, srow, skeep, G.nb_d, wlive, blk, acc);
    } else {
        int arow[R];
        bool alive[R];
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int m = 16 * r + n;
            alive[r] = m < t.M;
            arow[r] = row_token(a, t, alive[r] ? m : 0);
        }
        tile_product<QT, PREC, XB, R, 2>(a.x, a.d, arow, alive, G.nb_d, blk, acc);
    }
    if (!wlive || (KH == 2 && threadIdx.x >= 256)) return;  // (the second K half's waves hold no result)
    // C register e of row group r: token row 16 r + 4 (lane / 16) + e, feature lane % 16
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int m = 16 * r + 4 * (lane >> 4) + e;
            if (m < t.M) {
                const int64_t idx = (int64_t)row_slot(a, t, m) * a.f + n0 + n;
                const float hv = silu(acc[0][r][e]) * acc[1][r][e];
                if (PREC == MOE_PREC_BF16) ((__bf16*)a.h)[idx] = (__bf16)hv;
                else ((float*)a.h)[idx] = hv;
            }
        }
}

// BIGT: the 64-token tiles (bf16 mode), else the 16-token tiles.  Each size is
// its own launch so that the 16-token one keeps to 128 registers (the 64-token
// one to 168).  KH = 2 (64-token tiles of a call with few of them): 8 waves
// per workgroup, K in two halves (tile_product_lds).
template <int QT, int PREC, bool XB, bool BIGT, int KH>
__global__ __launch_bounds__(256 * KH, KH == 2 ? 1 : BIGT ? 3 : (PREC == MOE_PREC_BF16 ? 4 : 3)) void prefill_gate_up_kernel(PrefillArgs a) {
    static_assert(KH == 1 || (BIGT && PREC == MOE_PREC_BF16), "K halves: 64-token tiles only");
    const int ngroups = (a.f + COLS - 1) / COLS;
    const int wave = (threadIdx.x >> 6) & (WAVES - 1);
    const int n_items = a.n_tiles[BIGT ? 0 : 1] * ngroups;
    const int32_t* recs = BIGT ? a.sched_big : a.sched_small;
    for (int i = blockIdx.x; i < n_items; i += gridDim.x) {
        const TileRec t = load_rec(recs, i / ngroups);
        const int c0 = (i % ngroups) * COLS;
        // a wave past d_ff (d_ff not a multiple of COLS) still takes part in the
        // workgroup's staging, on a valid column group, and stores nothing
        const bool wlive = c0 + 16 * wave < a.f;
        const int n0 = wlive ? c0 + 16 * wave : a.f - 16;
        const uint8_t* base = tile_base(a, t);
        if (!base) {  // fail closed: NaN hidden rows (the schedule set the error word)
            if (!wlive || (KH == 2 && threadIdx.x >= 256)) continue;
            for (int j = threadIdx.x & 63; j < t.M * 16; j += 64) {
                const int64_t idx = (int64_t)row_slot(a, t, j / 16) * a.f + n0 + j % 16;
                if (PREC == MOE_PREC_BF16) ((uint16_t*)a.h)[idx] = 0x7FC0;
                else ((float*)a.h)[idx] = __uint_as_float(0x7FC00000u);
            }
            continue;
        }
        gate_up_item<QT, PREC, XB, BIGT ? BIG / 16 : 1, KH>(a, t, base, n0, wlive);
    }
}

// ---- down ---------------------------------------------------------------------------

template <int QT, int PREC, int R>
__device__ void down_item(const PrefillArgs& a, const TileRec& t, const uint8_t* base, int r0) {
    const int lane = threadIdx.x & 63, n = lane & 15;
    const Geom& G = a.g;
    auto blk = [&](int, int col, int kb, const uint8_t** t, int* i) {
        int64_t tile;
        G.down_block(r0 + col, kb, &tile, i);
        *t = base + G.down_tile(tile);
    };
    f32x4 acc[1][R];
    if constexpr (PREC == MOE_PREC_BF16) {
        int srow[R];
        bool skeep[R];
#pragma unroll
        for (int q = 0; q < R; q++) {
            const int m = (threadIdx.x >> 4) + 16 * q;
            skeep[q] = m < t.M;
            srow[q] = row_slot(a, t, skeep[q] ? m : 0);
        }
        tile_product_lds<QT, true, R, 1, 3, 1>(a.h, a.f, srow, skeep, G.nb_f, true, blk, acc);
    } else {
        int arow[R];
        bool alive[R];
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int m = 16 * r + n;
            alive[r] = m < t.M;
            arow[r] = row_slot(a, t, alive[r] ? m : 0);
        }
        tile_product<QT, PREC, false, R, 1>(a.h, a.f, arow, alive, G.nb_f, blk, acc);
    }
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int m = 16 * r + 4 * (lane >> 4) + e;
            if (m < t.M) a.part[(int64_t)row_slot(a, t, m) * a.d + r0 + n] = acc[0][r][e];
        }
}

template <int QT, int PREC, bool BIGT>
__global__ __launch_bounds__(256, BIGT ? 2 : (PREC == MOE_PREC_BF16 ? 4 : 3)) void prefill_down_kernel(PrefillArgs a) {
    const int ngroups = a.d / COLS;
    const int wave = threadIdx.x >> 6;
    const int n_items = a.n_tiles[BIGT ? 0 : 1] * ngroups;
    const int32_t* recs = BIGT ? a.sched_big : a.sched_small;
    for (int i = blockIdx.x; i < n_items; i += gridDim.x) {
        const TileRec t = load_rec(recs, i / ngroups);
        const int r0 = (i % ngroups) * COLS + 16 * wave;
        const uint8_t* base = tile_base(a, t);
        if (!base) {
            for (int j = threadIdx.x & 63; j < t.M * 16; j += 64)
                a.part[(int64_t)row_slot(a, t, j / 16) * a.d + r0 + j % 16] = __uint_as_float(0x7FC00000u);
            continue;
        }
        down_item<QT, PREC, BIGT ? BIG / 16 : 1>(a, t, base, r0);
    }
}

// ---- wide tiles: buckets of at least wide_min tokens (bf16 mode) -----------------
//
// A workgroup of 4 waves owns 128 token rows of one bucket and, per item, 64
// hidden units of gate and up (gate/up) or 128 output rows (down).  Each K step
// of 64 columns (two quant blocks per row) every thread dequantises one weight
// block into bf16 in LDS, so a weight is dequantised once per 128 tokens
// instead of once per 16 or 64; the token rows are staged in LDS beside it.
// Wave w computes rows 64 (w % 2) .. + 64 against 32 hidden units of both
// matrices (gate/up) or 64 output rows (down) with v_mfma_f32_32x32x16_bf16:
// four 32 x 32 products per 16 columns, from two A and two B fragments.
// The raw loads of a step (the thread's four 16-byte pieces of token rows and
// its weight block) are issued WST steps ahead into registers; LDS holds two
// steps (the one being multiplied and the next, written before the product).

constexpr int WFEAT = 64;             // hidden units per wide gate/up item (both matrices: 128 LDS rows)
constexpr int WROWS = 128;            // output rows per wide down item
constexpr int WBK = 64;               // K columns per step: two blocks per row
// steps of raw loads in registers: 4 with bf16 activations (244 registers),
// 3 with fp32 ones (twice the bytes per stage; 4 would spill)
template <bool AXB> constexpr int WST = AXB ? 4 : 3;
constexpr int WPITCH = WBK + 8;       // bf16 per LDS row: 144 bytes, conflict-free 16-byte reads

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct WideLds {
    __bf16 a[2][WIDE][WPITCH];
    __bf16 b[2][128][WPITCH];
};

// One thread's raw loads for one step: four 8-element pieces of token rows
// (rows (tid >> 3) + 32 i, columns 8 (tid & 7) of the step) and one weight block.
template <int QT, bool XB> struct WideRaw;
template <int QT> struct WideRaw<QT, true> {
    uint4 x[4];
    Raw<QT> w;
};
template <int QT> struct WideRaw<QT, false> {
    float4 x[8];
    Raw<QT> w;
};

// GATEUP: A = activation rows of the tile's tokens (x, bf16 or fp32 rounded to
// bf16), B = gate rows (LDS rows 0..63) and up rows (64..127) of hidden units
// c0 .. c0 + 63.  Otherwise (down): A = the tile's hidden rows (bf16), B = the
// down rows r0 .. r0 + 127.
template <int QT, bool XB, bool GATEUP>
__device__ void wide_item(const PrefillArgs& a, const TileRec& t, const uint8_t* base, int c0, WideLds& L) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const Geom& G = a.g;
    const int nk = (GATEUP ? G.nb_d : G.nb_f) / 2;  // steps
    constexpr bool AXB = GATEUP ? XB : true;         // the hidden rows are bf16
    // Loads go through buffer resources (a base and a size in scalar registers):
    // each thread keeps fixed 32-bit offsets, and a step adds one uniform
    // scalar offset, so a step's addressing costs no vector instructions.
    // A: x (gate/up; token rows) or the tile's hidden rows (down; rows
    // row_slot(0) .. + M - 1, which are consecutive).  Padding rows (m >= M)
    // read row 0 again: a product row depends only on its own A row, and the
    // epilogue drops those rows.
    constexpr int AE = AXB ? 2 : 4;  // bytes per activation element
    const int64_t a_row0 = GATEUP ? 0 : (int64_t)row_slot(a, t, 0);
    const int a_rowlen = GATEUP ? a.d : a.f;
    const uint8_t* A = GATEUP ? (const uint8_t*)a.x : (const uint8_t*)a.h + a_row0 * a.f * 2;
    const int a_bytes = GATEUP ? a.T * a.d * AE : t.M * a.f * 2;
    const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, a_bytes, kBufWord3);
    const int ach = (tid & 7) * 8;  // column of the thread's pieces within a step
    int aoff[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int m = (tid >> 3) + 32 * i;
        const int mm = m < t.M ? m : 0;
        const int row = GATEUP ? row_token(a, t, mm) : mm;
        aoff[i] = (row * a_rowlen + ach) * AE;
    }
    // this thread's weight block: LDS row brow, block kbit of each step.  Step
    // s reads column block 2 s + kbit: tile s / 2 of the row group's run of
    // tiles, lane 16 (2 (s % 2) + kbit) + brow % 16 of it.
    const int kbit = (tid >> 4) & 1;
    int brow;
    if constexpr (GATEUP) brow = (tid >> 7) * 64 + 16 * ((tid >> 5) & 3) + (tid & 15);
    else brow = 16 * (tid >> 5) + (tid & 15);
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)G.payload, kBufWord3);
    int64_t t0;  // the row group's first tile and the matrix's tile stride
    int tstride;
    if constexpr (GATEUP) {
        int li;
        G.gu_block(c0 + (brow & 63), 0, &t0, &li);
        tstride = 2 * (int)G.tile_bytes;
    } else {
        int li;
        G.down_block(c0 + brow, 0, &t0, &li);
        tstride = (int)G.tile_bytes;
    }
    const int64_t mat0 = GATEUP ? ((brow >> 6) == 0 ? G.gate_tile(t0) : G.up_tile(t0)) : G.down_tile(t0);
    const int li0 = 16 * kbit + (brow & 15);
    const int woff = (int)mat0 + (QT == MOE_Q8_0 ? q8_lo(li0) : q4_nib(li0));
    const int soff_w = (int)mat0 + (QT == MOE_Q8_0 ? q8_scale(li0) : q4_scale(li0));
    auto load = [&](WideRaw<QT, AXB>& r, int step) {
        step = min(step, nk - 1);  // past the end: the last step again (unused)
        const int sa = step * WBK * AE;
        const int sw = (step >> 1) * tstride, odd = step & 1;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if constexpr (AXB) {
                r.x[i] = buf_load16(ar, aoff[i], sa);
            } else {
                r.x[2 * i] = as_float4(buf_load16(ar, aoff[i], sa));
                r.x[2 * i + 1] = as_float4(buf_load16(ar, aoff[i] + 16, sa));
            }
        }
        // lanes 2 (s % 2) + kbit: 32 lanes further on odd steps
        r.w.load_buf(wr, woff, soff_w, sw + odd * (QT == MOE_Q8_0 ? q8_lo(32) : q4_nib(32)),
                     sw + odd * (QT == MOE_Q8_0 ? q8_scale(32) - q8_scale(0) : q4_scale(32) - q4_scale(0)));
    };
    // piece i (0..3) of a step's stores: the thread's i-th activation piece
    // and the i-th 8 weights of its block, bf16
    auto store_piece = [&](const WideRaw<QT, AXB>& r, int buf, int i) {
        uint4 v;
        if constexpr (AXB) {
            v = r.x[i];
        } else {
            const float4 f0 = r.x[2 * i], f1 = r.x[2 * i + 1];
            v = make_uint4(pack_bf16(f0.x, f0.y), pack_bf16(f0.z, f0.w), pack_bf16(f1.x, f1.y), pack_bf16(f1.z, f1.w));
        }
        *(uint4*)&L.a[buf][(tid >> 3) + 32 * i][ach] = v;
        *(bf16x8*)&L.b[buf][brow][kbit * kQK + 8 * i] = b_operand<QT>(r.w, i);
    };
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.f;
    // B rows of this wave's two 32-column groups
    const int bro0 = GATEUP ? 32 * wn : 64 * wn;
    const int bro1 = GATEUP ? 64 + 32 * wn : 64 * wn + 32;
    // the products of 16 columns (substep s) of the step in LDS buffer buf
    auto compute_sub = [&](int buf, int s) {
        const int r = lane & 31, kq = 8 * (lane >> 5);
        const bf16x8 a0 = *(const bf16x8*)&L.a[buf][64 * wm + r][16 * s + kq];
        const bf16x8 a1 = *(const bf16x8*)&L.a[buf][64 * wm + 32 + r][16 * s + kq];
        const bf16x8 b0 = *(const bf16x8*)&L.b[buf][bro0 + r][16 * s + kq];
        const bf16x8 b1 = *(const bf16x8*)&L.b[buf][bro1 + r][16 * s + kq];
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
    };
    // step k: LDS buffer k & 1 holds it; the register stage of step k + 1 is
    // written to the other buffer, a quarter beside each quarter of the
    // products (independent work the matrix cores and the vector ALU can
    // overlap), then reloaded with step k + 1 + WST
    WideRaw<QT, AXB> st[WST<AXB>];
#pragma unroll
    for (int q = 0; q < WST<AXB>; q++) load(st[q], q);
#pragma unroll
    for (int i = 0; i < 4; i++) store_piece(st[0], 0, i);
    load(st[0], WST<AXB>);
    lds_barrier();
    auto iter = [&](int k, WideRaw<QT, AXB>& r) {
        const int cur = k & 1, nxt = cur ^ 1;
#pragma unroll
        for (int s = 0; s < WBK / 16; s++) {
            compute_sub(cur, s);
            store_piece(r, nxt, s);
        }
        load(r, k + 1 + WST<AXB>);
        lds_barrier();
    };
    // step k + 1 is in register stage (k + 1) % WST<AXB>
    int k = 0;
    for (; k + WST<AXB> <= nk; k += WST<AXB>) {
#pragma unroll
        for (int q = 0; q < WST<AXB>; q++) iter(k + q, st[(q + 1) % WST<AXB>]);
    }
#pragma unroll
    for (int q = 0; q + 1 < WST<AXB>; q++)
        if (k + q < nk) iter(k + q, st[(q + 1) % WST<AXB>]);
    // C element e of product (i, j): row 64 wm + 32 i + 8 (e / 4) + 4 (lane / 32) + e % 4,
    // column lane % 32 of the j-th B row group
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int e = 0; e < 16; e++) {
            const int m = 64 * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            if (m >= t.M) continue;
            const int64_t slot = row_slot(a, t, m);
            if constexpr (GATEUP) {
                const float z = acc[i][0][e];
                const float hv = z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)) * acc[i][1][e];
                ((__bf16*)a.h)[slot * a.f + c0 + 32 * wn + (lane & 31)] = (__bf16)hv;
            } else {
                a.part[slot * a.d + c0 + 64 * wn + (lane & 31)] = acc[i][0][e];
                a.part[slot * a.d + c0 + 64 * wn + 32 + (lane & 31)] = acc[i][1][e];
            }
        }
}

// Workgroup b runs on XCD b % 8 (the dispatcher deals workgroups to the eight
// XCDs in turn), and each XCD has its own L2.  The items, tile-major (a tile's
// feature or row groups next to each other), are cut into eight contiguous
// runs, one per XCD, so that the groups of one tile, which read the same
// token rows, and the tiles of one bucket, which read the same weights, share
// an L2 instead of each XCD fetching them again.  The grid is a multiple of 8.
constexpr int kXcds = 8;

template <int QT, bool XB, bool GATEUP>
__global__ __launch_bounds__(256, 2) void prefill_wide_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) WideLds L;
    const int ngroups = GATEUP ? a.f / WFEAT : a.d / WROWS;
    const int n_items = a.n_tiles[3] * ngroups;
    const int xcd = blockIdx.x % kXcds, per_xcd = gridDim.x / kXcds;
    const int i0 = (int)((int64_t)n_items * xcd / kXcds), i1 = (int)((int64_t)n_items * (xcd + 1) / kXcds);
    for (int it = i0 + (int)blockIdx.x / kXcds; it < i1; it += per_xcd) {
        const TileRec t = load_rec(a.sched_wide, it / ngroups);
        const int c0 = (it % ngroups) * (GATEUP ? WFEAT : WROWS);
        const uint8_t* base = tile_base(a, t);
        if (!base) {  // fail closed: NaN rows (the schedule set the error word)
            const int ncol = GATEUP ? WFEAT : WROWS;
            for (int j = threadIdx.x; j < t.M * ncol; j += blockDim.x) {
                const int64_t slot = row_slot(a, t, j / ncol);
                if (GATEUP) ((uint16_t*)a.h)[slot * a.f + c0 + j % ncol] = 0x7FC0;
                else a.part[slot * a.d + c0 + j % ncol] = __uint_as_float(0x7FC00000u);
            }
            continue;
        }
        wide_item<QT, XB, GATEUP>(a, t, base, c0, L);
        // the next item's first stores into LDS wait for this one's last reads
        lds_barrier();
    }
}

// ---- combine ---------------------------------------------------------------------

// A token's entry is taken only if the inverse map leads to a plan position
// the units cover that holds that very entry; otherwise (the plan dropped it,
// or the map holds a stale word from an earlier call) the row is quiet NaN.
__global__ __launch_bounds__(256) void prefill_combine_kernel(PrefillArgs a) {
    const int t = blockIdx.y;
    const int i4 = blockIdx.x * blockDim.x + threadIdx.x;  // output quad
    if (i4 * 4 >= a.d) return;
    const int n_valid = a.n_tiles[2];
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
    bool ok = true;
    for (int j = 0; j < a.k; j++) {
        const int e = t * a.k + j;
        const int p = a.inv[e];
        const bool in = p >= 0 && p < n_valid;
        const int pc = in ? p : 0;
        const float w = a.topk_w[e];
        const float4 v = *(const float4*)(a.part + (int64_t)pc * a.d + i4 * 4);
        ok = ok && in && a.entries[pc] == e;
        y.x = fmaf(w, v.x, y.x); y.y = fmaf(w, v.y, y.y); y.z = fmaf(w, v.z, y.z); y.w = fmaf(w, v.w, y.w);
    }
    if (a.shared) {
        const float4 v = *(const float4*)(a.part + (int64_t)(a.T * a.k + t) * a.d + i4 * 4);
        y.x += v.x; y.y += v.y; y.z += v.z; y.w += v.w;
    }
    if (!ok) {
        const float q = __uint_as_float(0x7FC00000u);
        y = make_float4(q, q, q, q);
    }
    *(float4*)(a.y + (int64_t)t * a.d + i4 * 4) = y;
}

// Workgroups per product launch: several per CU; each loops over the items.
constexpr int kGrid = 2048;

// Compute units of the current device (cached per device; 256 if unknown).
int cu_count() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cus[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

template <class K>
hipError_t launch_items(K kernel, int64_t items, const PrefillArgs& a, hipStream_t s, int threads = 256) {
    if (items <= 0) return hipSuccess;
    hipLaunchKernelGGL(kernel, dim3((unsigned)std::min<int64_t>(items, kGrid)), dim3(threads), 0, s, a);
    return hipGetLastError();
}

// Wide-tile launches: a multiple of 8 workgroups (one run of items per XCD),
// at most the 512 that are resident at once (2 per CU), each looping over its
// XCD's items.
constexpr int kWideGrid = 512;

template <class K>
hipError_t launch_wide(K kernel, int64_t items, const PrefillArgs& a, hipStream_t s) {
    if (items <= 0) return hipSuccess;
    const int64_t g = std::min<int64_t>((items + kXcds - 1) / kXcds * kXcds, kWideGrid);
    hipLaunchKernelGGL(kernel, dim3((unsigned)g), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int QT, int PREC, bool XB>
hipError_t launch_qp(const PrefillArgs& a, int big_tiles, int small_tiles, int wide_tiles, const PrefillStreams& st) {
    const hipStream_t s = st.s;
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, s, a, PREC);
    hipError_t e = hipGetLastError();
    const int gf = (a.f + COLS - 1) / COLS, gd = a.d / COLS;
    constexpr bool BF = PREC == MOE_PREC_BF16;  // 64-token tiles only in bf16 mode
    if constexpr (BF) {
        // The tile sizes are independent chains (disjoint buckets: their own
        // hidden and partial rows) on two streams, so that they share the GPU
        // instead of running one after the other.  The chains expected to be
        // busy run on the caller's stream, right after the schedule; the
        // others wait for the fork on the auxiliary stream.  A chain with no
        // tiles in a call still launches: there it runs beside the busy ones.
        // Expected from the mean routed bucket, T k / min(T k, E): 128-token
        // tiles if it reaches wide_min, 64-token tiles if it reaches 64
        // tokens, else 16-token tiles.
        const int64_t rows = (int64_t)a.T * a.k, units = std::min<int64_t>(rows, a.E);
        const bool wide_main = rows >= (int64_t)a.wide_min * units;
        const bool big_main = rows >= (int64_t)BIG * units;
        const bool two = st.aux != nullptr;
        const hipStream_t sb = two ? st.aux : s;
        const hipStream_t s_wide = wide_main ? s : sb, s_big = big_main ? s : sb, s_small = big_main ? sb : s;
        if (two && e == hipSuccess) e = hipEventRecord(st.fork, s);
        if (two && e == hipSuccess) e = hipStreamWaitEvent(sb, st.fork, 0);
        if (e == hipSuccess && wide_main)
            e = launch_wide(prefill_wide_kernel<QT, XB, true>, (int64_t)wide_tiles * (a.f / WFEAT), a, s_wide);
        if (e == hipSuccess && wide_main)
            e = launch_wide(prefill_wide_kernel<QT, XB, false>, (int64_t)wide_tiles * (a.d / WROWS), a, s_wide);
        if (e == hipSuccess)
            e = launch_items(prefill_gate_up_kernel<QT, PREC, XB, false, 1>, (int64_t)small_tiles * gf, a, s_small);
        if (e == hipSuccess) e = launch_items(prefill_down_kernel<QT, PREC, false>, (int64_t)small_tiles * gd, a, s_small);
        // 64-token gate/up items in K halves when the call would have at most
        // one item per CU (so one wave per SIMD at most) otherwise, counting
        // 64-token tiles as if every routed and shared row were in one
        if (e == hipSuccess) {
            const int64_t est = ((rows + (a.shared ? a.T : 0) + BIG - 1) / BIG) * gf;
            e = est <= cu_count() ? launch_items(prefill_gate_up_kernel<QT, PREC, XB, true, 2>, (int64_t)big_tiles * gf,
                                                 a, s_big, 512)
                                  : launch_items(prefill_gate_up_kernel<QT, PREC, XB, true, 1>, (int64_t)big_tiles * gf,
                                                 a, s_big);
        }
        if (e == hipSuccess) e = launch_items(prefill_down_kernel<QT, PREC, true>, (int64_t)big_tiles * gd, a, s_big);
        if (e == hipSuccess && !wide_main)
            e = launch_wide(prefill_wide_kernel<QT, XB, true>, (int64_t)wide_tiles * (a.f / WFEAT), a, s_wide);
        if (e == hipSuccess && !wide_main)
            e = launch_wide(prefill_wide_kernel<QT, XB, false>, (int64_t)wide_tiles * (a.d / WROWS), a, s_wide);
        if (two && e == hipSuccess) e = hipEventRecord(st.join, sb);
        if (two && e == hipSuccess) e = hipStreamWaitEvent(s, st.join, 0);
    } else {
        if (e == hipSuccess) e = launch_items(prefill_gate_up_kernel<QT, PREC, XB, false, 1>, (int64_t)small_tiles * gf, a, s);
        if (e == hipSuccess) e = launch_items(prefill_down_kernel<QT, PREC, false>, (int64_t)small_tiles * gd, a, s);
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_combine_kernel, dim3((a.d / 4 + 255) / 256, a.T), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

void prefill_max_tiles(int64_t T, int k, int E, bool shared, int* big_tiles, int* small_tiles, int* wide_tiles) {
    const int64_t units = (T * k < E ? T * k : E) + (shared ? 1 : 0);
    const int64_t rows = T * k + (shared ? T : 0);
    *big_tiles = (int)((rows + BIG - 1) / BIG + units);
    *small_tiles = (int)((rows + SMALL - 1) / SMALL + units);
    *wide_tiles = (int)((rows + WIDE - 1) / WIDE + units);
}

PrefillLayout prefill_layout(int64_t T, int k, int E, int d, int f, bool bf16_hidden) {
    PrefillLayout L{};
    prefill_max_tiles(T, k, E, true, &L.cap_big, &L.cap_small, &L.cap_wide);
    auto up = [](size_t n) { return (n + 255) / 256 * 256; };
    const size_t rows = (size_t)(T * k + T);
    size_t o = 0;
    L.h = o;           o += up(rows * (size_t)f * (bf16_hidden ? 2 : 4));
    L.part = o;        o += up(rows * (size_t)d * 4);
    L.inv = o;         o += up((size_t)T * k * 4);
    L.sched_big = o;   o += up((size_t)L.cap_big * 16);
    L.sched_small = o; o += up((size_t)L.cap_small * 16);
    L.sched_wide = o;  o += up((size_t)L.cap_wide * 16);
    L.n_tiles = o;     o += 256;
    L.total = o;
    return L;
}

hipError_t launch_ffn_prefill(const PrefillArgs& a, int prec, const PrefillStreams& s) {
    if (a.d % COLS || a.f % 16) return hipErrorInvalidValue;
    int bt, st, wt;
    prefill_max_tiles(a.T, a.k, a.E, a.shared != nullptr, &bt, &st, &wt);
    // A bucket holds at most T tokens (a token picks an expert once; the shared
    // expert's bucket is all T): below wide_min no 128-token tile can exist.
    if (a.T < a.wide_min) wt = 0;
    const bool xb = a.x_bf16 != 0, bf = prec == MOE_PREC_BF16;
    if (a.g.qtype == MOE_Q8_0) {
        if (bf) return xb ? launch_qp<MOE_Q8_0, MOE_PREC_BF16, true>(a, bt, st, wt, s)
                          : launch_qp<MOE_Q8_0, MOE_PREC_BF16, false>(a, bt, st, wt, s);
        return xb ? launch_qp<MOE_Q8_0, MOE_PREC_F32, true>(a, bt, st, wt, s)
                  : launch_qp<MOE_Q8_0, MOE_PREC_F32, false>(a, bt, st, wt, s);
    }
    if (bf) return xb ? launch_qp<MOE_Q4_0, MOE_PREC_BF16, true>(a, bt, st, wt, s)
                      : launch_qp<MOE_Q4_0, MOE_PREC_BF16, false>(a, bt, st, wt, s);
    return xb ? launch_qp<MOE_Q4_0, MOE_PREC_F32, true>(a, bt, st, wt, s)
              : launch_qp<MOE_Q4_0, MOE_PREC_F32, false>(a, bt, st, wt, s);
}

}  // namespace moe
