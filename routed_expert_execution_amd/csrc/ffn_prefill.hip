// Routed experts for a chunk of T > 4 tokens (prefill): per bucket, the gate/up
// and down products as tile GEMMs.  Buckets of at least gemm_min tokens run on
// the bf16 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation), the
// others on an FMA dot over the same staged tiles with the same roundings, so
// one call has one numerics.  The expert union ("Nanite for Experts", §5.3)
// lets every weight tile be read once per 64 tokens of its bucket.
//
//   schedule  one workgroup: every bucket (and the shared expert over all T
//             tokens) is cut into m-tiles of 64 rows; the inverse of the plan's
//             entries is written for the combine
//   gate/up   one workgroup per (m-tile, 64 features): K loop over d_model in
//             steps of 64; weights dequantised into LDS (bf16 in bf16 mode),
//             x rows gathered by token id; h = silu(g) * u (rounded to bf16 in
//             bf16 mode) to a workspace row per (bucket entry)
//   down      one workgroup per (m-tile, 64 output rows): K loop over d_ff in
//             column blocks of 32 — one down tile each (the tile layout stores
//             a column block's d_model rows contiguously); partial rows to the
//             workspace
//   combine   y[t] = sum_j w[t,j] * partial(t,j) + shared partial(t), in rank
//             order j, shared last: fixed, slot-independent.
#include "device_util.h"
#include "internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = kPrefillBM;  // tokens per m-tile
constexpr int BN = 64;          // features (gate/up) or output rows (down) per tile
constexpr int BKG = 64;         // K step of the gate/up product (2 blocks)
constexpr int BKD = 32;         // K step of the down product (1 block)
constexpr int PADG = BKG + 8;   // LDS row pitch in elements (bank spread)
constexpr int PADD = BKD + 8;

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

__global__ __launch_bounds__(1024) void schedule_kernel(PrefillArgs a) {
    __shared__ int wave_tot[16];
    __shared__ int total;
    const int na = *a.n_active;
    const int n_units = na + (a.shared ? 1 : 0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int base = 0;
    for (int u0 = 0; u0 < n_units; u0 += 1024) {
        const int u = u0 + threadIdx.x;
        int tiles = 0;
        if (u < n_units) {
            int p0, M;
            unit_rows(a, u, na, &p0, &M);
            tiles = (M + BM - 1) / BM;
        }
        int incl = tiles;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int n = __shfl_up(incl, o, 64);
            if (lane >= o) incl += n;
        }
        if (lane == 63) wave_tot[wave] = incl;
        __syncthreads();
        if (threadIdx.x == 0) {
            int s = 0;
            for (int w = 0; w < 16; w++) { const int v = wave_tot[w]; wave_tot[w] = s; s += v; }
            total = s;
        }
        __syncthreads();
        const int first = base + wave_tot[wave] + incl - tiles;
        for (int i = 0; i < tiles; i++) {
            a.sched[2 * (first + i)] = u;
            a.sched[2 * (first + i) + 1] = i * BM;
        }
        base += total;
        __syncthreads();
    }
    if (threadIdx.x == 0) *a.n_tiles = base;
    const int n_ent = a.T * a.k;
    for (int p = threadIdx.x; p < n_ent; p += blockDim.x) {
        const int ent = a.entries[p];
        if (ent >= 0 && ent < n_ent) a.inv[ent] = p;
    }
}

// 32 weights of one block as the product multiplies them: PREC_F32 exact d*q,
// PREC_BF16 rounded to bf16.
template <int QT, int PREC>
__device__ inline void block_values(const uint8_t* tile, int i, float (&w)[32]) {
    if constexpr (QT == MOE_Q8_0) {
        const float s = f16_bits_to_f32(*(const uint16_t*)(tile + q8_scale(i)));
        const uint4 lo = *(const uint4*)(tile + q8_lo(i));
        const uint4 hi = *(const uint4*)(tile + q8_hi(i));
        const uint32_t c[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int m = 0; m < 8; m++)
#pragma unroll
            for (int j = 0; j < 4; j++) w[4 * m + j] = i8(c[m], j) * s;
    } else {
        const float s = f16_bits_to_f32(*(const uint16_t*)(tile + q4_scale(i)));
        const uint4 nb = *(const uint4*)(tile + q4_nib(i));
        const uint32_t c[4] = {nb.x, nb.y, nb.z, nb.w};
#pragma unroll
        for (int m = 0; m < 4; m++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t b = (c[m] >> (8 * j)) & 0xFF;
                w[4 * m + j] = (float)((int)(b & 15) - 8) * s;
                w[16 + 4 * m + j] = (float)((int)(b >> 4) - 8) * s;
            }
    }
    if (PREC == MOE_PREC_BF16) {
#pragma unroll
        for (int j = 0; j < 32; j++) w[j] = round_bf16(w[j]);
    }
}

// LDS tile element: bf16 for the matrix-core path, float for the FMA path.
template <bool MFMA> struct Elt { typedef float T; };
template <> struct Elt<true> { typedef __bf16 T; };

template <bool MFMA>
__device__ inline void put(typename Elt<MFMA>::T* p, float v) { *p = (typename Elt<MFMA>::T)v; }

__device__ inline float x_value(const PrefillArgs& a, int t, int k) {
    return a.x_bf16 ? bf16_bits_to_f32(((const uint16_t*)a.x)[(int64_t)t * a.d + k])
                    : ((const float*)a.x)[(int64_t)t * a.d + k];
}

// ---- gate/up ------------------------------------------------------------

template <int QT, int PREC, bool MFMA>
__device__ void gate_up_tile(const PrefillArgs& a, const uint8_t* base, int u, int na, int p0, int m0, int M,
                             int n0, char* smem) {
    typedef typename Elt<MFMA>::T E;
    E* As = (E*)smem;            // [BM][PADG]
    E* Gs = As + BM * PADG;      // [BN][PADG]
    E* Us = Gs + BN * PADG;      // [BN][PADG]
    __shared__ int s_tok[BM];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < BM) s_tok[tid] = tid < M ? row_token(a, u, na, p0, m0 + tid) : -1;
    __syncthreads();

    // accumulators: MFMA: wave quadrant 32x32 of gate and up; FMA: (feature, 4 token lanes)
    f32x16 cg = {}, cu = {};
    float fg[BM / 4], fu[BM / 4];
    if constexpr (!MFMA) {
#pragma unroll
        for (int j = 0; j < BM / 4; j++) fg[j] = fu[j] = 0.f;
    }
    for (int k0 = 0; k0 < a.d; k0 += BKG) {
        // weights: 64 features x 2 blocks x {gate, up} = 256 blocks, one per thread
        {
            const int n = tid & 63, b = (tid >> 6) & 1, mat = tid >> 7;
            int64_t t;
            int i;
            a.g.gu_block(n0 + n, k0 / kQK + b, &t, &i);
            const uint8_t* tile = base + (mat == 0 ? a.g.gate_tile(t) : a.g.up_tile(t));
            float w[32];
            block_values<QT, PREC>(tile, i, w);
            E* dst = (mat == 0 ? Gs : Us) + n * PADG + b * kQK;
#pragma unroll
            for (int j = 0; j < 32; j++) put<MFMA>(dst + j, w[j]);
        }
        // activations: BM rows x 64 columns, 16 per thread (zero rows beyond M)
        {
            const int m = tid >> 2, c0 = (tid & 3) * 16;
            const int t = s_tok[m];
            E* dst = As + m * PADG + c0;
#pragma unroll
            for (int j = 0; j < 16; j++) {
                float v = t >= 0 ? x_value(a, t, k0 + c0 + j) : 0.f;
                if (PREC == MOE_PREC_BF16) v = round_bf16(v);
                put<MFMA>(dst + j, v);
            }
        }
        __syncthreads();
        if constexpr (MFMA) {
            const int r0 = (wave >> 1) * 32, c0 = (wave & 1) * 32;
#pragma unroll
            for (int kk = 0; kk < BKG; kk += 16) {
                const int ko = kk + 8 * (lane >> 5);
                const bf16x8 av = *(const bf16x8*)(As + (r0 + (lane & 31)) * PADG + ko);
                const bf16x8 gv = *(const bf16x8*)(Gs + (c0 + (lane & 31)) * PADG + ko);
                const bf16x8 uv = *(const bf16x8*)(Us + (c0 + (lane & 31)) * PADG + ko);
                cg = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, gv, cg, 0, 0, 0);
                cu = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, uv, cu, 0, 0, 0);
            }
        } else {
            const int n = tid & 63, tl = tid >> 6;
            for (int kk = 0; kk < BKG; kk++) {
                const float gw = Gs[n * PADG + kk], uw = Us[n * PADG + kk];
#pragma unroll
                for (int j = 0; j < BM / 4; j++) {
                    const int m = tl + 4 * j;
                    if (m < M) {
                        const float xv = As[m * PADG + kk];
                        fg[j] = fmaf(gw, xv, fg[j]);
                        fu[j] = fmaf(uw, xv, fu[j]);
                    }
                }
            }
        }
        __syncthreads();
    }
    const float qnan = __uint_as_float(0x7FC00000u);
    auto emit = [&](int m, int n, float g, float uu) {
        if (m >= M) return;
        float h = silu(g) * uu;
        if (PREC == MOE_PREC_BF16) h = round_bf16(h);
        a.h[(int64_t)row_slot(a, u, na, p0, m0 + m) * a.f + n0 + n] = base ? h : qnan;
    };
    if constexpr (MFMA) {
        const int r0 = (wave >> 1) * 32, c0 = (wave & 1) * 32;
#pragma unroll
        for (int r = 0; r < 16; r++)
            emit(r0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), c0 + (lane & 31), cg[r], cu[r]);
    } else {
        const int n = tid & 63, tl = tid >> 6;
#pragma unroll
        for (int j = 0; j < BM / 4; j++) emit(tl + 4 * j, n, fg[j], fu[j]);
    }
}

template <int QT, int PREC>
__global__ __launch_bounds__(256) void prefill_gate_up_kernel(PrefillArgs a) {
    extern __shared__ char smem[];
    if ((int)blockIdx.x >= *a.n_tiles) return;
    const int u = a.sched[2 * blockIdx.x], m0 = a.sched[2 * blockIdx.x + 1];
    const int na = *a.n_active;
    int p0, Mu;
    unit_rows(a, u, na, &p0, &Mu);
    const int M = min(BM, Mu - m0);
    const int n0 = blockIdx.y * BN;
    const uint8_t* base = unit_base(a, u, na);
    if (!base) {
        if (threadIdx.x == 0) atomicOr(a.err, kErrMiss);
        const float qnan = __uint_as_float(0x7FC00000u);
        for (int i = threadIdx.x; i < M * BN; i += blockDim.x)
            a.h[(int64_t)row_slot(a, u, na, p0, m0 + i / BN) * a.f + n0 + i % BN] = qnan;
        return;
    }
    if (PREC == MOE_PREC_BF16 && Mu >= a.gemm_min)
        gate_up_tile<QT, PREC, true>(a, base, u, na, p0, m0, M, n0, smem);
    else
        gate_up_tile<QT, PREC, false>(a, base, u, na, p0, m0, M, n0, smem);
}

// ---- down ---------------------------------------------------------------

template <int QT, int PREC, bool MFMA>
__device__ void down_tile_work(const PrefillArgs& a, const uint8_t* base, int u, int na, int p0, int m0, int M,
                               int n0, char* smem) {
    typedef typename Elt<MFMA>::T E;
    E* As = (E*)smem;        // [BM][PADD]  hidden rows
    E* Ws = As + BM * PADD;  // [BN][PADD]  down weights
    __shared__ int s_row[BM];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < BM) s_row[tid] = tid < M ? row_slot(a, u, na, p0, m0 + tid) : -1;
    __syncthreads();
    f32x16 cy = {};
    float fy[BM / 4];
    if constexpr (!MFMA) {
#pragma unroll
        for (int j = 0; j < BM / 4; j++) fy[j] = 0.f;
    }
    const int dt_per_col = a.d / kTileBlocks;
    for (int kb = 0; kb < a.f / kQK; kb++) {
        // down tile of column block kb, rows n0..n0+63: 64 blocks, 4 threads each
        {
            const int n = tid >> 2, part = tid & 3;
            const uint8_t* tile = base + a.g.down_tile((int64_t)kb * dt_per_col + n0 / kTileBlocks);
            float w[32];
            block_values<QT, PREC>(tile, n, w);  // lane index = row within the tile
            E* dst = Ws + n * PADD;
#pragma unroll
            for (int j = 0; j < 8; j++) put<MFMA>(dst + part * 8 + j, w[part * 8 + j]);
        }
        // hidden rows: BM x 32, 8 per thread
        {
            const int m = tid >> 2, c0 = (tid & 3) * 8;
            const int r = s_row[m];
            E* dst = As + m * PADD + c0;
#pragma unroll
            for (int j = 0; j < 8; j++) put<MFMA>(dst + j, r >= 0 ? a.h[(int64_t)r * a.f + kb * kQK + c0 + j] : 0.f);
        }
        __syncthreads();
        if constexpr (MFMA) {
            const int r0 = (wave >> 1) * 32, c0 = (wave & 1) * 32;
#pragma unroll
            for (int kk = 0; kk < BKD; kk += 16) {
                const int ko = kk + 8 * (lane >> 5);
                const bf16x8 av = *(const bf16x8*)(As + (r0 + (lane & 31)) * PADD + ko);
                const bf16x8 wv = *(const bf16x8*)(Ws + (c0 + (lane & 31)) * PADD + ko);
                cy = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, wv, cy, 0, 0, 0);
            }
        } else {
            const int n = tid & 63, tl = tid >> 6;
            for (int kk = 0; kk < BKD; kk++) {
                const float wv = Ws[n * PADD + kk];
#pragma unroll
                for (int j = 0; j < BM / 4; j++) {
                    const int m = tl + 4 * j;
                    if (m < M) fy[j] = fmaf(wv, As[m * PADD + kk], fy[j]);
                }
            }
        }
        __syncthreads();
    }
    auto emit = [&](int m, int n, float v) {
        if (m < M) a.part[(int64_t)s_row[m] * a.d + n0 + n] = v;
    };
    if constexpr (MFMA) {
        const int r0 = (wave >> 1) * 32, c0 = (wave & 1) * 32;
#pragma unroll
        for (int r = 0; r < 16; r++) emit(r0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), c0 + (lane & 31), cy[r]);
    } else {
        const int n = tid & 63, tl = tid >> 6;
#pragma unroll
        for (int j = 0; j < BM / 4; j++) emit(tl + 4 * j, n, fy[j]);
    }
}

template <int QT, int PREC>
__global__ __launch_bounds__(256) void prefill_down_kernel(PrefillArgs a) {
    extern __shared__ char smem[];
    if ((int)blockIdx.x >= *a.n_tiles) return;
    const int u = a.sched[2 * blockIdx.x], m0 = a.sched[2 * blockIdx.x + 1];
    const int na = *a.n_active;
    int p0, Mu;
    unit_rows(a, u, na, &p0, &Mu);
    const int M = min(BM, Mu - m0);
    const int n0 = blockIdx.y * BN;
    const uint8_t* base = unit_base(a, u, na);
    if (!base) {
        const float qnan = __uint_as_float(0x7FC00000u);
        for (int i = threadIdx.x; i < M * BN; i += blockDim.x)
            a.part[(int64_t)row_slot(a, u, na, p0, m0 + i / BN) * a.d + n0 + i % BN] = qnan;
        return;
    }
    if (PREC == MOE_PREC_BF16 && Mu >= a.gemm_min)
        down_tile_work<QT, PREC, true>(a, base, u, na, p0, m0, M, n0, smem);
    else
        down_tile_work<QT, PREC, false>(a, base, u, na, p0, m0, M, n0, smem);
}

// ---- combine --------------------------------------------------------------

__global__ __launch_bounds__(256) void prefill_combine_kernel(PrefillArgs a) {
    const int t = blockIdx.y;
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= a.d) return;
    float y = 0.f;
    for (int j = 0; j < a.k; j++) {
        const int p = a.inv[t * a.k + j];
        y = fmaf(a.topk_w[t * a.k + j], a.part[(int64_t)p * a.d + i], y);
    }
    if (a.shared) y += a.part[(int64_t)(a.T * a.k + t) * a.d + i];
    a.y[(int64_t)t * a.d + i] = y;
}

template <int QT, int PREC>
hipError_t launch_qp(const PrefillArgs& a, int max_tiles, hipStream_t s) {
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(1024), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds_gu = (size_t)(BM + 2 * BN) * PADG * sizeof(float);
    const size_t lds_d = (size_t)(BM + BN) * PADD * sizeof(float);
    hipLaunchKernelGGL((prefill_gate_up_kernel<QT, PREC>), dim3(max_tiles, a.f / BN), dim3(256), lds_gu, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_down_kernel<QT, PREC>), dim3(max_tiles, a.d / BN), dim3(256), lds_d, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_combine_kernel, dim3((a.d + 255) / 256, a.T), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int prefill_max_tiles(int64_t T, int k, int E, bool shared) {
    const int64_t units = T * k < E ? T * k : E;
    return (int)((T * k + BM - 1) / BM + units + (shared ? (T + BM - 1) / BM : 0));
}

hipError_t launch_ffn_prefill(const PrefillArgs& a, int prec, hipStream_t s) {
    if (a.f % BN || a.d % BN) return hipErrorInvalidValue;
    const int max_tiles = prefill_max_tiles(a.T, a.k, a.E, a.shared != nullptr);
    if (a.g.qtype == MOE_Q8_0)
        return prec == MOE_PREC_BF16 ? launch_qp<MOE_Q8_0, MOE_PREC_BF16>(a, max_tiles, s)
                                     : launch_qp<MOE_Q8_0, MOE_PREC_F32>(a, max_tiles, s);
    return prec == MOE_PREC_BF16 ? launch_qp<MOE_Q4_0, MOE_PREC_BF16>(a, max_tiles, s)
                                 : launch_qp<MOE_Q4_0, MOE_PREC_F32>(a, max_tiles, s);
}

}  // namespace moe
