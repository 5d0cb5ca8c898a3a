// Fused decode step of the routed experts: one launch over every expert the
// step touches — the persistent expert-major operator that consumes routed
// positions and page-table entries for several resident experts at once
// ("Nanite for Experts", §12, milestone 1; §11.5: the execution unit should be
// expert-major, not many independently orchestrated fragments).
//
// Work split (T <= 4 tokens, F32 or BF16 arithmetic):
//  * gate/up waves (the lower workgroup ids): unit u (a routed expert of the
//    plan, ascending, or the shared expert last) and a run of TPW gate/up tile
//    pairs.  Each lane loads its block of every tile with 16-byte loads (a
//    tile is 64 blocks = one 128-bit load per lane per code half, fully
//    coalesced), dequantises in registers, dots it with the lane's 32-column
//    slice of x, and the lanes of one row are summed by a fixed butterfly.
//    h = silu(g) * u is written to the workspace, then the wave bumps a
//    counter (release, agent scope).
//  * down waves (the higher ids): one 64-block tile of W_d (64/nb_f rows) for
//    every unit.  They issue their weight loads first, wait for all gate/up
//    waves (acquire), stage every h row in LDS, then accumulate each token's
//    output rows over its experts in ascending expert order, shared expert
//    last, and write y directly — no float atomics, no second pass.
// Workgroups are dispatched in id order on each XCD, so whenever a down
// workgroup is resident every gate/up workgroup of its XCD has been
// dispatched; gate/up waves never wait, so the waits always end.  The wait is
// bounded anyway (spin_limit): on expiry the error word is set and the
// affected rows are NaN.
//
// Expert weights come from slot_pool + page_table[layer, e] * payload_bytes
// ("Nanite for Experts", §5.4: device page table with sentinels); a -1 entry
// sets the error word and makes every row routed to it NaN (fail closed).
#include "device_util.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kTPW = 4;  // gate/up tile pairs per wave
constexpr int kPF = 8;   // down tiles kept in flight per wave

struct DecodeGrid {
    int n_gu_waves, n_gu_blocks, n_d_blocks, wpu;
    int gu_tiles, d_tiles, nbd, nbf, d, f, n_h_rows;
    int64_t tile_bytes, down_off;
};

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

// Dot products of the lane's block with N column slices v[n][0..32).
// PREC_F32: sum of code * v, then one multiply by the scale (the products
// d*q*v are the exact dequantised weights times v); PREC_BF16: each exact d*q
// is rounded to bf16 first.  Codes are converted one 32-bit word at a time.
template <int PREC>
__device__ inline float wq(float code, float s) { return PREC == MOE_PREC_BF16 ? round_bf16(code * s) : code; }

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

// The lane's 32 weights as the kernel multiplies them (codes for PREC_F32,
// whose scale is applied after the dot product; bf16-rounded d*q for
// PREC_BF16).  Returns the factor to apply after the dot product.
template <int QT, int PREC>
__device__ inline float tile_weights(const Tile<QT>& t, float (&w)[32]) {
    const float s = f16_bits_to_f32(t.s);
    if constexpr (QT == MOE_Q8_0) {
        const uint32_t c[8] = {t.lo.x, t.lo.y, t.lo.z, t.lo.w, t.hi.x, t.hi.y, t.hi.z, t.hi.w};
#pragma unroll
        for (int m = 0; m < 8; m++)
#pragma unroll
            for (int j = 0; j < 4; j++) w[4 * m + j] = wq<PREC>(i8(c[m], j), s);
    } else {
        const uint32_t c[4] = {t.nib.x, t.nib.y, t.nib.z, t.nib.w};
#pragma unroll
        for (int m = 0; m < 4; m++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t b = (c[m] >> (8 * j)) & 0xFF;
                w[4 * m + j] = wq<PREC>((float)((int)(b & 15) - 8), s);
                w[16 + 4 * m + j] = wq<PREC>((float)((int)(b >> 4) - 8), s);
            }
    }
    return PREC == MOE_PREC_F32 ? s : 1.0f;
}

__device__ inline float seg_sum_rt(float v, int seg) {
    for (int m = seg >> 1; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

template <int PREC>
__device__ inline void load_x(const FfnArgs& a, int d, int t, int cb, float (&xs)[32]) {
    if (a.x_bf16) {
        const uint4* p = (const uint4*)((const uint16_t*)a.x + (int64_t)t * d + cb * kQK);
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const uint4 v = p[m];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                xs[8 * m + 2 * j] = bf16_bits_to_f32(w[j] & 0xFFFF);
                xs[8 * m + 2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
            }
        }
    } else {
        const float4* p = (const float4*)((const float*)a.x + (int64_t)t * d + cb * kQK);
#pragma unroll
        for (int m = 0; m < 8; m++) {
            const float4 v = p[m];
            xs[4 * m] = v.x; xs[4 * m + 1] = v.y; xs[4 * m + 2] = v.z; xs[4 * m + 3] = v.w;
        }
        if (PREC == MOE_PREC_BF16) {
#pragma unroll
            for (int j = 0; j < 32; j++) xs[j] = round_bf16(xs[j]);
        }
    }
}

__device__ inline const uint8_t* unit_base(const FfnArgs& a, int u, int na) {
    if (u == na) return a.shared;
    const int e = a.experts[u];
    if (e < 0 || e >= a.E) return nullptr;
    const int s = a.pt[(int64_t)a.layer * a.E + e];
    if (s < 0 || s >= a.n_slots) return nullptr;
    return a.pool + (int64_t)s * a.payload_bytes;
}

template <int QT, int PREC, int TG>
__device__ void gate_up_wave(const FfnArgs& a, const DecodeGrid& g, int u, int part, int na, int lane) {
    const uint8_t* base = unit_base(a, u, na);
    if (!base && lane == 0) atomicOr(a.err, kErrMiss);
    const bool routed = u < na;
    const int b0 = routed ? a.offsets[u] : 0;
    const int b1 = routed ? a.offsets[u + 1] : a.T;
    const int tile0 = part * kTPW;
    const int nt = min(kTPW, g.gu_tiles - tile0);

    Tile<QT> tg[kTPW], tu[kTPW];
#pragma unroll
    for (int q = 0; q < kTPW; q++) {
        if (q < nt && base) {
            tg[q].load(base + 2 * (int64_t)(tile0 + q) * g.tile_bytes, lane);
            tu[q].load(base + (2 * (int64_t)(tile0 + q) + 1) * g.tile_bytes, lane);
        } else {
            tg[q].clear();
            tu[q].clear();
        }
    }
    const int cb = lane & (g.nbd - 1);     // column block of this lane within its row
    const bool writer = cb == 0;
    const float qnan = __uint_as_float(0x7FC00000u);

    // a bucket holds at most T <= TG tokens: one pass covers it
    float xs[TG][32];
    int hrow[TG];
#pragma unroll
    for (int gi = 0; gi < TG; gi++) {
        const int p = b0 + gi;
        if (p < b1) {
            const int t = routed ? a.entries[p] / a.k : p;
            hrow[gi] = routed ? p : a.T * a.k + p;
            load_x<PREC>(a, g.d, t, cb, xs[gi]);
        } else {
            hrow[gi] = -1;
#pragma unroll
            for (int j = 0; j < 32; j++) xs[gi][j] = 0.f;
        }
    }
#pragma unroll
    for (int q = 0; q < kTPW; q++) {
        if (q >= nt) break;
        const int row = ((tile0 + q) * kTileBlocks + lane) / g.nbd;
        float accg[TG], accu[TG];
        tile_dots<QT, PREC, TG>(tg[q], xs, accg);
        tile_dots<QT, PREC, TG>(tu[q], xs, accu);
#pragma unroll
        for (int gi = 0; gi < TG; gi++) {
            const float gs = seg_sum_rt(accg[gi], g.nbd);
            const float us = seg_sum_rt(accu[gi], g.nbd);
            if (writer && hrow[gi] >= 0) {
                float hv = silu(gs) * us;
                if (PREC == MOE_PREC_BF16) hv = round_bf16(hv);
                a.h[(int64_t)hrow[gi] * g.f + row] = base ? hv : qnan;
            }
        }
    }
}

template <int QT, int PREC>
__device__ void down_block(const FfnArgs& a, const DecodeGrid& g, int na, int n_units, int lane, int wave,
                           float* hlds) {
    __shared__ int s_timeout;
    const int dt = (blockIdx.x - g.n_gu_blocks) * 4 + wave;
    const bool active = dt < g.d_tiles;
    const int cb = lane & (g.nbf - 1);
    const int row = active ? (dt * kTileBlocks + lane) / g.nbf : 0;
    const int64_t toff = g.down_off + (int64_t)dt * g.tile_bytes;

    // 1. weight loads first: they do not depend on h
    Tile<QT> tl[kPF];
    bool ok[kPF];
#pragma unroll
    for (int p = 0; p < kPF; p++) {
        const uint8_t* b = (active && p < n_units) ? unit_base(a, p, na) : nullptr;
        ok[p] = b != nullptr;
        if (b) tl[p].load(b + toff, lane); else tl[p].clear();
    }
    // 2. wait for every gate/up wave
    if (threadIdx.x == 0) {
        s_timeout = 0;
        int it = 0;
        while (__hip_atomic_load(&a.sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
               (unsigned)g.n_gu_waves) {
            if (++it > a.spin_limit) {
                atomicOr(a.err, kErrTimeout);
                s_timeout = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // 3. stage all hidden states
    const int nh = g.n_h_rows * g.f;
    for (int i = threadIdx.x * 4; i < nh; i += blockDim.x * 4)
        *(float4*)(hlds + i) = *(const float4*)(a.h + i);
    __syncthreads();

    if (active) {
        const float qnan = __uint_as_float(0x7FC00000u);
        float acc[kDecodeMaxT];
#pragma unroll
        for (int t = 0; t < kDecodeMaxT; t++) acc[t] = 0.f;
        for (int u0 = 0; u0 < n_units; u0 += kPF) {
#pragma unroll
            for (int p = 0; p < kPF; p++) {
                const int u = u0 + p;
                if (u >= n_units) break;
                const bool okp = ok[p];
                float wf[32];
                const float post = tile_weights<QT, PREC>(tl[p], wf);
                const bool routed = u < na;
                const int b0 = routed ? a.offsets[u] : 0;
                const int b1 = routed ? a.offsets[u + 1] : a.T;
                for (int q = b0; q < b1; q++) {
                    int t, hr;
                    float rw;
                    if (routed) {
                        const int ent = a.entries[q];
                        t = ent / a.k;
                        rw = a.topk_w[ent];
                        hr = q;
                    } else {
                        t = q;
                        rw = 1.0f;
                        hr = a.T * a.k + q;
                    }
                    const float4* h4 = (const float4*)(hlds + hr * g.f + cb * kQK);
                    float dot = 0.f;
#pragma unroll
                    for (int m = 0; m < 8; m++) {
                        const float4 v = h4[m];
                        dot = fmaf(wf[4 * m], v.x, dot);
                        dot = fmaf(wf[4 * m + 1], v.y, dot);
                        dot = fmaf(wf[4 * m + 2], v.z, dot);
                        dot = fmaf(wf[4 * m + 3], v.w, dot);
                    }
                    dot = seg_sum_rt(dot * post, g.nbf);
                    if (!okp) dot = qnan;
#pragma unroll
                    for (int tt = 0; tt < kDecodeMaxT; tt++)
                        if (tt == t) acc[tt] = fmaf(rw, dot, acc[tt]);
                }
                // refill this register slot with the unit kPF ahead
                const int un = u + kPF;
                if (un < n_units) {
                    const uint8_t* b = unit_base(a, un, na);
                    ok[p] = b != nullptr;
                    if (b) tl[p].load(b + toff, lane); else tl[p].clear();
                }
            }
        }
        if (cb == 0) {
            const bool bad = s_timeout != 0;
#pragma unroll
            for (int t = 0; t < kDecodeMaxT; t++)
                if (t < a.T) a.y[(int64_t)t * g.d + row] = bad ? qnan : acc[t];
        }
    }
    // 4. the last down workgroup re-arms the counters for the next launch
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(&a.sync[1], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == (unsigned)g.n_d_blocks - 1) {
            __hip_atomic_store(&a.sync[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.sync[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int QT, int PREC, int TG>
__global__ __launch_bounds__(256) void ffn_decode_kernel(FfnArgs a, DecodeGrid g) {
    extern __shared__ float hlds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int na = *a.n_active;
    const int n_units = na + (a.shared ? 1 : 0);
    if ((int)blockIdx.x < g.n_gu_blocks) {
        const int gw = blockIdx.x * 4 + wave;
        if (gw >= g.n_gu_waves) return;
        const int u = gw / g.wpu, part = gw - u * g.wpu;
        if (u < n_units) gate_up_wave<QT, PREC, TG>(a, g, u, part, na, lane);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        if (lane == 0) __hip_atomic_fetch_add(&a.sync[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    down_block<QT, PREC>(a, g, na, n_units, lane, wave, hlds);
}

template <int QT, int PREC, int TG>
hipError_t launch_t(const DecodeGrid& dg, const FfnArgs& a, size_t lds, hipStream_t s) {
    auto kern = ffn_decode_kernel<QT, PREC, TG>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kern, dim3(dg.n_gu_blocks + dg.n_d_blocks), dim3(256), lds, s, a, dg);
    return hipGetLastError();
}

template <int QT, int PREC>
hipError_t launch_tg(const DecodeGrid& dg, const FfnArgs& a, size_t lds, hipStream_t s) {
    if (a.T <= 1) return launch_t<QT, PREC, 1>(dg, a, lds, s);
    if (a.T <= 2) return launch_t<QT, PREC, 2>(dg, a, lds, s);
    return launch_t<QT, PREC, 4>(dg, a, lds, s);
}

}  // namespace

hipError_t launch_ffn_decode(const Geom& g, const FfnArgs& a, int prec, hipStream_t s) {
    DecodeGrid dg{};
    const int units_max = min(a.T * a.k, a.E) + (a.shared ? 1 : 0);
    dg.gu_tiles = (int)g.gu_tiles;
    dg.d_tiles = (int)g.d_tiles;
    dg.wpu = (dg.gu_tiles + kTPW - 1) / kTPW;
    dg.n_gu_waves = units_max * dg.wpu;
    dg.n_gu_blocks = (dg.n_gu_waves + 3) / 4;
    dg.n_d_blocks = (dg.d_tiles + 3) / 4;
    dg.nbd = g.nb_d;
    dg.nbf = g.nb_f;
    dg.d = g.d;
    dg.f = g.f;
    dg.n_h_rows = a.T * a.k + (a.shared ? a.T : 0);
    dg.tile_bytes = g.tile_bytes;
    dg.down_off = 2 * g.gu_tiles * g.tile_bytes;
    const size_t lds = (size_t)dg.n_h_rows * g.f * sizeof(float);
    if (g.qtype == MOE_Q8_0)
        return prec == MOE_PREC_BF16 ? launch_tg<MOE_Q8_0, MOE_PREC_BF16>(dg, a, lds, s)
                                     : launch_tg<MOE_Q8_0, MOE_PREC_F32>(dg, a, lds, s);
    return prec == MOE_PREC_BF16 ? launch_tg<MOE_Q4_0, MOE_PREC_BF16>(dg, a, lds, s)
                                 : launch_tg<MOE_Q4_0, MOE_PREC_F32>(dg, a, lds, s);
}

}  // namespace moe
