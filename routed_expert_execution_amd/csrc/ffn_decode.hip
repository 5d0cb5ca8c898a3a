// Decode step of the routed experts (T <= 4 tokens) in ONE launch: every
// expert of the step and the weighted merge into the tokens' rows -- the
// expert-major operator that consumes routed positions and page-table entries
// for several resident experts at once ("Nanite for Experts", §12, milestone
// 1; §11.5: one expert-major unit of execution rather than many separately
// orchestrated fragments; §5.5: results merged into the original positions).
// The launch can also route the step itself (moe_route_ffn).
//
// A unit is a routed expert of the plan (ascending expert id) or the shared
// expert (last).  A hidden row is one (unit, token) pair: row q < T*k is plan
// position q, row T*k + t is the shared expert on token t.  The launch has two
// kinds of workgroups:
//
//   gate/up workgroups, as many as stay resident beside the down ones, each
//     working through items (a unit and 16 or 32 hidden units; the shared
//     expert's items first): the item's rows of W_g and W_u dequantised in
//     registers against the bucket's activations (LDS); h = silu(W_g x) *
//     (W_u x) for each token of the bucket, stored to the hidden-row
//     workspace.  Nothing waits for the stores.
//   down workgroup R, one per 16 output rows: reads the page-table row and the
//     plan, issues the loads of its 16 rows of every unit's W_d (d_ff/128
//     contiguous tiles per unit), then polls the hidden rows it needs until
//     every value has been written, stages them in LDS, and sums
//     y[t, rows] = sum over t's hidden rows of w * (W_d[rows] h)
//     in one fixed order that depends only on expert ids and ranks, never on
//     slots: per lane over its tiles in order, then the four lanes of a row,
//     then the waves.  Steps of three or four tokens give each 16 output rows
//     two down workgroups, the first taking the first units in plan order and
//     the second the rest; the second adds the first's sums (handed over like
//     the hidden rows), then its own.
//
// A launch that routes takes the caller's logits, or computes them: router
// workgroups, the first in dispatch order, compute one router row per wave and
// store it with device scope into the workspace, then exit.  Every other
// workgroup then reads the logits (polling until none is pending), selects
// each token's top-k and forms the union itself, with the same code as the
// route kernels; down workgroup 0 also writes ids, weights and plan out.  The
// shared expert's items start before the routing is known.  No workgroup ever
// waits for one of higher index, so the launch needs no co-residency.
//
// Every weight byte of the step is requested as soon as its workgroup has the
// unit's slot: each role reads what it needs from the plan and the whole
// page-table row in one round of independent loads.  Gate/up workgroups take
// the first block indices, so their weights lead the memory queue and the down
// weights arrive about when the hidden rows are ready.
//
// Hand-off without counters or cache-wide fences: the workspace holds two
// halves, each with hidden rows and logits.  A launch writes into half p with
// device-scope (sc1) stores, which are coherent across the XCDs' L2 caches;
// readers load half p with device-scope loads until no "pending" word
// 0xFFFFFFFF (a NaN no arithmetic on finite values produces) is left, and the
// down workgroups refill half p ^ 1 with it for the next launch.  p is the
// parity of the launch count, a device word that each down workgroup writing
// output rows increments (without return) when it is done, d/16 per launch: it
// reaches the next launch's value only once every down workgroup of this one
// has read it (a row group's first workgroup finishes before its second).  Every gate/up workgroup
// with rows to write has read it before any down workgroup can finish; in a
// launch that routes from x, where a gate/up workgroup reads logits before it
// knows whether it has items, the gate/up workgroups also count their arrival
// (per parity) and the down workgroups count themselves done only after all
// have arrived.  Every wait is bounded in time: past it the error word gets
// kErrSync and the rows are NaN.
#include <algorithm>
#include <cstddef>
#include <map>
#include <mutex>
#include <utility>

#include "device_util.h"
#include "internal.h"
#include "route_device.h"

namespace moe {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxE = 1024;                       // page-table row staged in LDS (2 words per thread)
constexpr int kMaxUnits = kDecodeMaxT * 32 + 1;   // routed units (<= T * top_k) + shared
constexpr int kMaxEnt = kDecodeMaxT * 32;         // plan positions (T * top_k)
constexpr int kMaxRows = kMaxEnt + kDecodeMaxT;   // hidden rows: plan positions + shared rows
constexpr int kMaxD = 2048;                       // largest d_model
constexpr int kHCap = 72 * 1024;                  // LDS bytes for staged hidden rows
static_assert(kMaxUnits + 1 <= kThreads && kMaxRows <= kThreads, "one plan word per thread");
static_assert(kMaxEnt <= 128, "union_small holds two entries per lane of one wave");
constexpr int kDeviceScope = 16;                  // load cache policy: sc1 (device scope)
constexpr uint32_t kPending = 0xFFFFFFFFu;        // hidden-row word not yet written in this launch

template <int QT> struct Tile;
template <> struct Tile<MOE_Q8_0> {
    uint4 lo, hi;
    uint32_t s;
    __device__ void load(const uint8_t* t, int i) {
        lo = *(const uint4*)(t + q8_lo(i));
        hi = *(const uint4*)(t + q8_hi(i));
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
};

// Weight as multiplied: PREC_F32 keeps the code (the scale is applied once after
// the dot product, so each product is the exact dequantised weight times v up
// to rounding); PREC_BF16 rounds each exact d*q to bf16.
template <int PREC>
__device__ inline float wq(float code, float s) { return PREC == MOE_PREC_BF16 ? round_bf16(code * s) : code; }

// Hides a value from the optimiser where it is used.  Loaded words pass through
// it so that the compiler neither converts a tile's codes once, outside a loop
// (32 live floats per tile), nor computes on a loaded value right where it is
// loaded (a load issued under a condition, or used at once, makes the compiler
// wait for it -- and, loads completing in order, for every load before it --
// before the next load is even issued).
__device__ inline uint32_t opaque(uint32_t w) {
    asm volatile("" : "+v"(w));
    return w;
}

// Code e (0..31) of the lane's block, as the weight multiplied (see wq).
template <int QT, int PREC>
__device__ inline float code_at(const uint32_t (&w)[8], int e, float s) {
    if constexpr (QT == MOE_Q8_0) {
        return wq<PREC>(i8(w[e >> 2], e & 3), s);  // w: lo words, then hi words
    } else {
        const int b = e & 15;                     // w[0..3]: the 16 nibble bytes
        const uint32_t nib = (w[b >> 2] >> (8 * (b & 3) + (e >> 4) * 4)) & 15;
        return wq<PREC>((float)((int)nib - 8), s);
    }
}

// Dot products of M tiles' blocks (one block per lane) with N activation
// vectors of 32 floats (LDS, 16-byte aligned): out[m][n] = block_m . v_n.
// The codes are taken in chunks of CH (4 or 8), each dequantised once for all
// N vectors (a smaller chunk keeps fewer activations live); each product chain
// is split into QA interleaved partial sums (code e into partial e mod QA),
// added in fixed order at the end, so that the chains are independent.
// PREC_F32 multiplies by the scale at the end.
template <int QT, int PREC, int M, int N, int QA, int CH = 8>
__device__ __forceinline__ void tile_dots(const Tile<QT> (&t)[M], const float* const (&v)[N], float (&out)[M][N]) {
    float acc[M][N][QA];
    uint32_t w[M][8];
    float s[M];
#pragma unroll
    for (int m = 0; m < M; m++) {
        s[m] = f16_bits_to_f32(opaque(t[m].s));
        if constexpr (QT == MOE_Q8_0) {
            w[m][0] = opaque(t[m].lo.x); w[m][1] = opaque(t[m].lo.y); w[m][2] = opaque(t[m].lo.z); w[m][3] = opaque(t[m].lo.w);
            w[m][4] = opaque(t[m].hi.x); w[m][5] = opaque(t[m].hi.y); w[m][6] = opaque(t[m].hi.z); w[m][7] = opaque(t[m].hi.w);
        } else {
            w[m][0] = opaque(t[m].nib.x); w[m][1] = opaque(t[m].nib.y); w[m][2] = opaque(t[m].nib.z); w[m][3] = opaque(t[m].nib.w);
            w[m][4] = w[m][5] = w[m][6] = w[m][7] = 0;
        }
#pragma unroll
        for (int n = 0; n < N; n++)
#pragma unroll
            for (int r = 0; r < QA; r++) acc[m][n][r] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < kQK / CH; q++) {
        float x[N][CH];
#pragma unroll
        for (int n = 0; n < N; n++)
#pragma unroll
            for (int c4 = 0; c4 < CH / 4; c4++) {
                const float4 a0 = *(const float4*)(v[n] + CH * q + 4 * c4);
                x[n][4 * c4] = a0.x; x[n][4 * c4 + 1] = a0.y; x[n][4 * c4 + 2] = a0.z; x[n][4 * c4 + 3] = a0.w;
            }
#pragma unroll
        for (int m = 0; m < M; m++)
#pragma unroll
            for (int j = 0; j < CH; j++) {
                const int e = CH * q + j;
                const float c = code_at<QT, PREC>(w[m], e, s[m]);
#pragma unroll
                for (int n = 0; n < N; n++) acc[m][n][e % QA] = fmaf(c, x[n][j], acc[m][n][e % QA]);
            }
    }
#pragma unroll
    for (int m = 0; m < M; m++)
#pragma unroll
        for (int n = 0; n < N; n++) {
            float r = acc[m][n][0];
#pragma unroll
            for (int k = 1; k < QA; k++) r += acc[m][n][k];
            out[m][n] = PREC == MOE_PREC_F32 ? r * s[m] : r;
        }
}

struct DGrid {
    int n_down;      // down workgroups: d / 16, twice that for steps of three or four tokens
    int n_rg;        // gate/up workgroups per unit: d_ff / 16
    int units_max;   // routed units allotted (T * top_k, at most E) + shared
    int gu_tpr;      // gate (or up) tiles per 16 hidden units: d_model / 128
    int dn_tpr;      // down tiles per 16 output rows: d_ff / 128
    int nb_rows;     // hidden rows that fit the LDS at once
    int n_router;    // router workgroups (block indices [0, n_router)), a launch that computes the logits
    int n_gu_wg;     // gate/up workgroups (block indices [n_router, n_router + n_gu_wg))
    int reset_per;   // pending words each down workgroup writes into the other half
    int64_t half;    // floats per workspace half
    int64_t lg_off;  // offset of the logits in a copy (after the hidden rows)
    int64_t copy;    // floats per copy of a half
    int d, f;
    int64_t tile_bytes, down_off;
};

__device__ inline const uint8_t* slot_base(const FfnArgs& a, int e, const int* pts) {
    if (e < 0 || e >= a.E) return nullptr;
    const int slot = pts[e];
    return (slot >= 0 && slot < a.n_slots) ? a.pool + (int64_t)slot * a.payload_bytes : nullptr;
}

// Launch parity: which workspace half this launch writes.
__device__ inline int launch_parity(uint32_t count, int n_down) { return (int)((count / (uint32_t)n_down) & 1u); }

// Whether a split launch computes the unit of expert e (-1: the shared
// expert).  The mask word is picked by comparison, so that the argument array
// is only ever indexed by constants.
__device__ inline bool split_takes(const SplitSel& s, int e) {
    if (s.which == kSplitAll) return true;
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < kSplitMaskWords; j++) word = (e >> 5) == j ? s.miss[j] : word;
    const bool miss = e >= 0 && ((word >> (e & 31)) & 1u);
    return s.which == kSplitHits ? !miss : miss;
}

// ---- routing inside the launch --------------------------------------------------

// Experts a launch that routes takes: kRouteKpl logits per lane of a wave.
constexpr int kRouteKpl = 4;

// LDS of one workgroup's copy of the step's routing.
struct PlanLds {
    float* lg;    // [T, E] logits
    int* ids;     // [T * k] selected experts by entry t * k + j
    float* w;     // [T * k] routing weights by entry
    int* exp;     // units: expert ids ascending
    int* off;     // units: first plan position (and the end)
    int* ent;     // plan position -> entry
    int* na;      // [1] distinct experts
};

static_assert(kDecodeMaxT * kRouteKpl * 64 <= 2 * kThreads, "a step's logits are two words per thread");
// top-k scratch (128 64-bit words per token) in the logits' array, after the logits
constexpr int kTopkScratch = kDecodeMaxT * kRouteKpl * 64;
static_assert(kTopkScratch + kDecodeMaxT * 256 <= kDecodeMaxT * kMaxE && kTopkScratch % 4 == 0,
              "the top-k scratch fits after a step's logits, 16-byte aligned");

// The caller's logits (kRouteLogits), two words per thread, loaded with the
// workgroup's first round of loads and stored to LDS after it.
struct LgIn {
    uint32_t v0, v1;
    __device__ void load(const FfnArgs& a) {
        const bool on = a.route == kRouteLogits;
        const float* src = on ? a.logits_in : (const float*)a.pt;  // a valid address either way
        const int n = on ? a.T * a.E : 1;
        v0 = __float_as_uint(src[min((int)threadIdx.x, n - 1)]);
        v1 = __float_as_uint(src[min((int)threadIdx.x + kThreads, n - 1)]);
    }
    __device__ void store(const FfnArgs& a, float* lg) const {
        if (a.route != kRouteLogits) return;
        const int n = a.T * a.E, i = threadIdx.x;
        if (i < n) lg[i] = __uint_as_float(opaque(v0));
        if (i + kThreads < n) lg[i + kThreads] = __uint_as_float(opaque(v1));
    }
};

// Router workgroups (a launch that computes the logits): the first n_router
// workgroups in dispatch order, wave w of workgroup r computing expert row
// r * kRouterRows + w for every token with the route kernel's row dot (the same
// bits), so that the router weights stream through as many CUs as there are
// rows; the other waves exit at once.  (With 2 rows per workgroup the decode
// step took as long; with 4 and 8 the rows came about 1.5 us later and the
// step 0.8 and 2.2 us later, although the grid was dispatched sooner.)
// The rows are stored with device scope into every copy of the logits of this
// launch's workspace half (from the launch count).  They wait for nothing and exit, and
// every workgroup that waits for the logits has a higher index: workgroups are
// dispatched in index order, so the rows are always computed, whatever else
// occupies the GPU, with no need for all workgroups to be resident at once.
// A router workgroup reads the launch count before the down workgroups can
// move it: they finish only after the gate/up workgroups have routed, which
// needs every row.
constexpr int kRouterRows = 1;  // rows per router workgroup (one per wave)
__device__ void router_role(const FfnArgs& a, const DGrid& g, int r) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = r * kRouterRows + wave;
    if (wave >= kRouterRows || e >= a.E) return;
    const uint32_t count = __hip_atomic_load(a.sync + kSyncCount, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float* row = a.w_router + (int64_t)e * g.d;
    float* dst = a.hbuf + (int64_t)launch_parity(count, g.d / 16) * g.half + g.lg_off + e;
    for (int t = 0; t < a.T; t++) {
        const float v = row_dot(row, a.x, a.x_bf16, t, g.d, lane);
        if (lane < kDecodeCopies)
            __hip_atomic_store(dst + (int64_t)t * a.E + lane * g.copy, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// The step's routing, computed by this workgroup from the logits into LDS: the
// top-k of token t on wave t, then the union (the same code and so the same
// bits as the route kernels).  The logits are the caller's (kRouteLogits,
// already in P.lg from LgIn) or the router rows' device-scope stores into the
// workspace half `par` (copy `reader` mod kDecodeCopies), read until no
// pending word is left.  A wait past the bound sets kErrSync and returns false
// (the routing then comes from whatever was read; its ids are still in
// range).  `publish`: also write ids, weights and plan to the caller's arrays.
// Every thread of the workgroup calls it.
__device__ bool plan_from_logits(const FfnArgs& a, const DGrid& g, int par, int reader, const PlanLds& P, bool publish) {
    const int n = a.T * a.E;
    bool ok = true;
    if (a.route == kRouteRouter) {
        const uint32_t* src = (const uint32_t*)(a.hbuf + (int64_t)par * g.half + (reader % kDecodeCopies) * g.copy +
                                                g.lg_off);
        const uint64_t t0 = wall_clock64();
        for (;;) {
            int pend = 0;
            // (the second word only where there is one: a clamped duplicate
            // would add requests to the few lines every workgroup polls)
            for (int i = threadIdx.x; i < n; i += 2 * kThreads) {
                const bool two = i + kThreads < n;
                const int i2 = two ? i + kThreads : i;
                const uint32_t v0 = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint32_t v1 =
                    two ? __hip_atomic_load(src + i2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : v0;
                pend |= (v0 == kPending) | (v1 == kPending);
                P.lg[i] = __uint_as_float(v0);
                P.lg[i2] = __uint_as_float(v1);
            }
            if (!__syncthreads_or(pend) && a.wait_ticks >= 0) break;
            const int expired = threadIdx.x == 0 && (a.wait_ticks < 0 || (int64_t)(wall_clock64() - t0) > a.wait_ticks);
            if (__syncthreads_or(expired)) {
                if (threadIdx.x == 0) atomicOr(a.err, kErrSync);
                ok = false;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    const int t = threadIdx.x >> 6;
    if (t < a.T) {
        topk_wave<kRouteKpl>(P.lg + t * a.E, a.E, a.k, a.norm, P.ids + t * a.k, P.w + t * a.k,
                             (uint64_t*)(P.lg + kTopkScratch) + t * 128);
    }
    __syncthreads();
    const int N = a.T * a.k;
    union_small(P.ids, N, P.na, P.exp, P.off, P.ent);
    __syncthreads();
    if (publish) {
        const int na = *P.na;
        for (int i = threadIdx.x; i < N; i += kThreads) {
            a.ids_out[i] = P.ids[i];
            a.w_out[i] = P.w[i];
            a.o_entries[i] = P.ent[i];
        }
        for (int i = threadIdx.x; i <= na; i += kThreads) {
            if (i < na) a.o_experts[i] = P.exp[i];
            a.o_offsets[i] = P.off[i];
        }
        if (threadIdx.x == 0) *a.o_n_active = na;
    }
    return ok;
}

// Global -> LDS copies issue every load of the thread before the first LDS
// store, so they cost one memory round trip, not one per element.  Loads are
// unconditional, from clamped (always valid) addresses.

// The page-table row of the layer (E <= kMaxE = 2 words per thread).
struct PtRow {
    uint32_t v[kMaxE / kThreads];
    __device__ void load(const FfnArgs& a) {
        const int32_t* row = a.pt + (int64_t)a.layer * a.E;
#pragma unroll
        for (int j = 0; j < kMaxE / kThreads; j++) v[j] = (uint32_t)row[min((int)threadIdx.x + j * kThreads, a.E - 1)];
    }
    __device__ void store(const FfnArgs& a, int* pts) const {
#pragma unroll
        for (int j = 0; j < kMaxE / kThreads; j++) {
            const int i = threadIdx.x + j * kThreads;
            const uint32_t w = opaque(v[j]);
            if (i < a.E) pts[i] = (int)w;
        }
    }
};

// One token's activations (d <= 2048: one 16-byte load per thread: 8 bf16 or 4
// fp32 values), fp32 in LDS (bf16-rounded in bf16 mode); tok -1 gives zeros.
template <int PREC>
struct XRow {
    uint4 raw;
    int live;
    __device__ void load(const FfnArgs& a, int d, int tok) {
        const int per = a.x_bf16 ? 8 : 4, esz = a.x_bf16 ? 2 : 4;
        const int i = threadIdx.x * per;
        live = (tok >= 0 && i < d) ? 1 : 0;
        const int64_t off = live ? ((int64_t)tok * d + i) * esz : 0;
        raw = *(const uint4*)((const uint8_t*)a.x + off);
    }
    __device__ void store(const FfnArgs& a, int d, float* xr) const {
        const uint4 w = make_uint4(opaque(raw.x), opaque(raw.y), opaque(raw.z), opaque(raw.w));
        const bool z = live == 0;
        if (a.x_bf16) {
            const int i = threadIdx.x * 8;
            if (i >= d) return;
            *(float4*)&xr[i] = z ? make_float4(0.f, 0.f, 0.f, 0.f)
                                 : make_float4(bf16_bits_to_f32(w.x & 0xFFFF), bf16_bits_to_f32(w.x >> 16),
                                               bf16_bits_to_f32(w.y & 0xFFFF), bf16_bits_to_f32(w.y >> 16));
            *(float4*)&xr[i + 4] = z ? make_float4(0.f, 0.f, 0.f, 0.f)
                                     : make_float4(bf16_bits_to_f32(w.z & 0xFFFF), bf16_bits_to_f32(w.z >> 16),
                                                   bf16_bits_to_f32(w.w & 0xFFFF), bf16_bits_to_f32(w.w >> 16));
        } else {
            const int i = threadIdx.x * 4;
            if (i >= d) return;
            float4 v = z ? make_float4(0.f, 0.f, 0.f, 0.f)
                         : make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z),
                                       __uint_as_float(w.w));
            if (PREC == MOE_PREC_BF16)
                v = make_float4(round_bf16(v.x), round_bf16(v.y), round_bf16(v.z), round_bf16(v.w));
            *(float4*)&xr[i] = v;
        }
    }
};

// ---- gate/up ------------------------------------------------------------------------

// Arrays read as float4 (or written by 16-byte direct-to-LDS loads) are 16-byte
// aligned: a misaligned 128-bit LDS access is split and costs several times more.
template <int TG, int RG>
struct GuLds {
    int pts[kMaxE];
    int exp[kMaxUnits + 3];
    int off[kMaxUnits + 3];
    int ent[kMaxEnt];
    alignas(16) float red[2][kWaves][RG * TG][16];
    alignas(16) float x[TG][kMaxD];  // read as float4
    // routing inside the launch
    alignas(16) float lg[kDecodeMaxT * kMaxE];
    int ids[kMaxEnt];
    float wr[kMaxEnt];
    int na;
};

// A gate/up workgroup works through items w, w + G, w + 2G, ... (G gate/up
// workgroups, as many as the device holds beside the others).  An item is RG
// groups of 16 hidden units of one unit: the shared expert's items come first
// (they need no routing, so a launch that routes starts them at once), then
// those of the routed units in plan order.
// The split variant (SPLIT) skips the items of the units the launch does not take.
template <int QT, int PREC, int TG, int RG, int PPW, bool SPLIT>
__device__ __forceinline__ void gate_up_role(const FfnArgs& a, const DGrid& g, int wg, unsigned char* lds_raw,
                                             const SplitSel* sel) {
    GuLds<TG, RG>& L = *(GuLds<TG, RG>*)lds_raw;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, jb = lane >> 4;
    const bool has_shared = a.shared != nullptr;
    const int n_ent = a.T * a.k;

    // Level 1, all independent loads: the launch count, the plan (units, entry
    // ranges, entries) or the caller's logits, the page-table row and, for one
    // token, its activations.
    const uint32_t count = __hip_atomic_load(a.sync + kSyncCount, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int S = has_shared ? g.n_rg / RG : 0;  // items of the shared expert
    const bool plan_in = a.route == kRoutePlan;  // a launch that routes reads no plan
    const int na_raw = plan_in ? *a.n_active : 0;
    PtRow ptr;
    ptr.load(a);
    const int i1 = threadIdx.x;
    const uint32_t ex1 = plan_in ? (uint32_t)a.experts[min(i1, a.E - 1)] : 0u;
    const uint32_t of1 = plan_in ? (uint32_t)a.offsets[min(i1, a.E)] : 0u;
    const uint32_t en1 = plan_in ? (uint32_t)a.entries[min(i1, n_ent - 1)] : 0u;
    XRow<PREC> x1;
    if constexpr (TG == 1) x1.load(a, g.d, 0);
    LgIn lg1;
    lg1.load(a);
    ptr.store(a, L.pts);
    if (i1 < kMaxUnits) L.exp[i1] = (int)opaque(ex1);
    if (i1 < kMaxUnits + 1) L.off[i1] = min(max((int)opaque(of1), 0), n_ent);
    if (i1 < n_ent) L.ent[i1] = min(max((int)opaque(en1), 0), n_ent - 1);
    if constexpr (TG == 1) x1.store(a, g.d, L.x[0]);
    lg1.store(a, L.lg);
    lds_barrier();
    const int par = __builtin_amdgcn_readfirstlane(launch_parity(opaque(count), g.d / 16));
    // A launch that routes counts its gate/up workgroups in: the down workgroups
    // finish (and so move the launch count) only once all have read it, so no
    // workgroup, not even one left without items, reads the next launch's half.
    if (a.route == kRouteRouter && threadIdx.x == 0)
        __hip_atomic_fetch_add(a.sync + kSyncArrive + par, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int na_max = g.units_max - (has_shared ? 1 : 0);
    int na = a.route == kRoutePlan ? min(max((int)opaque((uint32_t)na_raw), 0), na_max) : -1;
    const int per_unit = g.n_rg / RG;             // items per unit
    const int n_pairs = RG * g.gu_tpr;            // (gate, up) tile pairs per item

    for (int item = wg;; item += g.n_gu_wg) {
        const bool routed = item >= S;
        if (routed) {
            if (na < 0) {
                const PlanLds P{L.lg, L.ids, L.wr, L.exp, L.off, L.ent, &L.na};
                plan_from_logits(a, g, par, wg, P, false);
                na = min(L.na, na_max);
            }
            if (item >= S + na * per_unit) break;
        }
        const int ui = routed ? item - S : item;  // item within the routed items, or the shared ones
        const int u = ui / per_unit, rg0 = (ui - u * per_unit) * RG;
        if constexpr (SPLIT) {
            if (!split_takes(*sel, routed ? L.exp[u] : -1)) continue;
        }
        // The slot, then every weight load of the item.  Pair pi is column group
        // pi % gu_tpr of row group rg0 + pi / gu_tpr (gate tile and up tile);
        // lane (n, jb) holds block 4 (pi % gu_tpr) + jb of hidden unit n of that
        // group.  Loads are unconditional: a pair past the item reads its first
        // pair again (its sums are skipped), a missing expert reads pool slot 0
        // (its rows become NaN).
        const uint8_t* base = routed ? slot_base(a, L.exp[u], L.pts) : a.shared;
        if (!base && threadIdx.x == 0) atomicOr(a.err, kErrMiss);
        const uint8_t* src = base ? base : a.pool;
        Tile<QT> tg[PPW], tu[PPW];
#pragma unroll
        for (int q = 0; q < PPW; q++) {
            const int pi = wave + q * kWaves;
            const int64_t t = (int64_t)rg0 * g.gu_tpr + (pi < n_pairs ? pi : 0);
            tg[q].load(src + 2 * t * g.tile_bytes, lane);
            tu[q].load(src + (2 * t + 1) * g.tile_bytes, lane);
        }
        const int b0 = routed ? L.off[u] : 0;
        const int nb = routed ? min(max(L.off[u + 1] - b0, 0), TG) : a.T;  // tokens of the bucket
        if constexpr (TG > 1) {
            // the bucket's activations, issued after the weights (loads complete in order)
            XRow<PREC> xs[TG];
#pragma unroll
            for (int gi = 0; gi < TG; gi++)
                xs[gi].load(a, g.d, gi >= nb ? -1 : !routed ? gi : min(max(L.ent[min(b0 + gi, n_ent - 1)] / a.k, 0), a.T - 1));
#pragma unroll
            for (int gi = 0; gi < TG; gi++) xs[gi].store(a, g.d, L.x[gi]);
            lds_barrier();
        }

        // Per lane: sum over the wave's pairs of each row group; then the four
        // lanes of a row, then the waves (through LDS), in fixed order.
        float accg[RG][TG], accu[RG][TG];
#pragma unroll
        for (int r = 0; r < RG; r++)
#pragma unroll
            for (int gi = 0; gi < TG; gi++) accg[r][gi] = accu[r][gi] = 0.f;
#pragma unroll
        for (int q = 0; q < PPW; q++) {
            const int pi = wave + q * kWaves;
            if (pi >= n_pairs) break;
            const int rr = pi / g.gu_tpr, cb = 4 * (pi - rr * g.gu_tpr) + jb;
            const float* xv[TG];
#pragma unroll
            for (int gi = 0; gi < TG; gi++) xv[gi] = L.x[gi] + cb * kQK;
            const Tile<QT> pair[2] = {tg[q], tu[q]};
            float dd[2][TG];
            // only the bucket's tokens (most buckets of a few tokens hold one)
            if (TG > 1 && nb == 1) {
                const float* x1[1] = {xv[0]};
                float d1[2][1];
                tile_dots<QT, PREC, 2, 1, 4, 8>(pair, x1, d1);
#pragma unroll
                for (int gi = 0; gi < TG; gi++) {
                    dd[0][gi] = gi == 0 ? d1[0][0] : 0.f;
                    dd[1][gi] = gi == 0 ? d1[1][0] : 0.f;
                }
            } else if (TG > 2 && nb == 2) {
                const float* x2[2] = {xv[0], xv[1]};
                float d2[2][2];
                tile_dots<QT, PREC, 2, 2, 2, 4>(pair, x2, d2);
#pragma unroll
                for (int gi = 0; gi < TG; gi++) {
                    dd[0][gi] = gi < 2 ? d2[0][gi < 2 ? gi : 0] : 0.f;
                    dd[1][gi] = gi < 2 ? d2[1][gi < 2 ? gi : 0] : 0.f;
                }
            } else {
                tile_dots<QT, PREC, 2, TG, TG == 1 ? 4 : TG == 2 ? 2 : 1, TG == 1 ? 8 : 4>(pair, xv, dd);
            }
#pragma unroll
            for (int r = 0; r < RG; r++)
#pragma unroll
                for (int gi = 0; gi < TG; gi++) {
                    accg[r][gi] += rr == r ? dd[0][gi] : 0.f;
                    accu[r][gi] += rr == r ? dd[1][gi] : 0.f;
                }
        }
#pragma unroll
        for (int r = 0; r < RG; r++)
#pragma unroll
            for (int gi = 0; gi < TG; gi++) {
                if (gi >= nb) break;  // (rows of tokens the bucket does not have are not read)
                const float gs = cross_row_sum(accg[r][gi]), us = cross_row_sum(accu[r][gi]);
                if (jb == 0) {
                    L.red[0][wave][r * TG + gi][n] = gs;
                    L.red[1][wave][r * TG + gi][n] = us;
                }
            }
        lds_barrier();
        // Threads (row group, token, unit): 16 * TG * RG <= 128.
        if (threadIdx.x < 16 * TG * RG) {
            const int rt = threadIdx.x >> 4, hr = threadIdx.x & 15;
            const int r = rt / TG, gi = rt - r * TG;
            if (gi < nb) {
                float gs = 0.f, us = 0.f;
                for (int w = 0; w < kWaves; w++) {
                    gs += L.red[0][w][rt][hr];
                    us += L.red[1][w][rt][hr];
                }
                float hv = silu(gs) * us;
                if (PREC == MOE_PREC_BF16) hv = round_bf16(hv);
                const int row = routed ? b0 + gi : a.T * a.k + gi;
                // device scope: written through to where every XCD reads it; every copy
                float* dst = a.hbuf + (int64_t)par * g.half + (int64_t)row * g.f + 16 * (rg0 + r) + hr;
                const float hw = base ? hv : __uint_as_float(0x7FC00000u);
#pragma unroll
                for (int c = 0; c < kDecodeCopies; c++)
                    __hip_atomic_store(dst + c * g.copy, hw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        lds_barrier();  // L.red and L.x are reused by the next item
    }
}

// ---- down + merge --------------------------------------------------------------------

struct DownLds {
    int exp[kMaxUnits + 3];
    int off[kMaxUnits + 3];
    int ent[kMaxEnt];                 // plan position -> entry t * k + j
    float wbe[kMaxEnt];               // routing weight by entry
    int tok[kMaxRows];                // hidden row -> token
    float w[kMaxRows];                // hidden row -> weight
    int flag[4];
    int cnt[kDecodeMaxT];             // plan positions the units cover, per token
    int64_t uoff[kMaxUnits + 3];      // unit -> payload offset in the pool (-1 absent, -2 shared)
    uint8_t rdone[kMaxRows];          // hidden row -> every word of it staged (or a row no unit has)
    alignas(16) float red[kWaves][kDecodeMaxT][16];
    alignas(16) float zero[kQK];      // a zero block of activations (rows a bucket does not have)
    int ids[kMaxEnt];                 // routing inside the launch: selected experts by entry
    int na;
    union alignas(16) {               // the page-table row and the logits are read before staging
                                      // starts; hs is read as float4 and written 16 bytes per lane
        struct {
            int pts[kMaxE];
            float lg[kDecodeMaxT * kMaxE];
        } pre;
        float hs[kHCap / 4];
    };
};

// The split variant (SPLIT, one token, every tile in registers) computes each
// unit's term on its own and merges them at the end; see SplitSel.
template <int QT, int PREC, int TG, int DPW, bool SPLIT>
__device__ __forceinline__ void down_role(const FfnArgs& a, const DGrid& g, int D, unsigned char* lds_raw,
                                          const SplitSel* sel) {
    static_assert(!SPLIT || TG == 1, "the split variant takes one token");
    DownLds& L = *(DownLds*)lds_raw;
    // Down workgroup D: rows 16 R .. 16 R + 15 of the output, half hv of the
    // units (steps of three or four tokens split each row group in two)
    constexpr int kSplit = TG == kDecodeMaxT ? 2 : 1;
    const int R = kSplit == 1 ? D : D % (g.d / 16), hv = kSplit == 1 ? 0 : D / (g.d / 16);
    const bool last = hv == kSplit - 1;  // the half that writes y (and counts the launch done)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, jb = lane >> 4;
    const bool has_shared = a.shared != nullptr;
    const int n_ent = a.T * a.k;

    // Level 1, all independent loads: the launch count, n_active, the
    // page-table row and the whole plan (units, entry ranges, entries, weights).
    const uint32_t count = __hip_atomic_load(a.sync + kSyncCount, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool plan_in = a.route == kRoutePlan;  // a launch that routes reads no plan
    const int na_raw = plan_in ? *a.n_active : 0;
    PtRow ptr;
    ptr.load(a);
    const int i1 = threadIdx.x;
    const uint32_t ex1 = plan_in ? (uint32_t)a.experts[min(i1, a.E - 1)] : 0u;
    const uint32_t of1 = plan_in ? (uint32_t)a.offsets[min(i1, a.E)] : 0u;
    const uint32_t en1 = plan_in ? (uint32_t)a.entries[min(i1, n_ent - 1)] : 0u;
    const uint32_t w1 = plan_in ? __float_as_uint(a.topk_w[min(i1, n_ent - 1)]) : 0u;
    LgIn lg1;
    lg1.load(a);
    ptr.store(a, L.pre.pts);
    lg1.store(a, L.pre.lg);
    if (i1 < kMaxUnits) L.exp[i1] = (int)opaque(ex1);
    if (i1 < kMaxUnits + 1) L.off[i1] = min(max((int)opaque(of1), 0), n_ent);
    if (i1 < n_ent) {
        L.ent[i1] = min(max((int)opaque(en1), 0), n_ent - 1);
        L.wbe[i1] = __uint_as_float(opaque(w1));
    }
    if (threadIdx.x == 0) L.flag[0] = 1;
    if (threadIdx.x < kDecodeMaxT) L.cnt[threadIdx.x] = 0;
    if (threadIdx.x < kQK) L.zero[threadIdx.x] = 0.f;
    lds_barrier();
    const int par = __builtin_amdgcn_readfirstlane(launch_parity(opaque(count), g.d / 16));
    // the arrivals of the next launch start from zero
    if (D == 0 && threadIdx.x == 0)
        __hip_atomic_store(a.sync + kSyncArrive + (par ^ 1), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int na_max = g.units_max - (has_shared ? 1 : 0);
    int na = min(max((int)opaque((uint32_t)na_raw), 0), na_max);
    if (a.route != kRoutePlan) {
        // the routing of the step, computed here (workgroup 0 also hands it to the caller)
        const PlanLds P{L.pre.lg, L.ids, L.wbe, L.exp, L.off, L.ent, &L.na};
        if (!plan_from_logits(a, g, par, g.n_gu_wg + D, P, D == 0) && threadIdx.x == 0) L.flag[0] = 0;
        na = min(L.na, na_max);
    }

    // Level 2: this workgroup's W_d tiles of every unit of its half.  Tile p
    // is (unit p / dn_tpr, column group p % dn_tpr); wave w holds tiles
    // p_lo + w + 8 i.  Each unit's payload offset is looked up once (-1: not
    // resident).  With two halves, the first takes units [0, ceil(0.55 U)):
    // the later units' hidden rows come last (their gate/up items are last),
    // so the second half, which also waits for the first's sums, gets fewer.
    const int U = na + (has_shared ? 1 : 0);
    const int u_mid = (11 * U + 19) / 20;
    const int u_lo = kSplit == 2 && hv == 1 ? u_mid : 0, u_hi = kSplit == 2 && hv == 0 ? u_mid : U;
    const int p_lo = u_lo * g.dn_tpr, P = u_hi * g.dn_tpr;
    if (threadIdx.x < U) {
        const int u = threadIdx.x;
        int64_t off = -1;
        if (u >= na) off = -2;  // shared expert
        else {
            const int ex = L.exp[u];
            const int slot = (ex >= 0 && ex < a.E) ? L.pre.pts[ex] : -1;
            if (slot >= 0 && slot < a.n_slots) off = (int64_t)slot * a.payload_bytes;
        }
        if constexpr (SPLIT) {
            if (!split_takes(*sel, u < na ? L.exp[u] : -1)) off = -3;  // a unit the other launch takes
        }
        L.uoff[u] = off;
    }
    lds_barrier();
    // Address of tile p, or null for a unit that is not resident.
    auto tile_ptr = [&](int p) __attribute__((always_inline)) -> const uint8_t* {
        const int u = p / g.dn_tpr, c = p - u * g.dn_tpr;
        const int64_t off = L.uoff[u];
        const uint8_t* b = off == -2 ? a.shared : off >= 0 ? a.pool + off : nullptr;
        return b ? b + g.down_off + ((int64_t)R * g.dn_tpr + c) * g.tile_bytes : nullptr;
    };
    // Loads are unconditional: a slot past the last tile, or a unit that is
    // not resident, reads pool slot 0 (no sums are taken from the former; the
    // latter's rows are NaN through h).
    const uint8_t* fallback = a.pool + g.down_off + (int64_t)R * g.dn_tpr * g.tile_bytes;
    Tile<QT> td[DPW];
#pragma unroll
    for (int i = 0; i < DPW; i++) {
        const int p = p_lo + wave + kWaves * i;
        const uint8_t* tp = p < P ? tile_ptr(p) : nullptr;
        td[i].load(tp ? tp : fallback, lane);
    }
    // A split launch that merges reads the terms of the units it does not take
    // (written by the launch before it): thread 16 u + r holds unit u's row r.
    float pre = 0.f;
    if constexpr (SPLIT) {
        const int u = threadIdx.x >> 4;
        const bool want = sel->which == kSplitMisses && u < U && L.uoff[u] == -3;
        const int v = u < na ? L.off[min(u, na)] : n_ent;
        pre = *(want ? sel->part + (int64_t)v * g.d + 16 * R + (threadIdx.x & 15) : sel->part);
    }
    // The arrivals of this launch's gate/up workgroups, read now (they arrive
    // as they start, long before this; the load waits with the tiles') and
    // checked at the end, so that the end does not wait for a round trip.
    const uint32_t arrived0 = a.route == kRouteRouter && threadIdx.x == 0
                                  ? __hip_atomic_load(a.sync + kSyncArrive + par, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT)
                                  : 0u;
    // Token and weight of every hidden row (the shared rows: token t, weight 1).
    // A token counts the plan positions the units cover that are its own: a
    // token with fewer than top_k (the plan dropped an out-of-range id) gets a
    // NaN row, as the chunk path's combine gives it.
    if (threadIdx.x < kMaxRows) {
        const int v = threadIdx.x;
        L.rdone[v] = v >= L.off[na] && v < n_ent;  // rows [off[na], T k): entries the plan dropped
        if (v < n_ent) {
            const int ent = L.ent[v];
            L.tok[v] = ent / a.k;
            L.w[v] = L.wbe[ent];
            if (v < L.off[na]) atomicAdd(&L.cnt[ent / a.k], 1);
        } else {
            L.tok[v] = v - n_ent;
            L.w[v] = 1.f;
        }
    }

    // Rows of unit u: its plan positions, or the shared rows.
    auto v_begin = [&](int u) __attribute__((always_inline)) { return u < na ? L.off[u] : n_ent; };
    auto v_end = [&](int u) __attribute__((always_inline)) { return u < na ? L.off[u + 1] : n_ent + a.T; };
    lds_barrier();
    if constexpr (SPLIT) {
        // rows of the units the other launch takes: never written here, never waited for
        if (threadIdx.x < U && L.uoff[threadIdx.x] == -3)
            for (int v = v_begin(threadIdx.x); v < v_end(threadIdx.x); v++) L.rdone[v] = 1;
        lds_barrier();
    }
    // Per register slot, read before the wait (wave-uniform, so scalar): the
    // unit's rows [sv0, sv1), their tokens (2 bits each; a bucket has at most
    // 4 rows) and the tile's column group.
    int sv0[DPW], sv1[DPW], stok[DPW], scol[DPW];
#pragma unroll
    for (int i = 0; i < DPW; i++) {
        const int p = p_lo + wave + kWaves * i;
        const int u = min(p, max(P - 1, p_lo)) / g.dn_tpr;
        const int v0 = v_begin(u), v1 = min(v_end(u), v0 + kDecodeMaxT);
        int tp = 0;
        for (int v = v0; v < v1; v++) tp |= (L.tok[v] & 3) << (2 * (v - v0));
        sv0[i] = __builtin_amdgcn_readfirstlane(v0);
        sv1[i] = __builtin_amdgcn_readfirstlane(p < P && !(SPLIT && L.uoff[u] == -3) ? v1 : v0);
        stok[i] = __builtin_amdgcn_readfirstlane(tp);
        scol[i] = __builtin_amdgcn_readfirstlane(min(p, max(P - 1, p_lo)) - u * g.dn_tpr);
    }

    const float* hhalf = a.hbuf + (int64_t)par * g.half + (D % kDecodeCopies) * g.copy;
    const uint64_t t0 = wall_clock64();
    float acc[TG];
#pragma unroll
    for (int t = 0; t < TG; t++) acc[t] = 0.f;
    float dv[SPLIT ? DPW : 1];  // split: each register slot's dot, kept apart
#pragma unroll
    for (int i = 0; i < (SPLIT ? DPW : 1); i++) dv[i] = 0.f;
    // Groups of units whose hidden rows fit the LDS, in plan order.  The first
    // group is peeled out of the loop: computing on the tiles inside a loop lets
    // the compiler hoist work on their loaded values above it, and so wait for
    // the tiles before the poll.
    auto group = [&](const int ua) __attribute__((always_inline)) -> int {
        const int va = __builtin_amdgcn_readfirstlane(v_begin(ua));
        int ub = ua + 1;
        while (ub < u_hi && v_end(ub) - va <= g.nb_rows) ub++;
        ub = __builtin_amdgcn_readfirstlane(ub);
        // (a valid plan never clips)
        const int vb = __builtin_amdgcn_readfirstlane(min(v_end(ub - 1), va + g.nb_rows));
        // Stage rows [va, vb) straight into LDS with device-scope loads (1 KB
        // per wave instruction, no registers), until no pending word is left.
        // Wave w takes rows w, w + 8, ... of the group: it stages a row until
        // one read finds every word of it written (the words are final then)
        // and not again, so that later reads carry only the rows still
        // pending.  (With rows not a whole number of 1 KB instructions, or one
        // token, whose few rows come in together, every row is staged each
        // time: one token's step was 0.3 us slower staging by row.)  Rows no
        // unit has (entries the plan dropped) are never written and never
        // checked.
        const int nrows = max(vb - va, 0);
        const int n16 = nrows * g.f / 4;  // 16-byte pieces
        const int n_ins = (n16 + 63) / 64;
        const int ppr = g.f / 4;          // pieces per row
        const bool by_row = TG > 1 && g.f % 256 == 0;
        const int ipr = g.f / 256;        // instructions per row (by_row)
        const float* src = hhalf + (int64_t)va * g.f;
        const int gap0 = (max(min(L.off[na], n_ent), va) - va) * g.f / 4;  // pieces [gap0, gap1): no unit's
        const int gap1 = (max(n_ent, va) - va) * g.f / 4;
        // Tiles beyond the registers (more units than DPW * 8 / dn_tpr): this
        // wave's tiles p = p0, p0 + 8, ... below pe, two loads in flight, the
        // first issued before the wait.
        const int pe = ub * g.dn_tpr;
        int p0 = p_lo + kWaves * DPW + wave;
        if (p0 < ua * g.dn_tpr) p0 += (ua * g.dn_tpr - p0 + kWaves - 1) / kWaves * kWaves;
        p0 = __builtin_amdgcn_readfirstlane(p0);
        auto beyond_ptr = [&](int p) __attribute__((always_inline)) -> const uint8_t* {
            const uint8_t* tp = p < pe ? tile_ptr(p) : nullptr;
            return tp ? tp : fallback;
        };
        Tile<QT> ta[1], tb[1];
        if (TG > 1 && p0 < pe) ta[0].load(beyond_ptr(p0), lane);  // (one token: after the wait)
        for (;;) {
            if (by_row) {
                for (int r = wave; r < nrows; r += kWaves) {
                    if (__builtin_amdgcn_readfirstlane(L.rdone[va + r])) continue;
                    for (int q = 0; q < ipr; q++) {
                        const int j = r * ipr + q;
                        __builtin_amdgcn_global_load_lds(src + 4 * (j * 64 + lane),
                                                          (__attribute__((address_space(3))) void*)(L.hs + j * 256),
                                                          16, 0, kDeviceScope);
                    }
                }
            } else {
                for (int j = wave; j < n_ins; j += kWaves)
                    __builtin_amdgcn_global_load_lds(src + 4 * min(j * 64 + lane, n16 - 1),
                                                      (__attribute__((address_space(3))) void*)(L.hs + j * 256), 16,
                                                      0, kDeviceScope);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            int pend = 0;
            if (by_row) {
                for (int r = wave; r < nrows; r += kWaves) {
                    if (__builtin_amdgcn_readfirstlane(L.rdone[va + r])) continue;
                    bool pr = false;
                    for (int q = lane; q < ppr; q += 64) {
                        const uint4 b = *(const uint4*)(L.hs + 4 * (r * ppr + q));
                        pr |= (b.x == kPending) | (b.y == kPending) | (b.z == kPending) | (b.w == kPending);
                    }
                    if (__ballot(pr)) pend = 1;
                    else if (lane == 0) L.rdone[va + r] = 1;
                }
            } else {
                for (int i = threadIdx.x; i < n16; i += kThreads) {
                    const uint4 b = *(const uint4*)(L.hs + 4 * i);
                    const bool used = SPLIT ? !L.rdone[va + i / ppr] : i < gap0 || i >= gap1;
                    pend |= used && ((b.x == kPending) | (b.y == kPending) | (b.z == kPending) | (b.w == kPending));
                }
            }
            if (!__syncthreads_or(pend) && a.wait_ticks >= 0) break;
            const int expired = threadIdx.x == 0 && (a.wait_ticks < 0 || (int64_t)(wall_clock64() - t0) > a.wait_ticks);
            if (__syncthreads_or(expired)) {
                if (threadIdx.x == 0) {
                    atomicOr(a.err, kErrSync);
                    L.flag[0] = 0;
                }
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        // Per lane: the tiles of units [ua, ub), each with the unit's rows:
        // acc[token] += w * (block . h).
#pragma unroll
        for (int i = 0; i < DPW; i++) {
            const int v0 = max(sv0[i], va), v1 = min(sv1[i], vb);
            if (v0 >= v1) continue;
            const Tile<QT> one[1] = {td[i]};
            if constexpr (TG <= 2) {
                // the unit's rows (at most TG), each block dequantised once for all
                const float* hr[TG];
#pragma unroll
                for (int r = 0; r < TG; r++)
                    hr[r] = v0 + r < v1 ? L.hs + (v0 + r - va) * g.f + (4 * scol[i] + jb) * kQK : L.zero;
                float dr[1][TG];
                tile_dots<QT, PREC, 1, TG, TG == 1 ? 4 : 2>(one, hr, dr);
                if constexpr (SPLIT) {
                    dv[i] = dr[0][0];
                    continue;
                }
#pragma unroll
                for (int r = 0; r < TG; r++) {
                    if (v0 + r >= v1) break;
                    const int tk = (stok[i] >> (2 * (v0 + r - sv0[i]))) & 3;
                    const float dw = L.w[v0 + r] * dr[0][r];
#pragma unroll
                    for (int q = 0; q < TG; q++) acc[q] += tk == q ? dw : 0.f;
                }
            } else {
                // the unit's rows two at a time, each block dequantised once per
                // pair (a last odd row alone): two pairs' activations in chunks
                // of 4 codes stay beside DPW tiles in registers
                for (int r = v0; r < v1; r += 2) {
                    float dr[2];
                    const float* h0p = L.hs + (r - va) * g.f + (4 * scol[i] + jb) * kQK;
                    if (r + 1 < v1) {
                        const float* h2[2] = {h0p, h0p + g.f};
                        float d[1][2];
                        tile_dots<QT, PREC, 1, 2, 2, 4>(one, h2, d);
                        dr[0] = d[0][0];
                        dr[1] = d[0][1];
                    } else {
                        const float* h1[1] = {h0p};
                        float d[1][1];
                        tile_dots<QT, PREC, 1, 1, 4>(one, h1, d);
                        dr[0] = d[0][0];
                    }
#pragma unroll
                    for (int j = 0; j < 2; j++) {
                        const int v = r + j;
                        if (v >= v1) break;
                        const int tk = (stok[i] >> (2 * (v - sv0[i]))) & 3;
                        const float dw = L.w[v] * dr[j];
#pragma unroll
                        for (int q = 0; q < TG; q++) acc[q] += tk == q ? dw : 0.f;
                    }
                }
            }
        }
        // the tiles beyond the registers, in order (a non-resident unit's
        // tiles read the fallback; its rows are NaN through h)
        auto beyond = [&](const Tile<QT> (&t)[1], int p) __attribute__((always_inline)) {
            const int u = p / g.dn_tpr, c = p - u * g.dn_tpr;
            const int v0 = max(v_begin(u), va), v1 = min(v_end(u), vb);
            for (int v = v0; v < v1; v++) {
                const float* hv1[1] = {L.hs + (v - va) * g.f + (4 * c + jb) * kQK};
                float d1[1][1];
                tile_dots<QT, PREC, 1, 1, 4>(t, hv1, d1);
                const int tk = L.tok[v];
                const float dw = L.w[v] * d1[0][0];
#pragma unroll
                for (int q = 0; q < TG; q++) acc[q] += tk == q ? dw : 0.f;
            }
        };
        if (TG == 1 && p0 < pe) ta[0].load(beyond_ptr(p0), lane);
        for (int p = p0; p < pe;) {
            if (p + kWaves < pe) tb[0].load(beyond_ptr(p + kWaves), lane);
            beyond(ta, p);
            p += kWaves;
            if (p >= pe) break;
            if (p + kWaves < pe) ta[0].load(beyond_ptr(p + kWaves), lane);
            beyond(tb, p);
            p += kWaves;
        }
        __syncthreads();
        return ub;
    };
    if (u_lo < u_hi) {
        int ua = group(u_lo);
        while (ua < u_hi) ua = group(ua);
    }
    if constexpr (SPLIT) {
        // Unit u's term for row r: per tile the row's four lanes, then the
        // unit's tiles in order, times the routing weight (one fixed order in
        // either launch).  The staged rows are done with, so the LDS holds the
        // tile sums [P][16] and then the merged terms [U][16].
        float* tv = L.hs;
        float* tu = L.hs + 16 * P;
#pragma unroll
        for (int i = 0; i < DPW; i++) {
            const int p = wave + kWaves * i;
            const float s = cross_row_sum(dv[i]);
            if (jb == 0 && p < P) tv[16 * p + n] = s;
        }
        __syncthreads();
        const int u = threadIdx.x >> 4, r = threadIdx.x & 15;
        const bool ok = L.flag[0];
        if (u < U) {
            float t = 0.f;
            for (int c = 0; c < g.dn_tpr; c++) t += tv[16 * (u * g.dn_tpr + c) + r];
            t *= L.w[v_begin(u)];
            const bool mine = L.uoff[u] != -3;
            if (sel->which == kSplitHits) {
                if (mine)
                    sel->part[(int64_t)v_begin(u) * g.d + 16 * R + r] = ok ? t : __uint_as_float(0x7FC00000u);
            } else {
                tu[16 * u + r] = mine ? t : pre;
            }
        }
        __syncthreads();
        if (sel->which != kSplitHits && threadIdx.x < 16) {
            float y = 0.f;
            for (int q = 0; q < U; q++) y += tu[16 * q + r];
            a.y[16 * R + r] = ok && L.cnt[0] == a.k ? y : __uint_as_float(0x7FC00000u);
        }
    } else {
        // The four lanes of a row, then the waves in order.
#pragma unroll
        for (int t = 0; t < TG; t++) {
            const float s = cross_row_sum(acc[t]);
            if (jb == 0) L.red[wave][t][n] = s;
        }
        __syncthreads();
        // The first half of a split row group hands its sums to the second with
        // device scope (a NaN as the canonical NaN, never the pending word); the
        // second adds them first, then its own: one fixed order.
        // (the partial rows follow the copies in each half)
        uint32_t* prow = (uint32_t*)(a.hbuf + (int64_t)par * g.half + kDecodeCopies * g.copy) + 16 * R;
        const int tq = threadIdx.x >> 4, rq = threadIdx.x & 15;
        float y = 0.f;
        if (threadIdx.x < 16 * a.T)
            for (int w = 0; w < kWaves; w++) y += L.red[w][tq][rq];
        if (!last) {
            if (threadIdx.x < 16 * a.T) {
                const float v = L.flag[0] && y == y ? y : __uint_as_float(0x7FC00000u);
                __hip_atomic_store(prow + (int64_t)tq * g.d + rq, __float_as_uint(v), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        } else {
            bool ok = true;
            if constexpr (kSplit == 2) {
                float y0 = 0.f;
                const uint64_t t1 = wall_clock64();
                for (;;) {
                    int pend = 0;
                    if (threadIdx.x < 16 * a.T) {
                        const uint32_t v = __hip_atomic_load(prow + (int64_t)tq * g.d + rq, __ATOMIC_RELAXED,
                                                             __HIP_MEMORY_SCOPE_AGENT);
                        pend = v == kPending;
                        y0 = __uint_as_float(v);
                    }
                    if (!__syncthreads_or(pend) && a.wait_ticks >= 0) break;
                    const int expired =
                        threadIdx.x == 0 && (a.wait_ticks < 0 || (int64_t)(wall_clock64() - t1) > a.wait_ticks);
                    if (__syncthreads_or(expired)) {
                        if (threadIdx.x == 0) atomicOr(a.err, kErrSync);
                        ok = false;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                y = y0 + y;
            }
            if (threadIdx.x < 16 * a.T)
                a.y[(int64_t)tq * g.d + 16 * R + rq] =
                    ok && L.flag[0] && L.cnt[tq] == a.k ? y : __uint_as_float(0x7FC00000u);
        }
    }
    // This workgroup's share of the other half back to pending for the next
    // launch (no one uses that half during this one).  Done last: a store loop
    // before the tile loads made them wait for every earlier load.
    {
        float* nxt = a.hbuf + (int64_t)(par ^ 1) * g.half;
        const int64_t r0 = (int64_t)D * g.reset_per;
        for (int j = threadIdx.x; j < g.reset_per; j += kThreads)
            if (r0 + j < g.half) nxt[r0 + j] = __uint_as_float(kPending);
    }
    // This launch is done with its half: count it (no return needed), once every
    // gate/up workgroup of a launch that routes has arrived.  Only the row
    // groups' last halves count, so that a launch moves the count by d / 16
    // whatever its token count, and a last half finishes only after its first.
    if (threadIdx.x == 0 && last) {
        if (a.route == kRouteRouter && (a.wait_ticks < 0 || arrived0 < (uint32_t)g.n_gu_wg)) {
            const uint64_t t1 = wall_clock64();
            while (a.wait_ticks < 0 ||
                   __hip_atomic_load(a.sync + kSyncArrive + par, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                       (uint32_t)g.n_gu_wg) {
                if (a.wait_ticks < 0 || (int64_t)(wall_clock64() - t1) > a.wait_ticks) {
                    atomicOr(a.err, kErrSync);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        __hip_atomic_fetch_add(a.sync + kSyncCount, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

using GuLdsMax = GuLds<kDecodeMaxT, 2>;
static_assert(offsetof(DownLds, hs) % 16 == 0 && offsetof(DownLds, zero) % 16 == 0 &&
                  offsetof(GuLdsMax, x) % 16 == 0 && offsetof(GuLdsMax, lg) % 16 == 0,
              "LDS arrays read as float4 must be 16-byte aligned");

constexpr int kLdsBytes = sizeof(DownLds) > sizeof(GuLds<kDecodeMaxT, 2>) ? sizeof(DownLds) : sizeof(GuLds<kDecodeMaxT, 2>);

// Hidden-unit groups of 16 per gate/up item.  (Two for steps of several tokens,
// so that one round of workgroups held the step, left 32 tile pairs per item,
// 4 per wave in registers, and spilled: the four-token Q4_0 step's gate/up
// phase took 8 us longer than with one group and two rounds.)
template <int QT, int TG> constexpr int rows_per_item() { return 1; }

template <int QT, int PREC, int TG, int PPW, int DPW>
__global__ __launch_bounds__(kThreads, 4) void ffn_decode_kernel(FfnArgs a, DGrid g) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
    const int b = blockIdx.x - g.n_router;
    if (b < 0) router_role(a, g, blockIdx.x);
    else if (b < g.n_gu_wg) gate_up_role<QT, PREC, TG, rows_per_item<QT, TG>(), PPW, false>(a, g, b, lds, nullptr);
    else down_role<QT, PREC, TG, DPW, false>(a, g, b - g.n_gu_wg, lds, nullptr);
}

// The hit/miss split's launches (one token, the plan given): the same roles,
// each unit's term kept apart (SplitSel).
template <int QT, int PREC, int PPW, int DPW>
__global__ __launch_bounds__(kThreads, 4) void ffn_split_kernel(FfnArgs a, DGrid g, SplitSel s) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
    const int b = blockIdx.x;
    if (b < g.n_gu_wg) gate_up_role<QT, PREC, 1, rows_per_item<QT, 1>(), PPW, true>(a, g, b, lds, &s);
    else down_role<QT, PREC, 1, DPW, true>(a, g, b - g.n_gu_wg, lds, &s);
}

// Workgroups of `kern` the device holds at once (0 if unknown).
int resident_capacity(const void* kern) {
    static std::mutex mu;
    static std::map<std::pair<const void*, int>, int> cap;  // (kernel, device) -> workgroups
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cap.find({kern, dev});
    if (it == cap.end()) {
        int occ = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, kThreads, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            occ = cus = 0;
        it = cap.emplace(std::make_pair(kern, dev), occ * cus).first;
    }
    return it->second;
}

template <int QT, int PREC, int TG, int PPW, int DPW>
hipError_t launch_k(DGrid g, const FfnArgs& a, hipStream_t s) {
    auto kern = ffn_decode_kernel<QT, PREC, TG, PPW, DPW>;
    // As many gate/up workgroups as the device holds beside the down ones (all
    // resident: no workgroup waits for a slot), at most one per item.
    const int items = g.units_max * (g.n_rg / rows_per_item<QT, TG>());
    const int cap = resident_capacity((const void*)kern);
    // Every wait in a launch is for workgroups of lower index that wait for
    // nothing of higher index: gate/up workgroups wait only for router
    // workgroups (which wait for nothing), down workgroups for router and
    // gate/up workgroups.  Workgroups are dispatched in index order, so what a
    // workgroup waits for has been dispatched and finishes even when other
    // kernels leave room for only part of the grid; sizing the grid to what is
    // resident only keeps every workgroup running from the start.
    // Router workgroups exit after one row, so the gate/up and down workgroups
    // that do not fit beside them at first are dispatched a few microseconds
    // in, long before the routing they wait for is complete.
    g.n_router = a.route == kRouteRouter ? (a.E + kRouterRows - 1) / kRouterRows : 0;
    const int room = cap - g.n_down;
    g.n_gu_wg = room > 0 ? std::min(items, room) : std::min(items, 64);
    hipLaunchKernelGGL(kern, dim3(g.n_router + g.n_gu_wg + g.n_down), dim3(kThreads), 0, s, a, g);
    return hipGetLastError();
}

// Down tiles held in registers per wave: every tile of the step's units in the
// usual cases with d_ff 512 (top-8: 9 units at T = 1; at T = 2, 6 (Q8_0) or
// 12 (Q4_0); at T = 4, 6 (Q8_0)); more are loaded after the wait.  Four Q4_0
// tokens (about 20 units) keep 8, so that two rows' activations fit beside them.
template <int QT, int TG> constexpr int down_per_wave() {
    return TG == 1 ? 5 : QT == MOE_Q4_0 ? (TG == 2 ? 6 : 8) : 3;
}

template <int QT, int PREC, int TG>
hipError_t launch_w(const DGrid& g, const FfnArgs& a, hipStream_t s) {
    constexpr int D = down_per_wave<QT, TG>();
    const int pairs = rows_per_item<QT, TG>() * g.gu_tpr;  // tile pairs per gate/up item
    if (g.n_rg % rows_per_item<QT, TG>()) return hipErrorInvalidValue;
    if (pairs <= kWaves) return launch_k<QT, PREC, TG, 1, D>(g, a, s);
    if (pairs <= 2 * kWaves) return launch_k<QT, PREC, TG, 2, D>(g, a, s);
    if (pairs <= 4 * kWaves) return launch_k<QT, PREC, TG, 4, D>(g, a, s);
    return hipErrorInvalidValue;
}

template <int QT, int PREC>
hipError_t launch_tg(const DGrid& g, const FfnArgs& a, hipStream_t s) {
    if (a.T <= 1) return launch_w<QT, PREC, 1>(g, a, s);
    if (a.T <= 2) return launch_w<QT, PREC, 2>(g, a, s);
    return launch_w<QT, PREC, 4>(g, a, s);
}

// The split variant: grid as launch_k's (no router workgroups), every W_d tile
// of the step in registers.
template <int QT, int PREC, int PPW>
hipError_t launch_split_k(DGrid g, const FfnArgs& a, const SplitSel& sel, hipStream_t s) {
    constexpr int D = down_per_wave<QT, 1>();
    static_assert(kWaves * D >= kSplitMaxTiles, "every tile of a split step in registers");
    auto kern = ffn_split_kernel<QT, PREC, PPW, D>;
    const int items = g.units_max * (g.n_rg / rows_per_item<QT, 1>());
    const int cap = resident_capacity((const void*)kern);
    g.n_router = 0;
    const int room = cap - g.n_down;
    g.n_gu_wg = room > 0 ? std::min(items, room) : std::min(items, 64);
    hipLaunchKernelGGL(kern, dim3(g.n_gu_wg + g.n_down), dim3(kThreads), 0, s, a, g, sel);
    return hipGetLastError();
}

template <int QT, int PREC>
hipError_t launch_split_w(const DGrid& g, const FfnArgs& a, const SplitSel& sel, hipStream_t s) {
    const int pairs = rows_per_item<QT, 1>() * g.gu_tpr;
    if (pairs <= kWaves) return launch_split_k<QT, PREC, 1>(g, a, sel, s);
    if (pairs <= 2 * kWaves) return launch_split_k<QT, PREC, 2>(g, a, sel, s);
    if (pairs <= 4 * kWaves) return launch_split_k<QT, PREC, 4>(g, a, sel, s);
    return hipErrorInvalidValue;
}

// Grid and workspace geometry of a decode launch (false: a shape the kernel
// does not take).
bool decode_grid(const Geom& geo, const FfnArgs& a, DGrid* out) {
    if (a.T < 1 || a.T > kDecodeMaxT || a.E > kMaxE || a.k > 32 || geo.d > kMaxD) return false;
    DGrid g{};
    g.units_max = min(a.T * a.k, a.E) + (a.shared ? 1 : 0);
    // Steps of three or four tokens (the four-token kernel; about 20 units of
    // Q4_0 products per row group) split each row group's units over two
    // down workgroups.
    g.n_down = geo.d / 16 * (a.T > 2 ? 2 : 1);
    g.n_rg = geo.f / 16;
    g.gu_tpr = geo.nb_d / 4;
    g.dn_tpr = geo.nb_f / 4;
    g.d = geo.d;
    g.f = geo.f;
    g.tile_bytes = geo.tile_bytes;
    g.down_off = 2 * geo.gu_tiles * geo.tile_bytes;
    g.nb_rows = kHCap / (4 * geo.f);
    g.half = decode_half_floats(a.k, geo.f, a.E, geo.d);
    g.copy = decode_copy_floats(a.k, geo.f, a.E);
    g.lg_off = decode_h_rows_floats(a.k, geo.f);
    g.reset_per = (int)((g.half + g.n_down - 1) / g.n_down);
    if (g.nb_rows < kDecodeMaxT) return false;
    *out = g;
    return true;
}

}  // namespace

hipError_t launch_ffn_decode(const Geom& geo, const FfnArgs& a, int prec, hipStream_t s) {
    DGrid g{};
    if (!decode_grid(geo, a, &g)) return hipErrorInvalidValue;
    if (geo.qtype == MOE_Q8_0)
        return prec == MOE_PREC_BF16 ? launch_tg<MOE_Q8_0, MOE_PREC_BF16>(g, a, s)
                                     : launch_tg<MOE_Q8_0, MOE_PREC_F32>(g, a, s);
    return prec == MOE_PREC_BF16 ? launch_tg<MOE_Q4_0, MOE_PREC_BF16>(g, a, s)
                                 : launch_tg<MOE_Q4_0, MOE_PREC_F32>(g, a, s);
}

hipError_t launch_ffn_split(const Geom& geo, const FfnArgs& a, int prec, const SplitSel& sel, hipStream_t s) {
    DGrid g{};
    if (a.T != 1 || a.route != kRoutePlan || !sel.part || !decode_grid(geo, a, &g) ||
        g.units_max * g.dn_tpr > kSplitMaxTiles)
        return hipErrorInvalidValue;
    if (geo.qtype == MOE_Q8_0)
        return prec == MOE_PREC_BF16 ? launch_split_w<MOE_Q8_0, MOE_PREC_BF16>(g, a, sel, s)
                                     : launch_split_w<MOE_Q8_0, MOE_PREC_F32>(g, a, sel, s);
    return prec == MOE_PREC_BF16 ? launch_split_w<MOE_Q4_0, MOE_PREC_BF16>(g, a, sel, s)
                                 : launch_split_w<MOE_Q4_0, MOE_PREC_F32>(g, a, sel, s);
}

}  // namespace moe
