// Routing steps shared by the route kernels and the decode kernel that routes
// in its own launch, so that both give the same bits: the router row dot, the
// top-k of one token on one wave and the union of a few tokens' assignments
// ("Nanite for Experts", §3.1 and §1; "Paging the Experts", §3.1: top-8 of
// 256 routed experts; "Nanite for Experts", §5.3: the expert-major union).
#pragma once
#include "device_util.h"

namespace moe {

// Lane's share of row . x[t] (float4 slices at a 1 KiB stride, in order), then
// the fixed lane butterfly: every lane returns the same bits.  Every load of a
// pass is issued before any is used, from a clamped (always valid) address:
// a load under a condition makes the compiler wait for it before the next one
// is issued, which turned one memory round trip into several.
__device__ inline float row_dot(const float* row, const void* x, int x_bf16, int t, int d, int lane) {
    constexpr int U = 8;  // slices in flight per lane (d_model 2048 is 8 slices)
    float acc = 0.f;
    for (int c0 = lane * 4; c0 < d; c0 += 256 * U) {
        float4 wv[U], xv[U];
        if (x_bf16) {
            uint2 xb[U];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int c = min(c0 + 256 * u, d - 4);
                wv[u] = *(const float4*)(row + c);
                xb[u] = *(const uint2*)((const uint16_t*)x + (int64_t)t * d + c);
            }
#pragma unroll
            for (int u = 0; u < U; u++)
                xv[u] = make_float4(bf16_bits_to_f32(xb[u].x & 0xFFFF), bf16_bits_to_f32(xb[u].x >> 16),
                                    bf16_bits_to_f32(xb[u].y & 0xFFFF), bf16_bits_to_f32(xb[u].y >> 16));
        } else {
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int c = min(c0 + 256 * u, d - 4);
                wv[u] = *(const float4*)(row + c);
                xv[u] = *(const float4*)((const float*)x + (int64_t)t * d + c);
            }
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (c0 + 256 * u < d) {
                acc = fmaf(wv[u].x, xv[u].x, acc);
                acc = fmaf(wv[u].y, xv[u].y, acc);
                acc = fmaf(wv[u].z, xv[u].z, acc);
                acc = fmaf(wv[u].w, xv[u].w, acc);
            }
        }
    }
    return seg_sum<64>(acc);
}

__device__ inline uint32_t order_bits(float v) {
    uint32_t b = __float_as_uint(v);
    if (b == 0x80000000u) b = 0;  // -0 ranks with +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ inline float unorder_bits(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Selection on a candidate set, for E <= 256 (KPL <= 4) and k <= 32.  The
// keys split into 8 groups: key slot m of the lanes of one half-wave.  Every
// group that holds an expert has a largest key, and the smallest of those
// maxima, tau, is a lower bound of the k-th largest key as soon as there are
// at least k such groups (k keys are >= tau).  So every selected key is >= tau,
// and the top-k of the candidates (keys >= tau) is the top-k of all.  The
// candidates (usually a small fraction of E) are packed into one slot each
// of the wave's scratch as 64-bit keys (key, then the complemented expert
// index, so that equal keys rank the lower index first) and each candidate
// counts the candidates above it: its rank.  The candidate of rank j goes to
// lane j.  A wave's LDS accesses complete in order, so no barrier is needed
// between the writes and the reads of its own scratch.  Returns false (the
// caller then takes the k rounds below) when the bound does not apply or there
// are more than 64 candidates.
template <int KPL>
__device__ inline bool topk_candidates(const uint32_t (&val)[KPL], uint32_t avail, int E, int k, int lane,
                                       uint64_t* sc, float& my_logit, int& my_id) {
    if constexpr (KPL > 4) {
        return false;
    } else {
        if (k > 32) return false;
        const int half = lane >> 5;
        uint32_t gm[KPL];
#pragma unroll
        for (int m = 0; m < KPL; m++) gm[m] = ((avail >> m) & 1u) ? val[m] : 0u;
        // the groups' maxima: the max steps of seg_sum<32>, the slots interleaved
#pragma unroll
        for (int m = 0; m < KPL; m++) gm[m] = max(gm[m], (uint32_t)__builtin_amdgcn_update_dpp(0u, gm[m], 0xB1, 0xF, 0xF, false));
#pragma unroll
        for (int m = 0; m < KPL; m++) gm[m] = max(gm[m], (uint32_t)__builtin_amdgcn_update_dpp(0u, gm[m], 0x4E, 0xF, 0xF, false));
#pragma unroll
        for (int m = 0; m < KPL; m++) gm[m] = max(gm[m], (uint32_t)__builtin_amdgcn_update_dpp(0u, gm[m], 0x141, 0xF, 0xF, false));
#pragma unroll
        for (int m = 0; m < KPL; m++) gm[m] = max(gm[m], (uint32_t)__builtin_amdgcn_update_dpp(0u, gm[m], 0x140, 0xF, 0xF, false));
#pragma unroll
        for (int m = 0; m < KPL; m++) {
            const auto r = __builtin_amdgcn_permlane16_swap(gm[m], gm[m], false, false);
            gm[m] = max((uint32_t)r[0], (uint32_t)r[1]);
        }
        // tau over the groups that hold an expert (group (m, h) holds 64 m + 32 h < E)
        uint32_t tmin = 0xFFFFFFFFu;
#pragma unroll
        for (int m = 0; m < KPL; m++) tmin = 64 * m + 32 * half < E ? min(tmin, gm[m]) : tmin;
        const auto r = __builtin_amdgcn_permlane32_swap(tmin, tmin, false, false);
        tmin = min((uint32_t)r[0], (uint32_t)r[1]);
        const int n_groups = min(2 * KPL, (E + 31) / 32);
        const uint32_t tau = n_groups >= k ? tmin : 0u;  // too few groups: every expert is a candidate
        uint64_t B[KPL];
        int base[KPL];
        int C = 0;
#pragma unroll
        for (int m = 0; m < KPL; m++) {
            B[m] = __ballot(((avail >> m) & 1u) && val[m] >= tau);
            base[m] = C;
            C += __popcll(B[m]);
        }
        if (C > 64) return false;
        // slots [0, C): the candidates; [C, 64): zero (above no key); [64, 128): a
        // place for the others' writes
        if (lane >= C) sc[lane] = 0ull;
#pragma unroll
        for (int m = 0; m < KPL; m++) {
            const bool c = (B[m] >> lane) & 1u;
            const int pos = c ? base[m] + lanes_below(B[m]) : 64 + lane;
            sc[pos] = ((uint64_t)val[m] << 32) | (uint32_t)~(uint32_t)(lane + 64 * m);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint64_t mine = sc[min(lane, C - 1)];
        int rank = 0;
        for (int c0 = 0; c0 < C; c0 += 8) {
            uint64_t o[8];
#pragma unroll
            for (int q = 0; q < 8; q++) o[q] = sc[c0 + q];  // (c0 <= 56: slots below 64)
#pragma unroll
            for (int q = 0; q < 8; q++) rank += o[q] > mine ? 1 : 0;
        }
        // the candidate of rank j to lane j (the others to lane 63, unused: k <= 32)
        const int to = 4 * (lane < C && rank < k ? rank : 63);
        const uint64_t sel = ((uint64_t)(uint32_t)__builtin_amdgcn_ds_permute(to, (int)(mine >> 32)) << 32) |
                             (uint32_t)__builtin_amdgcn_ds_permute(to, (int)(uint32_t)mine);
        if (lane < k) {
            my_id = (int)~(uint32_t)sel;
            my_logit = unorder_bits((uint32_t)(sel >> 32));
        }
        return true;
    }
}

// One wave: top-k of one token's E logits (KPL = ceil(E / 64) keys per lane).
// `sc`: 128 64-bit words of LDS for this wave (or null: the rounds only).
template <int KPL>
__device__ inline void topk_wave(const float* l, int E, int k, int norm, int32_t* ids, float* w,
                                 uint64_t* sc = nullptr) {
    const int lane = threadIdx.x & 63;
    // Expert e = lane + 64 m is value val[m] (order-preserving bits) while bit m
    // of avail is set.
    uint32_t val[KPL];
    uint32_t avail = 0;
    float lv[KPL];
#pragma unroll
    for (int m = 0; m < KPL; m++) lv[m] = l[min(lane + 64 * m, E - 1)];  // all loads first
#pragma unroll
    for (int m = 0; m < KPL; m++) {
        const int e = lane + 64 * m;
        val[m] = e < E ? order_bits(lv[m]) : 0u;
        avail |= (e < E ? 1u : 0u) << m;
    }
    float my_logit = 0.f;  // lane j keeps the j-th selected logit
    int my_id = 0;
    if (!sc || !topk_candidates<KPL>(val, avail, E, k, lane, sc, my_logit, my_id)) {
        // k rounds.  Each lane keeps the best of its available values.  A round
        // takes the wave's largest value (one 32-bit DPP max); every lane offers
        // its lowest expert index holding it, and one DPP min picks the lowest
        // of all (ties to the lower index); only the winning lane then
        // recomputes its best.
        auto lane_best = [&]() __attribute__((always_inline)) {
            uint32_t b = 0;
#pragma unroll
            for (int m = 0; m < KPL; m++) b = ((avail >> m) & 1u) ? max(b, val[m]) : b;
            return b;
        };
        uint32_t best = lane_best();
        for (int j = 0; j < k; j++) {
            const uint32_t top = wave_max_u32(best);
            uint32_t cand = 0xFFFFFFFFu;  // 64 m + lane of this lane's lowest m holding top
#pragma unroll
            for (int m = KPL - 1; m >= 0; m--)
                cand = (((avail >> m) & 1u) && val[m] == top) ? (uint32_t)(64 * m + lane) : cand;
            const uint32_t sel = wave_min_u32(cand);
            if (sel != 0xFFFFFFFFu && (int)(sel & 63u) == lane) {  // (some key is always left: k <= E)
                avail &= ~(1u << (sel >> 6));
                best = lane_best();
            }
            if (lane == j) {
                my_id = (int)sel;
                my_logit = unorder_bits(top);
            }
        }
    }
    // the largest selected logit (lane 0), then the softmax in a fixed order
    const float lmax = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(my_logit)));
    float z;
    if (norm) {
        float ex = lane < k ? expf(my_logit - lmax) : 0.f;
        z = seg_sum<64>(ex);
    } else {
        float part = 0.f;
#pragma unroll
        for (int m = 0; m < KPL; m++) {
            const int e = lane + 64 * m;
            if (e < E) part += expf(l[e] - lmax);
        }
        z = seg_sum<64>(part);
    }
    if (lane < k) {
        ids[lane] = my_id;
        w[lane] = expf(my_logit - lmax) / z;
    }
}

// The union of at most 128 assignments (a few tokens' top-k), computed by one
// wave.  Entry i goes to place |{j : e_j < e_i or (e_j == e_i and j < i)}|,
// its place in the stable order by expert, which is the same unique result
// the counting sort gives; each bucket's first entry gives the bucket's
// expert, its first place and its rank among the buckets.
//
// Lane l holds entries l and l + 64.  The relations come bit by bit from the
// expert ids (up to the highest bit any id has; E <= 1024), most significant
// first, one ballot per bit (per word of 64 entries):
// for each of its entries a lane keeps the mask of entries equal so far and
// the mask of those already found smaller.  Every thread of the workgroup
// calls it; the outputs are complete after the caller's next barrier.
__device__ inline void union_small(const int32_t* s_ids, int N, int32_t* n_active, int32_t* experts,
                                   int32_t* offsets, int32_t* entries) {
    const int l = threadIdx.x;
    if (l >= 64) return;
    const bool ok0 = l < N, ok1 = l + 64 < N;
    const int e0 = ok0 ? s_ids[l] : 0, e1 = ok1 ? s_ids[l + 64] : 0;
    const uint64_t V0 = __ballot(ok0), V1 = __ballot(ok1);
    uint64_t q00 = V0, q01 = V1, q10 = V0, q11 = V1;  // equal so far (entry 0: words 0, 1; entry 1)
    uint64_t s00 = 0, s01 = 0, s10 = 0, s11 = 0;      // found smaller
    // only the bits up to the highest set bit of any id matter (ids < 1024)
    const int top_bit = 31 - __builtin_clz(wave_max_u32((uint32_t)(e0 | e1)) | 1u);
    if (N <= 64) {  // one word of entries
        for (int b = top_bit; b >= 0; b--) {
            const uint64_t B0 = __ballot((e0 >> b) & 1);
            if ((e0 >> b) & 1) {
                s00 |= q00 & ~B0; q00 &= B0;
            } else {
                q00 &= ~B0;
            }
        }
    } else {
        for (int b = top_bit; b >= 0; b--) {
            const uint64_t B0 = __ballot((e0 >> b) & 1), B1 = __ballot((e1 >> b) & 1);
            if ((e0 >> b) & 1) {
                s00 |= q00 & ~B0; s01 |= q01 & ~B1; q00 &= B0; q01 &= B1;
            } else {
                q00 &= ~B0; q01 &= ~B1;
            }
            if ((e1 >> b) & 1) {
                s10 |= q10 & ~B0; s11 |= q11 & ~B1; q10 &= B0; q11 &= B1;
            } else {
                q10 &= ~B0; q11 &= ~B1;
            }
        }
    }
    // equal entries before each (entry l: only word 0 lies below it)
    const int eqb0 = lanes_below(q00);
    const int eqb1 = __popcll(q10) + lanes_below(q11);
    const int less0 = __popcll(s00) + __popcll(s01), less1 = __popcll(s10) + __popcll(s11);
    const bool first0 = ok0 && eqb0 == 0, first1 = ok1 && eqb1 == 0;
    const uint64_t F0 = __ballot(first0), F1 = __ballot(first1);
    if (ok0) entries[less0 + eqb0] = l;
    if (ok1) entries[less1 + eqb1] = l + 64;
    if (first0) {
        const int r = __popcll(s00 & F0) + __popcll(s01 & F1);
        experts[r] = e0;
        offsets[r] = less0;
    }
    if (first1) {
        const int r = __popcll(s10 & F0) + __popcll(s11 & F1);
        experts[r] = e1;
        offsets[r] = less1;
    }
    if (l == 0) {
        const int nb = __popcll(F0) + __popcll(F1);
        *n_active = nb;
        offsets[nb] = N;
    }
}

}  // namespace moe
