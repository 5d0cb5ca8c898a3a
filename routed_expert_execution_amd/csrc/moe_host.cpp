// libmoe host side: context, argument validation, payload packing, the slot
// manager (LRU with per-layer pins), page-table and fill ordering, dispatch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <set>
#include <string>
#include <utility>
#include <vector>

#include "internal.h"

using moe::Geom;

struct moe_ctx {
    moe_config cfg{};
    Geom g;
    bool host_only = true;
    std::string err;

    // device state
    int32_t* pt = nullptr;     // [L x E]
    int* err_word = nullptr;
    float* hbuf = nullptr;     // decode hidden rows
    uint32_t* sync = nullptr;  // decode launch count
    float* split_part = nullptr;  // hit/miss split: the resident units' terms [top_k + 1, d_model]
    hipEvent_t split_ev = nullptr;  // hit/miss split: the resident units' launch is done
    int32_t route_pull_layer = -1;  // layer of the last moe_route_pull (-1: none)

    // prefill workspace (max_tokens > 4)
    float* ph = nullptr;
    float* ppart = nullptr;
    int32_t* pinv = nullptr;
    int32_t* psched = nullptr;  // big tiles, small tiles, wide tiles, 4 counts
    int p_big = 0, p_small = 0, p_wide = 0;
    int wide_min = moe::kWideMinDefault;  // bf16 chunk calls: buckets from which 128-token tiles run
    bool split_route = false;  // moe_route_ffn with router weights: always the two-launch path (tests)
    uint64_t route_splits = 0; // moe_route_ffn calls that took the two-launch path
    int last_prefill_prec = -1; // mode of the last chunk call (-1: none yet)
    float* logits_ws = nullptr;// [max_T * E]
    int* plan_ws = nullptr;    // per-segment expert counts of a large plan (or null)

    // slot manager (host)
    std::vector<int64_t> owner;     // slot -> key = layer*E + expert, or -1
    std::vector<int32_t> slot_of;   // key -> slot, or -1
    std::vector<uint64_t> last;     // recency stamp per slot
    std::vector<int32_t> pin_layer; // layer pinning the slot, or -1
    // The same state indexed for the map's choices, so that a miss costs
    // O(log n_slots) plus the pinned or same-step slots the LRU walk skips,
    // not a pass over every slot: slots are taken lowest first and never
    // freed, so [first_free, n_slots) are the free ones; the owned slots
    // ordered by last touch (stamps are unique); the pinned count and each
    // layer's pinned slots.
    int32_t first_free = 0;
    std::set<std::pair<uint64_t, int32_t>> lru;
    int32_t n_pinned = 0;
    std::vector<std::vector<int32_t>> pinned_of;  // [L]
    std::vector<char> step_hit;                   // [n_slots] scratch of one map call
    std::vector<int64_t> evicted;   // key evicted by the last map of this slot (fill invalidates it)
    std::vector<char> spec;         // slot filled by a prefetch and not yet used by a demand map
    uint64_t clock = 0;
    uint64_t stats[5] = {0, 0, 0, 0, 0};
    uint64_t pstats[4] = {0, 0, 0, 0};  // prefetch fills, useful, wasted, bytes
    // lookahead prediction: moe_route_pull records each layer's last routing
    // and counts, per pair of consecutive layers of one step, which expert of
    // the second followed which of the first; moe_prefetch_next reads them
    std::vector<int32_t> last_ids;  // [L][4 * top_k]
    std::vector<float> last_w;      // [L][4 * top_k]
    std::vector<int32_t> last_n;    // [L] entries recorded (T * top_k; 0: none yet)
    std::vector<uint32_t> trans;    // [L - 1][E][E] (allocated by the first moe_route_pull)
    std::vector<uint64_t> trans_row;  // [L - 1][E] row sums
    int32_t prev_pull_layer = -1;
    std::vector<uint64_t> pull_clock;  // [L] slot clock when each of the last L moe_route_pull calls routed
    int32_t pull_pos = 0;

    // ordering
    int32_t* hmirror = nullptr;       // pinned [1 + E + 2 * 4 * top_k]: n_active, experts, ids and
                                      // weights of the last moe_route_pull
    int32_t* hmirror_dev = nullptr;   // the same memory as kernels address it
    hipEvent_t route_ev = nullptr;    // moe_route_pull: the routing is done
    hipStream_t aux = nullptr;        // prefill: the 64-token tile chain beside the caller's stream
    hipEvent_t fork_ev = nullptr, join_ev = nullptr;
    hipEvent_t release_ev = nullptr;  // last moe_slot_release point on the compute stream
    bool release_recorded = false;
    hipStream_t release_stream = nullptr;  // the stream release_ev was last recorded on
    // One re-recorded event per stream and kind of fill: after copy-engine
    // copies (the default event), or after kernels (moe_slot_pull: kernels of
    // one device fence their own memory, so the event skips the system-scope
    // fence, a cache write-back only the host and other devices would need).
    // A stream's pending fill is the completion mark (below) of its last fill
    // call (mark, gen); ev is the stream's own event for other uses.
    struct Pending { hipStream_t s; hipEvent_t ev; bool pending; bool kern; int32_t mark; uint64_t gen; };
    std::vector<Pending> fills;
    // Completion marks of fill calls: a ring of events, each recorded after one
    // call's writes (payloads and page-table entries); a slot remembers the mark
    // and generation of its last fill, so that a later fill of the slot on
    // another stream waits for exactly that one.  An entry is reused only after
    // its previous recording has completed, so a stale generation means done.
    struct Mark {
        hipEvent_t ev = nullptr, ev_kern = nullptr;  // copy-engine fill, kernel fill (as Pending)
        uint64_t gen = 0;
        hipStream_t s = nullptr;
        bool kern = false;  // which of the two was recorded last
        hipEvent_t last() const { return kern ? ev_kern : ev; }
    };
    std::vector<Mark> marks;
    uint32_t mark_next = 0;
    std::vector<int32_t> slot_mark;   // slot -> mark index, or -1
    std::vector<uint64_t> slot_gen;   // slot -> generation of that mark
};

namespace {

moe_status fail(moe_ctx* c, moe_status st, const char* fmt, ...) __attribute__((format(printf, 3, 4)));
moe_status fail(moe_ctx* c, moe_status st, const char* fmt, ...) {
    if (c) {
        char buf[512];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(buf, sizeof buf, fmt, ap);
        va_end(ap);
        c->err = buf;
    }
    return st;
}

#define HIP_TRY(ctx, call)                                                                   \
    do {                                                                                     \
        hipError_t e_ = (call);                                                              \
        if (e_ != hipSuccess)                                                                \
            return fail((ctx), MOE_EHIP, "%s: %s (%s:%d)", #call, hipGetErrorString(e_),     \
                        __FILE__, __LINE__);                                                 \
    } while (0)

bool cfg_valid(const moe_config* c, Geom* g, std::string* why) {
    auto bad = [&](const char* m) { if (why) *why = m; return false; };
    if (!c) return bad("null config");
    if (c->n_layers < 1) return bad("n_layers must be >= 1");
    if (c->n_experts < 1 || c->n_experts > 1024) return bad("n_experts must be in [1, 1024]");
    if (c->top_k < 1 || c->top_k > c->n_experts || c->top_k > 32) return bad("top_k must be in [1, min(n_experts, 32)]");
    if (c->n_slots < 1) return bad("n_slots must be >= 1");
    if (c->max_tokens < 1 || c->max_tokens > 65536) return bad("max_tokens must be in [1, 65536]");
    if (c->norm_topk != 0 && c->norm_topk != 1) return bad("norm_topk must be 0 or 1");
    if (c->gemm_min_tokens < 0) return bad("gemm_min_tokens must be >= 0");
    if (c->reserved != 0) return bad("reserved must be 0");
    if (c->device < -1) return bad("device must be >= -1");
    if ((int64_t)c->n_layers * c->n_experts > (1 << 26)) return bad("n_layers * n_experts too large");
    Geom gg;
    if (!gg.init(c->d_model, c->d_ff, c->qtype))
        return bad("unsupported shape or qtype: d_model/32 must be a power of two in [4, 64] "
                   "(d_model 128..2048), d_ff a multiple of 128 up to 2048; qtype Q8_0 or Q4_0");
    if (c->device >= 0) {
        if (!c->slot_pool) return bad("slot_pool is NULL");
        if (((uintptr_t)c->slot_pool) & 255) return bad("slot_pool must be 256-byte aligned");
    }
    if (g) *g = gg;
    return true;
}

struct DeviceGuard {
    int prev = -1;
    bool changed = false;
    explicit DeviceGuard(int dev) {
        if (dev >= 0 && hipGetDevice(&prev) == hipSuccess && prev != dev) {
            changed = hipSetDevice(dev) == hipSuccess;
        }
    }
    ~DeviceGuard() { if (changed) (void)hipSetDevice(prev); }
};

moe_status need_device(moe_ctx* c) {
    if (!c) return MOE_EINVAL;
    if (c->host_only) return fail(c, MOE_EINVAL, "host-only context has no device state");
    return MOE_OK;
}

// Q8_0 / Q4_0 repack between GGUF blocks (row-major, blocks along rows) and
// the tile layout.
void repack(const Geom& g, const uint8_t* src, uint8_t* dst, bool to_tiles) {
    const int bb = moe::block_bytes(g.qtype);
    const int64_t mat_gguf = (int64_t)g.f * g.nb_d * bb;  // bytes of gate (= up) in GGUF order
    for (int m = 0; m < 3; m++) {
        const int64_t rows = m < 2 ? g.f : g.d;
        const int nb = m < 2 ? g.nb_d : g.nb_f;
        for (int64_t r = 0; r < rows; r++)
            for (int cb = 0; cb < nb; cb++) {
                int64_t t;
                int i;
                int64_t toff;
                if (m < 2) {
                    g.gu_block(r, cb, &t, &i);
                    toff = m == 0 ? g.gate_tile(t) : g.up_tile(t);
                } else {
                    g.down_block(r, cb, &t, &i);
                    toff = g.down_tile(t);
                }
                const int64_t goff = m * mat_gguf + (r * nb + cb) * bb;
                const uint8_t* gs = src + goff;
                uint8_t* gd = dst + goff;
                if (g.qtype == MOE_Q8_0) {
                    const int off[3] = {moe::q8_scale(i), moe::q8_lo(i), moe::q8_hi(i)};
                    const int len[3] = {2, 16, 16};
                    int gpos = 0;
                    for (int k = 0; k < 3; k++) {
                        if (to_tiles) memcpy(dst + toff + off[k], gs + gpos, len[k]);
                        else memcpy(gd + gpos, src + toff + off[k], len[k]);
                        gpos += len[k];
                    }
                } else {
                    if (to_tiles) {
                        memcpy(dst + toff + moe::q4_scale(i), gs, 2);
                        memcpy(dst + toff + moe::q4_nib(i), gs + 2, 16);
                    } else {
                        memcpy(gd, src + toff + moe::q4_scale(i), 2);
                        memcpy(gd + 2, src + toff + moe::q4_nib(i), 16);
                    }
                }
            }
    }
}

// The address under which a kernel reads p: p itself for device memory, the
// mapped address for pinned host memory; false for anything else (pageable
// host memory, which a kernel cannot read).
bool device_view(const void* p, const void** out) {
    hipPointerAttribute_t at{};
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    if (at.type == hipMemoryTypeDevice) {
        *out = p;
        return true;
    }
    if (at.type == hipMemoryTypeHost && at.devicePointer && at.hostPointer) {
        *out = (const uint8_t*)at.devicePointer + ((const uint8_t*)p - (const uint8_t*)at.hostPointer);
        return true;
    }
    return false;
}

// The re-recorded ready event of stream s for fills of one kind (created on
// first use; kern: fills written by kernels).
unsigned fill_event_flags(bool kern) {
    return kern ? hipEventDisableTiming | hipEventDisableSystemFence : hipEventDisableTiming;
}
moe_status fill_event(moe_ctx* c, hipStream_t s, moe_ctx::Pending** out, bool kern = false) {
    for (auto& q : c->fills)
        if (q.s == s && q.kern == kern) {
            *out = &q;
            return MOE_OK;
        }
    hipEvent_t ev;
    HIP_TRY(c, hipEventCreateWithFlags(&ev, fill_event_flags(kern)));
    c->fills.push_back({s, ev, false, kern, -1, 0});
    *out = &c->fills.back();
    return MOE_OK;
}

constexpr int kMarks = 64;

// Before stream s overwrites the given slots: every released reader has
// finished, and the last fill of each slot, if another stream made it, has
// landed (its copy and its page-table writes).
moe_status order_before_fill(moe_ctx* c, hipStream_t s, const int32_t* slots, const uint8_t* use, int32_t n) {
    if (c->release_recorded && c->release_stream != s) HIP_TRY(c, hipStreamWaitEvent(s, c->release_ev, 0));
    uint64_t waited = 0;  // marks already waited for (kMarks <= 64)
    for (int32_t i = 0; i < n; i++) {
        if (use && !use[i]) continue;
        const int32_t m = c->slot_mark[slots[i]];
        if (m < 0 || c->slot_gen[slots[i]] != c->marks[m].gen || c->marks[m].s == s || (waited >> m & 1)) continue;
        HIP_TRY(c, hipStreamWaitEvent(s, c->marks[m].last(), 0));
        waited |= 1ull << m;
    }
    return MOE_OK;
}

// Records the next mark on s after a fill call's writes (kern: written by
// kernels) and assigns it to the filled slots.
moe_status mark_filled(moe_ctx* c, hipStream_t s, const int32_t* slots, const uint8_t* use, int32_t n,
                       bool kern = false, int32_t* mark_out = nullptr) {
    static_assert(kMarks <= 64, "order_before_fill keeps one bit per mark");
    if (c->marks.empty()) c->marks.resize(kMarks);
    const int32_t m = (int32_t)(c->mark_next++ % kMarks);
    moe_ctx::Mark& k = c->marks[m];
    if (k.gen) HIP_TRY(c, hipEventSynchronize(k.last()));  // its previous fill is done before the entry is reused
    hipEvent_t& ev = kern ? k.ev_kern : k.ev;
    if (!ev) HIP_TRY(c, hipEventCreateWithFlags(&ev, fill_event_flags(kern)));
    HIP_TRY(c, hipEventRecord(ev, s));
    k.kern = kern;
    k.gen++;
    k.s = s;
    for (int32_t i = 0; i < n; i++) {
        if (use && !use[i]) continue;
        c->slot_mark[slots[i]] = m;
        c->slot_gen[slots[i]] = k.gen;
    }
    if (mark_out) *mark_out = m;
    return MOE_OK;
}

// Slot state changes that keep the map's indexes (first_free, lru, n_pinned,
// pinned_of) in step.
void slot_touch(moe_ctx* c, int32_t s, uint64_t stamp) {
    c->lru.erase({c->last[s], s});  // (absent for a slot just taken from the free ones)
    c->last[s] = stamp;
    c->lru.insert({stamp, s});
}
void slot_pin(moe_ctx* c, int32_t s, int32_t layer) {
    if (c->pin_layer[s] < 0) {
        c->n_pinned++;
        c->pinned_of[layer].push_back(s);
    }
    c->pin_layer[s] = layer;  // (a slot's pin is always its key's layer)
}
// The least recently touched owned slot that is unpinned and not a hit of the
// current step (step_hit), touched before `horizon`; -1 if there is none.
int32_t slot_victim(const moe_ctx* c, uint64_t horizon) {
    for (const auto& e : c->lru) {
        if (e.first >= horizon) return -1;
        if (c->pin_layer[e.second] < 0 && !c->step_hit[e.second]) return e.second;
    }
    return -1;
}

// After a fill call's writes on s: one completion mark for the filled slots,
// which also stands for the call as s's pending fill (one event recorded on s,
// not two).
moe_status fill_done(moe_ctx* c, hipStream_t s, const int32_t* slots, const uint8_t* use, int32_t n,
                     bool kern = false) {
    int32_t m = -1;
    if (moe_status st = mark_filled(c, s, slots, use, n, kern, &m)) return st;
    moe_ctx::Pending* p = nullptr;
    if (moe_status st = fill_event(c, s, &p, kern)) return st;
    p->mark = m;
    p->gen = c->marks[m].gen;
    p->pending = true;
    return MOE_OK;
}

// The event a wait for pending fill p needs, or null: its mark has been
// reused, which happens only once the fill it marked has completed.
hipEvent_t pending_event(const moe_ctx* c, const moe_ctx::Pending& p) {
    if (p.mark < 0) return p.ev;
    const moe_ctx::Mark& k = c->marks[p.mark];
    return k.gen == p.gen ? k.last() : nullptr;
}

moe_status wait_pending_fills(moe_ctx* c, hipStream_t s) {
    for (auto& p : c->fills) {
        if (p.pending && p.s != s)
            if (hipEvent_t e = pending_event(c, p)) HIP_TRY(c, hipStreamWaitEvent(s, e, 0));
        p.pending = false;
    }
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int st) {
    switch (st) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument";
        case MOE_ENOMEM: return "out of memory";
        case MOE_EHIP: return "HIP error";
        case MOE_ENOSLOT: return "no free or unpinned slot";
        case MOE_EMISS: return "unmapped expert met by a kernel";
        case MOE_EBUSY: return "slot pinned by another expert";
        case MOE_ETIMEOUT: return "kernel wait timed out";
        default: return "unknown status";
    }
}

size_t moe_payload_bytes(const moe_config* cfg) {
    Geom g;
    if (!cfg || !g.init(cfg->d_model, cfg->d_ff, cfg->qtype)) return 0;
    return (size_t)g.payload;
}

moe_status moe_plan_bytes(const moe_config* cfg, int64_t T, size_t out[4]) {
    if (!cfg || !out || T < 0 || !cfg_valid(cfg, nullptr, nullptr)) return MOE_EINVAL;
    out[0] = sizeof(int32_t);
    out[1] = sizeof(int32_t) * (size_t)cfg->n_experts;
    out[2] = sizeof(int32_t) * ((size_t)cfg->n_experts + 1);
    out[3] = sizeof(int32_t) * (size_t)std::max<int64_t>(1, T * cfg->top_k);
    return MOE_OK;
}

moe_status moe_pack_expert(const moe_config* cfg, const void* gguf_blocks, void* payload) {
    Geom g;
    if (!cfg || !gguf_blocks || !payload || !g.init(cfg->d_model, cfg->d_ff, cfg->qtype)) return MOE_EINVAL;
    repack(g, (const uint8_t*)gguf_blocks, (uint8_t*)payload, true);
    return MOE_OK;
}

moe_status moe_unpack_expert(const moe_config* cfg, const void* payload, void* gguf_blocks) {
    Geom g;
    if (!cfg || !gguf_blocks || !payload || !g.init(cfg->d_model, cfg->d_ff, cfg->qtype)) return MOE_EINVAL;
    repack(g, (const uint8_t*)payload, (uint8_t*)gguf_blocks, false);
    return MOE_OK;
}

void moe_destroy(moe_ctx* c) {
    if (!c) return;
    if (!c->host_only) {
        DeviceGuard dg(c->cfg.device);
        (void)hipDeviceSynchronize();
        if (c->pt) (void)hipFree(c->pt);
        if (c->err_word) (void)hipFree(c->err_word);
        if (c->hbuf) (void)hipFree(c->hbuf);
        if (c->sync) (void)hipFree(c->sync);
        if (c->split_part) (void)hipFree(c->split_part);
        if (c->split_ev) (void)hipEventDestroy(c->split_ev);
        if (c->ph) (void)hipFree(c->ph);
        if (c->ppart) (void)hipFree(c->ppart);
        if (c->pinv) (void)hipFree(c->pinv);
        if (c->psched) (void)hipFree(c->psched);
        if (c->logits_ws) (void)hipFree(c->logits_ws);
        if (c->plan_ws) (void)hipFree(c->plan_ws);
        if (c->release_ev) (void)hipEventDestroy(c->release_ev);
        if (c->fork_ev) (void)hipEventDestroy(c->fork_ev);
        if (c->route_ev) (void)hipEventDestroy(c->route_ev);
        if (c->hmirror) (void)hipHostFree(c->hmirror);
        if (c->join_ev) (void)hipEventDestroy(c->join_ev);
        if (c->aux) (void)hipStreamDestroy(c->aux);
        for (auto& p : c->fills) (void)hipEventDestroy(p.ev);
        for (auto& m : c->marks) {
            if (m.ev) (void)hipEventDestroy(m.ev);
            if (m.ev_kern) (void)hipEventDestroy(m.ev_kern);
        }
    }
    delete c;
}

moe_status moe_create(const moe_config* cfg, moe_ctx** out) {
    if (!out) return MOE_EINVAL;
    *out = nullptr;
    Geom g;
    std::string why;
    if (!cfg_valid(cfg, &g, &why)) return MOE_EINVAL;
    moe_ctx* c = new (std::nothrow) moe_ctx();
    if (!c) return MOE_ENOMEM;
    c->cfg = *cfg;
    if (c->cfg.gemm_min_tokens == 0) c->cfg.gemm_min_tokens = 16;
    c->g = g;
    c->host_only = cfg->device < 0;
    // measurement knob: the bucket size from which bf16 chunk calls use 128-token tiles
    if (const char* e = getenv("MOE_WIDE_MIN_TOKENS")) c->wide_min = std::max(1, atoi(e));
    // test knob: take moe_route_ffn's two-launch path even where the cooperative launch would run
    if (const char* e = getenv("MOE_SPLIT_ROUTE")) c->split_route = atoi(e) != 0;
    const int64_t n_keys = (int64_t)cfg->n_layers * cfg->n_experts;
    c->owner.assign(cfg->n_slots, -1);
    c->slot_of.assign(n_keys, -1);
    c->last.assign(cfg->n_slots, 0);
    c->pin_layer.assign(cfg->n_slots, -1);
    c->pinned_of.assign(cfg->n_layers, {});
    c->step_hit.assign(cfg->n_slots, 0);
    c->evicted.assign(cfg->n_slots, -1);
    c->spec.assign(cfg->n_slots, 0);
    c->slot_mark.assign(cfg->n_slots, -1);
    c->slot_gen.assign(cfg->n_slots, 0);
    if (!c->host_only) {
        DeviceGuard dg(cfg->device);
        auto cleanup = [&](moe_status st) { moe_destroy(c); return st; };
        int ndev = 0;
        if (hipGetDeviceCount(&ndev) != hipSuccess || cfg->device >= ndev) return cleanup(MOE_EINVAL);
        const int64_t T = cfg->max_tokens;
        if (hipMalloc(&c->pt, sizeof(int32_t) * n_keys) != hipSuccess) return cleanup(MOE_ENOMEM);
        if (hipMalloc(&c->err_word, sizeof(int)) != hipSuccess) return cleanup(MOE_ENOMEM);
        if (hipMalloc(&c->hbuf, sizeof(float) * (size_t)moe::decode_h_floats(cfg->top_k, cfg->d_ff, cfg->n_experts, cfg->d_model)) != hipSuccess)
            return cleanup(MOE_ENOMEM);
        if (hipMalloc(&c->sync, sizeof(uint32_t) * moe::kSyncInts) != hipSuccess) return cleanup(MOE_ENOMEM);
        if (hipMalloc(&c->split_part, sizeof(float) * (size_t)moe::split_part_floats(cfg->top_k, cfg->d_model)) !=
            hipSuccess)
            return cleanup(MOE_ENOMEM);
        if (hipMalloc(&c->logits_ws, sizeof(float) * (size_t)T * cfg->n_experts) != hipSuccess)
            return cleanup(MOE_ENOMEM);
        if (const int64_t pw = moe::plan_workspace_ints(T, cfg->top_k, cfg->n_experts))
            if (hipMalloc(&c->plan_ws, sizeof(int) * (size_t)pw) != hipSuccess) return cleanup(MOE_ENOMEM);
        if (T > moe::kDecodeMaxT) {
            const size_t rows = (size_t)(T * cfg->top_k + T);
            moe::prefill_max_tiles(T, cfg->top_k, cfg->n_experts, true, &c->p_big, &c->p_small, &c->p_wide);
            if (hipMalloc(&c->ph, sizeof(float) * rows * cfg->d_ff) != hipSuccess) return cleanup(MOE_ENOMEM);
            if (hipMalloc(&c->ppart, sizeof(float) * rows * cfg->d_model) != hipSuccess) return cleanup(MOE_ENOMEM);
            if (hipMalloc(&c->pinv, sizeof(int32_t) * (size_t)T * cfg->top_k) != hipSuccess) return cleanup(MOE_ENOMEM);
            if (hipMalloc(&c->psched, sizeof(int32_t) * (4 * ((size_t)c->p_big + c->p_small + c->p_wide) + 4)) != hipSuccess)
                return cleanup(MOE_ENOMEM);
        }
        if (hipMemset(c->pt, 0xFF, sizeof(int32_t) * n_keys) != hipSuccess) return cleanup(MOE_EHIP);
        if (hipMemset(c->err_word, 0, sizeof(int)) != hipSuccess) return cleanup(MOE_EHIP);
        if (hipMemset(c->sync, 0, sizeof(uint32_t) * moe::kSyncInts) != hipSuccess) return cleanup(MOE_EHIP);
        if (hipMemset(c->hbuf, 0xFF, sizeof(float) * (size_t)moe::decode_h_floats(cfg->top_k, cfg->d_ff, cfg->n_experts, cfg->d_model)) != hipSuccess)
            return cleanup(MOE_EHIP);
        if (hipEventCreateWithFlags(&c->release_ev, hipEventDisableTiming) != hipSuccess) return cleanup(MOE_EHIP);
        // (they order kernels of one device, which fence their own memory: no
        // system-scope fence)
        if (hipEventCreateWithFlags(&c->split_ev, hipEventDisableTiming | hipEventDisableSystemFence) != hipSuccess)
            return cleanup(MOE_EHIP);
        // (coherent: the union kernel's stores reach host memory, where the
        // host polls the count, without waiting for the kernel's end)
        if (hipHostMalloc((void**)&c->hmirror,
                          sizeof(int32_t) * (size_t)(cfg->n_experts + 1 + 2 * moe::kFusedMaxT * cfg->top_k),
                          hipHostMallocCoherent) !=
                hipSuccess ||
            hipEventCreateWithFlags(&c->route_ev, hipEventDisableTiming) != hipSuccess)
            return cleanup(MOE_EHIP);
        const void* mdev = nullptr;
        if (!device_view(c->hmirror, &mdev)) return cleanup(MOE_EHIP);
        c->hmirror_dev = (int32_t*)mdev;
        // default priority (as every stream of the library); the fork and join
        // order kernels of one device, whose launches fence their own memory,
        // so the events skip the system-scope fence (a cache write-back the
        // host and other devices would need): 5 us less per prefill call
        if (hipStreamCreateWithFlags(&c->aux, hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&c->fork_ev, hipEventDisableTiming | hipEventDisableSystemFence) != hipSuccess ||
            hipEventCreateWithFlags(&c->join_ev, hipEventDisableTiming | hipEventDisableSystemFence) != hipSuccess)
            return cleanup(MOE_EHIP);
        if (hipDeviceSynchronize() != hipSuccess) return cleanup(MOE_EHIP);
    }
    *out = c;
    return MOE_OK;
}

const char* moe_last_error(const moe_ctx* c) { return c ? c->err.c_str() : ""; }

moe_status moe_route(moe_ctx* c, const void* x, int32_t x_dtype, const float* w_router,
                     const float* logits_in, int64_t T, int32_t* topk_ids, float* topk_w,
                     float* logits_out, moe_stream stream) {
    if (moe_status st = need_device(c)) return st;
    const moe_config& cf = c->cfg;
    if (T < 0 || T > cf.max_tokens) return fail(c, MOE_EINVAL, "moe_route: T=%lld outside [0, %d]", (long long)T, cf.max_tokens);
    if (T == 0) return MOE_OK;
    if (!topk_ids || !topk_w) return fail(c, MOE_EINVAL, "moe_route: null output");
    if (!logits_in) {
        if (!x || !w_router) return fail(c, MOE_EINVAL, "moe_route: need logits_in or both x and w_router");
        if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(c, MOE_EINVAL, "moe_route: bad x_dtype");
    }
    DeviceGuard dg(cf.device);
    hipStream_t s = (hipStream_t)stream;
    const float* logits = logits_in;
    if (!logits_in) {
        float* lo = logits_out ? logits_out : c->logits_ws;
        HIP_TRY(c, moe::launch_router_gemv(x, x_dtype == MOE_BF16, w_router, T, cf.n_experts, cf.d_model, lo, s));
        logits = lo;
    }
    HIP_TRY(c, moe::launch_topk(logits, T, cf.n_experts, cf.top_k, cf.norm_topk, topk_ids, topk_w, s));
    return MOE_OK;
}

moe_status moe_plan_union(moe_ctx* c, const int32_t* topk_ids, int64_t T, const moe_plan* plan,
                          moe_stream stream) {
    if (moe_status st = need_device(c)) return st;
    const moe_config& cf = c->cfg;
    if (T < 0 || T > cf.max_tokens) return fail(c, MOE_EINVAL, "moe_plan_union: T outside [0, max_tokens]");
    if (!plan || !plan->n_active || !plan->experts || !plan->offsets || !plan->entries)
        return fail(c, MOE_EINVAL, "moe_plan_union: null plan array");
    if (T > 0 && !topk_ids) return fail(c, MOE_EINVAL, "moe_plan_union: null topk_ids");
    DeviceGuard dg(cf.device);
    HIP_TRY(c, moe::launch_plan(topk_ids, T, cf.top_k, cf.n_experts, *plan, c->err_word, (hipStream_t)stream,
                                c->plan_ws));
    return MOE_OK;
}

moe_status moe_route_union(moe_ctx* c, const void* x, int32_t x_dtype, const float* w_router,
                           const float* logits_in, int64_t T, int32_t* topk_ids, float* topk_w,
                           float* logits_out, const moe_plan* plan, moe_stream stream) {
    if (moe_status st = need_device(c)) return st;
    const moe_config& cf = c->cfg;
    if (T < 0 || T > cf.max_tokens)
        return fail(c, MOE_EINVAL, "moe_route_union: T=%lld outside [0, %d]", (long long)T, cf.max_tokens);
    if (!plan || !plan->n_active || !plan->experts || !plan->offsets || !plan->entries)
        return fail(c, MOE_EINVAL, "moe_route_union: null plan array");
    if (T == 0 || T > moe::kFusedMaxT) {
        if (moe_status st = moe_route(c, x, x_dtype, w_router, logits_in, T, topk_ids, topk_w, logits_out, stream))
            return st;
        return moe_plan_union(c, topk_ids, T, plan, stream);
    }
    if (!topk_ids || !topk_w) return fail(c, MOE_EINVAL, "moe_route_union: null output");
    if (!logits_in) {
        if (!x || !w_router) return fail(c, MOE_EINVAL, "moe_route_union: need logits_in or both x and w_router");
        if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(c, MOE_EINVAL, "moe_route_union: bad x_dtype");
    }
    DeviceGuard dg(cf.device);
    float* lo = logits_out ? logits_out : c->logits_ws;
    HIP_TRY(c, moe::launch_route_union(x, x_dtype == MOE_BF16, w_router, logits_in, T, cf.n_experts, cf.d_model,
                                       cf.top_k, cf.norm_topk, lo, topk_ids, topk_w, *plan, (hipStream_t)stream));
    return MOE_OK;
}

// The routing of the moe_route_pull just done (ids and weights from the pinned
// mirror) as this layer's last, and, when the previous call routed the layer
// before with as many tokens (the same step), one count per (token, earlier
// expert, expert) in that pair of layers' transition table.
static void record_routing(moe_ctx* c, int32_t layer, int T) {
    const moe_config& cf = c->cfg;
    const int E = cf.n_experts, k = cf.top_k, N = T * k, stride = moe::kFusedMaxT * k;
    if (c->last_n.empty()) {
        c->last_ids.assign((size_t)cf.n_layers * stride, 0);
        c->last_w.assign((size_t)cf.n_layers * stride, 0.f);
        c->last_n.assign(cf.n_layers, 0);
        if (cf.n_layers > 1) {
            c->trans.assign((size_t)(cf.n_layers - 1) * E * E, 0u);
            c->trans_row.assign((size_t)(cf.n_layers - 1) * E, 0u);
        }
    }
    const int32_t* ids = c->hmirror + 1 + E;
    const float* w = (const float*)(ids + N);
    int32_t* li = &c->last_ids[(size_t)layer * stride];
    float* lw = &c->last_w[(size_t)layer * stride];
    for (int i = 0; i < N; i++) {
        li[i] = std::min(std::max(ids[i], 0), E - 1);
        lw[i] = w[i];
    }
    c->last_n[layer] = N;
    if (layer > 0 && c->prev_pull_layer == layer - 1 && c->last_n[layer - 1] == N) {
        const int32_t* pi = &c->last_ids[(size_t)(layer - 1) * stride];
        uint32_t* tr = &c->trans[(size_t)(layer - 1) * E * E];
        uint64_t* rs = &c->trans_row[(size_t)(layer - 1) * E];
        for (int t = 0; t < T; t++)
            for (int a = 0; a < k; a++)
                for (int b = 0; b < k; b++) {
                    tr[(size_t)pi[t * k + a] * E + li[t * k + b]]++;
                    rs[pi[t * k + a]]++;
                }
    }
    c->prev_pull_layer = layer;
    // the clock at the start of each of the last n_layers calls (pull_pos: the oldest)
    if (c->pull_clock.empty()) c->pull_clock.assign(cf.n_layers, 0);
    c->pull_clock[c->pull_pos] = c->clock;
    c->pull_pos = (c->pull_pos + 1) % cf.n_layers;
}

moe_status moe_route_pull(moe_ctx* c, int32_t layer, const void* x, int32_t x_dtype, const float* w_router,
                          const float* logits_in, int64_t T, int32_t* topk_ids, float* topk_w, float* logits_out,
                          const moe_plan* plan, const void* const* payloads, int32_t* n_out, int32_t* experts_out,
                          int32_t* slots_out, uint8_t* miss_out, moe_stream stream) {
    if (moe_status st = need_device(c)) return st;
    const moe_config& cf = c->cfg;
    if (T < 1 || T > moe::kFusedMaxT || T > cf.max_tokens)
        return fail(c, MOE_EINVAL, "moe_route_pull: T=%lld outside [1, %d]", (long long)T,
                    std::min(moe::kFusedMaxT, cf.max_tokens));
    if (layer < 0 || layer >= cf.n_layers) return fail(c, MOE_EINVAL, "moe_route_pull: bad layer");
    if (!plan || !plan->n_active || !plan->experts || !plan->offsets || !plan->entries || !topk_ids || !topk_w ||
        !payloads || !n_out || !experts_out || !slots_out || !miss_out)
        return fail(c, MOE_EINVAL, "moe_route_pull: null argument");
    if (!logits_in) {
        if (!x || !w_router) return fail(c, MOE_EINVAL, "moe_route_pull: need logits_in or both x and w_router");
        if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(c, MOE_EINVAL, "moe_route_pull: bad x_dtype");
    }
    DeviceGuard dg(cf.device);
    hipStream_t s = (hipStream_t)stream;
    float* lo = logits_out ? logits_out : c->logits_ws;
    __atomic_store_n(&c->hmirror[0], -1, __ATOMIC_RELEASE);
    HIP_TRY(c, moe::launch_route_union(x, x_dtype == MOE_BF16, w_router, logits_in, T, cf.n_experts, cf.d_model,
                                       cf.top_k, cf.norm_topk, lo, topk_ids, topk_w, *plan, s, c->hmirror_dev));
    HIP_TRY(c, hipEventRecord(c->route_ev, s));
    // The union kernel stores the count last, with system scope, after the
    // experts, ids and weights: the host proceeds when it sees the count,
    // before the kernel has ended.  The event reports a failed launch (and,
    // done with no count seen, a kernel that never wrote it).
    int32_t n = -1;
    for (uint32_t spin = 0;; spin++) {
        n = __atomic_load_n(&c->hmirror[0], __ATOMIC_ACQUIRE);
        if (n != -1) break;
        if ((spin & 255) == 255) {
            const hipError_t q = hipEventQuery(c->route_ev);
            if (q == hipSuccess) {
                n = __atomic_load_n(&c->hmirror[0], __ATOMIC_ACQUIRE);
                break;
            }
            if (q != hipErrorNotReady) HIP_TRY(c, q);
        }
    }
    if (n < 0 || n > cf.n_experts) return fail(c, MOE_EHIP, "moe_route_pull: routing returned %d experts", n);
    std::memcpy(experts_out, c->hmirror + 1, sizeof(int32_t) * (size_t)n);
    *n_out = n;
    record_routing(c, layer, (int)T);
    c->route_pull_layer = -1;
    if (moe_status st = moe_slot_pull(c, layer, experts_out, n, payloads, slots_out, miss_out, stream)) return st;
    c->route_pull_layer = layer;
    return MOE_OK;
}

moe_status moe_slot_map(moe_ctx* c, int32_t layer, const int32_t* experts, int32_t n,
                        int32_t* slots_out, uint8_t* miss_out) {
    if (!c) return MOE_EINVAL;
    const moe_config& cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers) return fail(c, MOE_EINVAL, "moe_slot_map: bad layer");
    if (n < 0 || n > cf.n_experts) return fail(c, MOE_EINVAL, "moe_slot_map: bad n");
    if (n > 0 && (!experts || !slots_out || !miss_out)) return fail(c, MOE_EINVAL, "moe_slot_map: null array");
    for (int32_t i = 0; i < n; i++) {
        if (experts[i] < 0 || experts[i] >= cf.n_experts) return fail(c, MOE_EINVAL, "moe_slot_map: expert id out of range");
        if (i && experts[i] <= experts[i - 1]) return fail(c, MOE_EINVAL, "moe_slot_map: experts must be ascending and distinct");
    }
    const int64_t base = (int64_t)layer * cf.n_experts;
    // capacity check first, so a refused step changes nothing: the slots
    // neither pinned nor holding one of this step's experts
    int need = 0, unpinned_hits = 0;
    for (int32_t i = 0; i < n; i++) {
        int32_t s = c->slot_of[base + experts[i]];
        if (s < 0) need++;
        else {
            c->step_hit[s] = 1;
            unpinned_hits += c->pin_layer[s] < 0;
        }
    }
    const int avail = cf.n_slots - c->n_pinned - unpinned_hits;
    auto clear_hits = [&]() {
        for (int32_t i = 0; i < n; i++) {
            const int32_t s = c->slot_of[base + experts[i]];
            if (s >= 0) c->step_hit[s] = 0;
        }
    };
    if (need > avail) {
        clear_hits();
        return fail(c, MOE_ENOSLOT, "moe_slot_map: %d misses but %d free or unpinned slots", need, avail);
    }
    for (int32_t i = 0; i < n; i++) {
        const int64_t key = base + experts[i];
        c->clock++;
        int32_t s = c->slot_of[key];
        if (s >= 0) {
            c->stats[0]++;
            miss_out[i] = 0;
            if (c->spec[s]) {  // a prefetch that demand now uses
                c->pstats[1]++;
                c->spec[s] = 0;
            }
        } else {
            int32_t pick = c->first_free < cf.n_slots ? c->first_free++ : -1;  // the lowest free slot
            if (pick < 0) {  // never a slot holding one of this step's experts
                pick = slot_victim(c, UINT64_MAX);
                c->slot_of[c->owner[pick]] = -1;
                c->evicted[pick] = c->owner[pick];
                c->stats[3]++;
                if (c->spec[pick]) {  // a prefetch evicted before any use
                    c->pstats[2]++;
                    c->spec[pick] = 0;
                }
            } else {
                c->evicted[pick] = -1;
            }
            s = pick;
            c->owner[s] = key;
            c->slot_of[key] = s;
            c->stats[1]++;
            c->stats[2] += (uint64_t)c->g.payload;
            miss_out[i] = 1;
        }
        slot_touch(c, s, c->clock);
        slot_pin(c, s, layer);
        slots_out[i] = s;
    }
    clear_hits();
    return MOE_OK;
}

// The mapping of moe_slot_prefetch (arguments already checked).
static void prefetch_map(moe_ctx* c, int32_t layer, const int32_t* experts, int32_t n, int64_t max_bytes,
                         int32_t* slots_out, uint8_t* fill_out, int32_t* n_done, uint64_t horizon = UINT64_MAX);

moe_status moe_slot_prefetch(moe_ctx* c, int32_t layer, const int32_t* experts, int32_t n, int64_t max_bytes,
                             int32_t* slots_out, uint8_t* fill_out, int32_t* n_done) {
    if (!c) return MOE_EINVAL;
    const moe_config& cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers) return fail(c, MOE_EINVAL, "moe_slot_prefetch: bad layer");
    if (n < 0 || n > cf.n_experts || max_bytes < 0) return fail(c, MOE_EINVAL, "moe_slot_prefetch: bad n or max_bytes");
    if (!n_done || (n > 0 && (!experts || !slots_out || !fill_out)))
        return fail(c, MOE_EINVAL, "moe_slot_prefetch: null array");
    for (int32_t i = 0; i < n; i++) {
        if (experts[i] < 0 || experts[i] >= cf.n_experts) return fail(c, MOE_EINVAL, "moe_slot_prefetch: expert id out of range");
        for (int32_t j = 0; j < i; j++)
            if (experts[j] == experts[i]) return fail(c, MOE_EINVAL, "moe_slot_prefetch: experts must be distinct");
    }
    prefetch_map(c, layer, experts, n, max_bytes, slots_out, fill_out, n_done);
    return MOE_OK;
}

// horizon: a victim must not have been touched at or after this clock value.
static void prefetch_map(moe_ctx* c, int32_t layer, const int32_t* experts, int32_t n, int64_t max_bytes,
                         int32_t* slots_out, uint8_t* fill_out, int32_t* n_done, uint64_t horizon) {
    const moe_config& cf = c->cfg;
    const int64_t base = (int64_t)layer * cf.n_experts;
    int64_t bytes = 0;
    int32_t done = 0;
    for (; done < n; done++) {
        const int64_t key = base + experts[done];
        int32_t s = c->slot_of[key];
        if (s < 0) {
            if (bytes + c->g.payload > max_bytes) break;
            // a free slot, else the least recently touched unpinned one; never one
            // that a layer in flight has pinned (demand outranks prediction)
            int32_t pick = c->first_free < cf.n_slots ? c->first_free++ : -1;
            if (pick < 0) {
                pick = slot_victim(c, horizon);
                if (pick < 0) break;
                c->slot_of[c->owner[pick]] = -1;
                c->evicted[pick] = c->owner[pick];
                c->stats[3]++;
                if (c->spec[pick]) c->pstats[2]++;
            } else {
                c->evicted[pick] = -1;
            }
            s = pick;
            c->owner[s] = key;
            c->slot_of[key] = s;
            c->spec[s] = 1;
            c->pstats[0]++;
            c->pstats[3] += (uint64_t)c->g.payload;
            bytes += c->g.payload;
            fill_out[done] = 1;
        } else {
            fill_out[done] = 0;
            if (horizon != UINT64_MAX) {  // moe_prefetch_next: a resident prediction keeps its place
                slots_out[done] = s;
                continue;
            }
        }
        slot_touch(c, s, ++c->clock);  // predicted: kept until the demand that should follow
        slots_out[done] = s;
    }
    *n_done = done;
}

moe_status moe_prefetch_next(moe_ctx* c, int32_t layer, const void* const* payloads, int64_t max_bytes,
                             float min_weight, float min_transition, moe_stream side, int32_t* n_out,
                             int32_t* experts_out, uint8_t* fill_out) {
    if (moe_status st = need_device(c)) return st;
    const moe_config& cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers) return fail(c, MOE_EINVAL, "moe_prefetch_next: bad layer");
    if (max_bytes < 0 || !(min_weight >= 0.f) || !(min_weight < 1e30f) || !(min_transition < 1e30f) ||
        min_transition != min_transition)
        return fail(c, MOE_EINVAL, "moe_prefetch_next: bad max_bytes, min_weight or min_transition");
    if (!payloads || !n_out || !experts_out || !fill_out) return fail(c, MOE_EINVAL, "moe_prefetch_next: null argument");
    *n_out = 0;
    if (c->last_n.empty()) return MOE_OK;  // nothing routed yet
    const int E = cf.n_experts, k = cf.top_k, stride = moe::kFusedMaxT * k;
    const int32_t next = (layer + 1) % cf.n_layers;
    // candidate -> score; the previous step's routing of `next` first (its
    // weights), then transitions from this step's experts of `layer`
    std::vector<std::pair<float, int32_t>> prev, trans;
    std::vector<char> taken(E, 0);
    {
        const int N = c->last_n[next];
        const int32_t* ids = &c->last_ids[(size_t)next * stride];
        const float* w = &c->last_w[(size_t)next * stride];
        std::vector<float> best(E, -1.f);
        for (int i = 0; i < N; i++) best[ids[i]] = std::max(best[ids[i]], w[i]);
        for (int e = 0; e < E; e++)
            if (best[e] >= min_weight && best[e] >= 0.f) prev.push_back({best[e], e});
    }
    if (min_transition > 0.f && next == layer + 1 && c->last_n[layer] > 0 && !c->trans.empty()) {
        const int N = c->last_n[layer];
        const int32_t* ids = &c->last_ids[(size_t)layer * stride];
        const float* w = &c->last_w[(size_t)layer * stride];
        const uint32_t* tr = &c->trans[(size_t)layer * E * E];
        const uint64_t* rs = &c->trans_row[(size_t)layer * E];
        std::vector<double> score(E, 0.0);
        for (int i = 0; i < N; i++) {
            const uint64_t tot = rs[ids[i]];
            if (!tot) continue;
            const uint32_t* row = tr + (size_t)ids[i] * E;
            for (int e = 0; e < E; e++)
                if (row[e]) score[e] += (double)w[i] * row[e] / (double)tot;
        }
        for (int e = 0; e < E; e++)
            if (score[e] >= min_transition) trans.push_back({(float)score[e], e});
    }
    auto by_score = [](const std::pair<float, int32_t>& a, const std::pair<float, int32_t>& b) {
        return a.first != b.first ? a.first > b.first : a.second < b.second;
    };
    std::sort(prev.begin(), prev.end(), by_score);
    std::sort(trans.begin(), trans.end(), by_score);
    std::vector<int32_t> pred;
    for (auto& q : prev) if (!taken[q.second] && payloads[q.second]) { taken[q.second] = 1; pred.push_back(q.second); }
    for (auto& q : trans) if (!taken[q.second] && payloads[q.second]) { taken[q.second] = 1; pred.push_back(q.second); }
    std::vector<int32_t> slots(pred.size());
    int32_t done = 0;
    // Victims: only slots untouched for a whole step (the last n_layers
    // moe_route_pull calls), which the next step would not use either; a
    // prediction that needs any other stops the staging.  A prediction already
    // resident is left where it is in the recency order.  (Evicting the least
    // recently touched slot regardless, or touching resident predictions, cost
    // a pool of one step's experts most of its hits: each moved another layer's
    // expert of the step to the front of the eviction order.)
    const uint64_t horizon = c->pull_clock.empty() ? 0 : c->pull_clock[c->pull_pos];
    prefetch_map(c, next, pred.data(), (int32_t)pred.size(), max_bytes, slots.data(), fill_out, &done, horizon);
    for (int32_t i = 0; i < done; i++) {
        experts_out[i] = pred[i];
        if (fill_out[i])
            if (moe_status st = moe_slot_fill(c, next, pred[i], slots[i], payloads[pred[i]], side)) return st;
    }
    *n_out = done;
    return MOE_OK;
}

moe_status moe_prefetch_stats(const moe_ctx* c, uint64_t out[4]) {
    if (!c || !out) return MOE_EINVAL;
    for (int i = 0; i < 4; i++) out[i] = c->pstats[i];
    return MOE_OK;
}

moe_status moe_slot_fill(moe_ctx* c, int32_t layer, int32_t expert, int32_t slot,
                         const void* host_payload, moe_stream side) {
    if (moe_status st = need_device(c)) return st;
    const moe_config& cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers || expert < 0 || expert >= cf.n_experts || slot < 0 || slot >= cf.n_slots)
        return fail(c, MOE_EINVAL, "moe_slot_fill: index out of range");
    if (!host_payload) return fail(c, MOE_EINVAL, "moe_slot_fill: null payload");
    const int64_t key = (int64_t)layer * cf.n_experts + expert;
    if (c->owner[slot] != key) return fail(c, MOE_EINVAL, "moe_slot_fill: slot %d is not mapped to (layer %d, expert %d)", slot, layer, expert);
    DeviceGuard dg(cf.device);
    hipStream_t s = (hipStream_t)side;
    if (moe_status st = order_before_fill(c, s, &slot, nullptr, 1)) return st;
    if (c->evicted[slot] >= 0) {
        HIP_TRY(c, hipMemsetD32Async((hipDeviceptr_t)(c->pt + c->evicted[slot]), -1, 1, s));
        c->evicted[slot] = -1;
    }
    uint8_t* dst = (uint8_t*)cf.slot_pool + (size_t)slot * (size_t)c->g.payload;
    HIP_TRY(c, hipMemcpyAsync(dst, host_payload, (size_t)c->g.payload, hipMemcpyDefault, s));
    HIP_TRY(c, hipMemsetD32Async((hipDeviceptr_t)(c->pt + key), slot, 1, s));
    if (moe_status st = fill_done(c, s, &slot, nullptr, 1)) return st;
    c->stats[4]++;
    return MOE_OK;
}

moe_status moe_slot_stage(moe_ctx* c, int32_t layer, const int32_t* experts, int32_t n,
                          const void* const* host_payloads, int32_t* slots_out, uint8_t* miss_out,
                          const moe_stream* sides, int32_t n_sides) {
    if (moe_status st = need_device(c)) return st;
    const moe_config& cf = c->cfg;
    if (!host_payloads || !sides || n_sides < 1 || n_sides > MOE_MAX_STAGE_STREAMS)
        return fail(c, MOE_EINVAL, "moe_slot_stage: null payload table or stream list, or n_sides not in 1..%d",
                    MOE_MAX_STAGE_STREAMS);
    if ((int64_t)cf.n_layers * cf.n_experts > INT32_MAX) return fail(c, MOE_EINVAL, "moe_slot_stage: page table too large");
    if (layer >= 0 && layer < cf.n_layers && n > 0 && experts) {
        // a miss without a payload is refused before anything is mapped
        const int64_t base = (int64_t)layer * cf.n_experts;
        for (int32_t i = 0; i < n; i++)
            if (experts[i] >= 0 && experts[i] < cf.n_experts && c->slot_of[base + experts[i]] < 0 &&
                !host_payloads[experts[i]])
                return fail(c, MOE_EINVAL, "moe_slot_stage: expert %d misses but has no payload", experts[i]);
    }
    if (moe_status st = moe_slot_map(c, layer, experts, n, slots_out, miss_out)) return st;
    int n_miss = 0;
    for (int32_t i = 0; i < n; i++) n_miss += miss_out[i];
    if (!n_miss) return MOE_OK;
    DeviceGuard dg(cf.device);
    const int used = std::min<int>(n_sides, n_miss);
    for (int j = 0; j < used; j++)
        if (moe_status st = order_before_fill(c, (hipStream_t)sides[j], slots_out, miss_out, n)) return st;
    const int64_t base = (int64_t)layer * cf.n_experts;
    int q = 0;
    for (int32_t i = 0; i < n; i++) {
        if (!miss_out[i]) continue;
        uint8_t* dst = (uint8_t*)cf.slot_pool + (size_t)slots_out[i] * (size_t)c->g.payload;
        HIP_TRY(c, hipMemcpyAsync(dst, host_payloads[experts[i]], (size_t)c->g.payload, hipMemcpyHostToDevice,
                                  (hipStream_t)sides[q++ % used]));
    }
    hipStream_t s0 = (hipStream_t)sides[0];
    for (int j = 1; j < used; j++) {  // the first stream writes the page table after every copy
        moe_ctx::Pending* p = nullptr;
        if (moe_status st = fill_event(c, (hipStream_t)sides[j], &p)) return st;
        HIP_TRY(c, hipEventRecord(p->ev, (hipStream_t)sides[j]));
        HIP_TRY(c, hipStreamWaitEvent(s0, p->ev, 0));
    }
    moe::PtWrites w{};
    auto put = [&](int64_t idx, int32_t val) -> moe_status {
        if (w.n == moe::kPtBatch) {
            HIP_TRY(c, moe::launch_pt_write(c->pt, w, s0));
            w.n = 0;
        }
        w.idx[w.n] = (int32_t)idx;
        w.val[w.n++] = val;
        return MOE_OK;
    };
    for (int32_t i = 0; i < n; i++) {
        if (!miss_out[i]) continue;
        const int32_t sl = slots_out[i];
        if (c->evicted[sl] >= 0) {
            if (moe_status st = put(c->evicted[sl], -1)) return st;
            c->evicted[sl] = -1;
        }
        if (moe_status st = put(base + experts[i], sl)) return st;
    }
    HIP_TRY(c, moe::launch_pt_write(c->pt, w, s0));
    if (moe_status st = fill_done(c, s0, slots_out, miss_out, n)) return st;
    c->stats[4] += (uint64_t)n_miss;
    return MOE_OK;
}

moe_status moe_slot_pull(moe_ctx* c, int32_t layer, const int32_t* experts, int32_t n,
                         const void* const* payloads, int32_t* slots_out, uint8_t* miss_out, moe_stream stream) {
    if (moe_status st = need_device(c)) return st;
    const moe_config& cf = c->cfg;
    if (!payloads) return fail(c, MOE_EINVAL, "moe_slot_pull: null payload table");
    if ((int64_t)cf.n_layers * cf.n_experts > INT32_MAX || c->g.payload % 16 ||
        (uint64_t)moe::kPullMax * (c->g.payload / 16) > 0x7FFFFFFFull)
        return fail(c, MOE_EINVAL, "moe_slot_pull: page table or payload size out of range");
    // every payload a miss will read must be addressable by a kernel; checked
    // before anything is mapped
    std::vector<const uint4*> src(std::max<int32_t>(n, 0), nullptr);
    if (layer >= 0 && layer < cf.n_layers && n > 0 && n <= cf.n_experts && experts) {
        const int64_t base = (int64_t)layer * cf.n_experts;
        for (int32_t i = 0; i < n; i++) {
            const int32_t e = experts[i];
            if (e < 0 || e >= cf.n_experts || c->slot_of[base + e] >= 0) continue;
            const void* dv = nullptr;
            if (!payloads[e] || !device_view(payloads[e], &dv))
                return fail(c, MOE_EINVAL, "moe_slot_pull: payload of expert %d is not pinned host or device memory", e);
            src[i] = (const uint4*)dv;
        }
    }
    if (moe_status st = moe_slot_map(c, layer, experts, n, slots_out, miss_out)) return st;
    int n_miss = 0;
    for (int32_t i = 0; i < n; i++) n_miss += miss_out[i];
    if (!n_miss) return MOE_OK;
    DeviceGuard dg(cf.device);
    hipStream_t s = (hipStream_t)stream;
    if (moe_status st = order_before_fill(c, s, slots_out, miss_out, n)) return st;
    const int64_t base = (int64_t)layer * cf.n_experts;
    moe::PullArgs a{};
    moe::PtWrites w{};
    a.words = (uint32_t)(c->g.payload / 16);
    auto flush = [&]() -> moe_status {
        HIP_TRY(c, moe::launch_pull(a, c->pt, w, s));
        a.n = 0;
        w.n = 0;
        return MOE_OK;
    };
    for (int32_t i = 0; i < n; i++) {
        if (!miss_out[i]) continue;
        const int32_t sl = slots_out[i];
        a.src[a.n] = src[i];
        a.dst[a.n++] = (uint4*)((uint8_t*)cf.slot_pool + (size_t)sl * (size_t)c->g.payload);
        if (c->evicted[sl] >= 0) {
            w.idx[w.n] = (int32_t)c->evicted[sl];
            w.val[w.n++] = -1;
            c->evicted[sl] = -1;
        }
        w.idx[w.n] = (int32_t)(base + experts[i]);
        w.val[w.n++] = sl;
        if (a.n == moe::kPullMax)
            if (moe_status st = flush()) return st;
    }
    if (a.n)
        if (moe_status st = flush()) return st;
    if (moe_status st = fill_done(c, s, slots_out, miss_out, n, true)) return st;
    c->stats[4] += (uint64_t)n_miss;
    return MOE_OK;
}

moe_status moe_slot_release(moe_ctx* c, int32_t layer, moe_stream compute) {
    if (!c) return MOE_EINVAL;
    const moe_config& cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers) return fail(c, MOE_EINVAL, "moe_slot_release: bad layer");
    for (const int32_t s : c->pinned_of[layer])
        if (c->pin_layer[s] == layer) {
            c->pin_layer[s] = -1;
            c->n_pinned--;
        }
    c->pinned_of[layer].clear();
    if (!c->host_only) {
        DeviceGuard dg(cf.device);
        HIP_TRY(c, hipEventRecord(c->release_ev, (hipStream_t)compute));
        c->release_recorded = true;
        c->release_stream = (hipStream_t)compute;
    }
    return MOE_OK;
}

moe_status moe_slot_bind(moe_ctx* c, int32_t layer, int32_t expert, int32_t slot, moe_stream stream) {
    if (moe_status st = need_device(c)) return st;
    const moe_config& cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers || expert < 0 || expert >= cf.n_experts || slot < -1 || slot >= cf.n_slots)
        return fail(c, MOE_EINVAL, "moe_slot_bind: index out of range");
    const int64_t key = (int64_t)layer * cf.n_experts + expert;
    if (slot >= 0 && c->pin_layer[slot] >= 0 && c->owner[slot] != key)
        return fail(c, MOE_EBUSY, "moe_slot_bind: slot %d is pinned by another expert", slot);
    DeviceGuard dg(cf.device);
    HIP_TRY(c, hipMemsetD32Async((hipDeviceptr_t)(c->pt + key), slot, 1, (hipStream_t)stream));
    return MOE_OK;
}

// Arguments of the expert kernels common to every call.
static moe::FfnArgs ffn_args(moe_ctx* c, int32_t layer, const void* x, int32_t x_dtype, int64_t T,
                             const moe_plan* plan, const float* topk_w, const void* shared_payload, float* y) {
    const moe_config& cf = c->cfg;
    moe::FfnArgs a{};
    a.pool = (const uint8_t*)cf.slot_pool;
    a.payload_bytes = c->g.payload;
    a.pt = c->pt;
    a.layer = layer;
    a.E = cf.n_experts;
    a.n_slots = cf.n_slots;
    a.shared = (const uint8_t*)shared_payload;
    a.n_active = plan->n_active;
    a.experts = plan->experts;
    a.offsets = plan->offsets;
    a.entries = plan->entries;
    a.topk_w = topk_w;
    a.k = cf.top_k;
    a.x = x;
    a.x_bf16 = x_dtype == MOE_BF16;
    a.T = (int)T;
    a.route = moe::kRoutePlan;
    a.norm = cf.norm_topk;
    a.hbuf = c->hbuf;
    a.sync = c->sync;
    // bound of the decode kernel's waits: 200 ms of the 100 MHz clock; tests of the
    // time-out path set MOE_SYNC_WAIT_TICKS (a negative value: every wait gives up
    // at its first check, whatever has arrived)
    a.wait_ticks = 20000000;
    if (const char* e = getenv("MOE_SYNC_WAIT_TICKS")) a.wait_ticks = std::max<int64_t>(-1, atoll(e));
    a.y = y;
    a.err = c->err_word;
    return a;
}

// Arguments of the chunk path's kernels, workspace pointers aside.
static moe::PrefillArgs prefill_args(moe_ctx* c, const moe::FfnArgs& a, int32_t layer, const void* x, int64_t T,
                                     const float* topk_w, float* y) {
    const moe_config& cf = c->cfg;
    moe::PrefillArgs p{};
    p.g = c->g;
    p.pool = a.pool;
    p.payload_bytes = a.payload_bytes;
    p.pt = a.pt;
    p.layer = layer;
    p.E = cf.n_experts;
    p.n_slots = cf.n_slots;
    p.shared = a.shared;
    p.n_active = a.n_active;
    p.experts = a.experts;
    p.offsets = a.offsets;
    p.entries = a.entries;
    p.topk_w = topk_w;
    p.k = cf.top_k;
    p.x = x;
    p.x_bf16 = a.x_bf16;
    p.T = (int)T;
    p.d = cf.d_model;
    p.f = cf.d_ff;
    p.gemm_min = cf.gemm_min_tokens;
    p.wide_min = c->wide_min;
    p.y = y;
    p.err = c->err_word;
    return p;
}

static moe_status ffn_check_args(moe_ctx* c, const char* fn, int32_t layer, const void* x, int32_t x_dtype,
                                 int64_t T, int64_t T_max, const moe_plan* plan, const float* topk_w, int32_t prec,
                                 float* y) {
    const moe_config& cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers) return fail(c, MOE_EINVAL, "%s: bad layer", fn);
    if (T < 0 || T > T_max) return fail(c, MOE_EINVAL, "%s: T=%lld outside [0, %lld]", fn, (long long)T, (long long)T_max);
    if (prec != MOE_PREC_F32 && prec != MOE_PREC_BF16) return fail(c, MOE_EINVAL, "%s: bad prec", fn);
    if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(c, MOE_EINVAL, "%s: bad x_dtype", fn);
    if (T > 0 && (!x || !plan || !plan->n_active || !plan->experts || !plan->offsets || !plan->entries || !topk_w || !y))
        return fail(c, MOE_EINVAL, "%s: null argument", fn);
    return MOE_OK;
}

moe_status moe_expert_ffn(moe_ctx* c, int32_t layer, const void* x, int32_t x_dtype, int64_t T,
                          const moe_plan* plan, const float* topk_w, const void* shared_payload,
                          int32_t prec, float* y, moe_stream stream) {
    if (moe_status st = need_device(c)) return st;
    const moe_config& cf = c->cfg;
    if (moe_status st = ffn_check_args(c, "moe_expert_ffn", layer, x, x_dtype, T, cf.max_tokens, plan, topk_w, prec, y))
        return st;
    DeviceGuard dg(cf.device);
    hipStream_t s = (hipStream_t)stream;
    if (moe_status st = wait_pending_fills(c, s)) return st;
    if (T == 0) return MOE_OK;
    moe::FfnArgs a = ffn_args(c, layer, x, x_dtype, T, plan, topk_w, shared_payload, y);
    if (T <= moe::kDecodeMaxT) {
        HIP_TRY(c, moe::launch_ffn_decode(c->g, a, prec, s));
        return MOE_OK;
    }
    moe::PrefillArgs p = prefill_args(c, a, layer, x, T, topk_w, y);
    p.h = c->ph;
    p.part = c->ppart;
    p.inv = c->pinv;
    p.sched_big = c->psched;
    p.sched_small = c->psched + 4 * (size_t)c->p_big;
    p.sched_wide = p.sched_small + 4 * (size_t)c->p_small;
    p.n_tiles = p.sched_wide + 4 * (size_t)c->p_wide;
    p.cap_big = c->p_big;
    p.cap_small = c->p_small;
    p.cap_wide = c->p_wide;
    HIP_TRY(c, moe::launch_ffn_prefill(p, prec, moe::PrefillStreams{s, c->aux, c->fork_ev, c->join_ev}));
    c->last_prefill_prec = prec;
    return MOE_OK;
}

moe_status moe_expert_ffn_split(moe_ctx* c, int32_t layer, const void* x, int32_t x_dtype, int64_t T,
                                const moe_plan* plan, const float* topk_w, const void* shared_payload,
                                int32_t prec, const int32_t* miss_experts, int32_t n_miss, float* y,
                                moe_stream side, moe_stream stream) {
    if (moe_status st = need_device(c)) return st;
    const moe_config& cf = c->cfg;
    if (moe_status st = ffn_check_args(c, "moe_expert_ffn_split", layer, x, x_dtype, T, 1, plan, topk_w, prec, y))
        return st;
    if (T != 1) return fail(c, MOE_EINVAL, "moe_expert_ffn_split: T must be 1");
    if (layer != c->route_pull_layer)
        return fail(c, MOE_EINVAL, "moe_expert_ffn_split: layer %d is not that of a moe_route_pull not yet split",
                    layer);
    if (n_miss < 0 || n_miss > cf.n_experts || (n_miss > 0 && !miss_experts))
        return fail(c, MOE_EINVAL, "moe_expert_ffn_split: bad miss list");
    if ((int64_t)(std::min(cf.top_k, cf.n_experts) + 1) * (cf.d_ff / 128) > moe::kSplitMaxTiles)
        return fail(c, MOE_EINVAL, "moe_expert_ffn_split: (top_k + 1) * d_ff / 128 exceeds %d", moe::kSplitMaxTiles);
    moe::SplitSel sel{};
    for (int32_t i = 0; i < n_miss; i++) {
        const int32_t e = miss_experts[i];
        if (e < 0 || e >= cf.n_experts) return fail(c, MOE_EINVAL, "moe_expert_ffn_split: expert id out of range");
        sel.miss[e >> 5] |= 1u << (e & 31);
    }
    sel.part = c->split_part;
    DeviceGuard dg(cf.device);
    hipStream_t s = (hipStream_t)stream, sd = (hipStream_t)side;
    moe::FfnArgs a = ffn_args(c, layer, x, x_dtype, T, plan, topk_w, shared_payload, y);
    // Units the step takes: its routed experts (at most top_k) and the shared one.
    if (n_miss > 0 && n_miss < cf.top_k + (shared_payload ? 1 : 0) && sd != s) {
        // The resident units on `side` as soon as the routing is done (which
        // follows the context's earlier work on `stream`, the last split's
        // launches among it: launches of the decode kernel never overlap, as
        // they share the context's workspace); the fills still pending on
        // other streams first (copies the routing does not follow), not the
        // copies `stream` received after the routing.
        HIP_TRY(c, hipStreamWaitEvent(sd, c->route_ev, 0));
        for (auto& p : c->fills)
            if (p.pending && p.s != s && p.s != sd)
                if (hipEvent_t e = pending_event(c, p)) HIP_TRY(c, hipStreamWaitEvent(sd, e, 0));
        sel.which = moe::kSplitHits;
        HIP_TRY(c, moe::launch_ffn_split(c->g, a, prec, sel, sd));
        HIP_TRY(c, hipEventRecord(c->split_ev, sd));
        if (moe_status st = wait_pending_fills(c, s)) return st;
        HIP_TRY(c, hipStreamWaitEvent(s, c->split_ev, 0));
        sel.which = moe::kSplitMisses;
    } else {
        // every unit resident, or every routed one copied in: one launch after the copies
        if (moe_status st = wait_pending_fills(c, s)) return st;
        sel.which = moe::kSplitAll;
    }
    HIP_TRY(c, moe::launch_ffn_split(c->g, a, prec, sel, s));
    c->route_pull_layer = -1;  // one split per moe_route_pull
    return MOE_OK;
}

moe_status moe_expert_ffn_static(moe_ctx* c, int32_t layer, const void* x, int32_t x_dtype, int64_t T,
                                 const moe_plan* plan, const float* topk_w, const void* shared_payload,
                                 int32_t prec, float* y, moe_stream stream) {
    if (moe_status st = need_device(c)) return st;
    const moe_config& cf = c->cfg;
    if (T >= 0 && T <= moe::kDecodeMaxT)  // the decode kernel, on the context's own workspace
        return moe_expert_ffn(c, layer, x, x_dtype, T, plan, topk_w, shared_payload, prec, y, stream);
    if (moe_status st = ffn_check_args(c, "moe_expert_ffn_static", layer, x, x_dtype, T, 65536, plan, topk_w, prec, y))
        return st;
    const moe::PrefillLayout L = moe::prefill_layout(T, cf.top_k, cf.n_experts, cf.d_model, cf.d_ff,
                                                     prec == MOE_PREC_BF16);
    if (L.total > moe::kStaticScratchBytes)
        return fail(c, MOE_EINVAL, "moe_expert_ffn_static: T=%lld needs %zu bytes of scratch; the static array holds %zu",
                    (long long)T, L.total, moe::kStaticScratchBytes);
    DeviceGuard dg(cf.device);
    void* base = nullptr;
    HIP_TRY(c, moe::static_scratch(&base));
    hipStream_t s = (hipStream_t)stream;
    if (moe_status st = wait_pending_fills(c, s)) return st;
    moe::FfnArgs a = ffn_args(c, layer, x, x_dtype, T, plan, topk_w, shared_payload, y);
    moe::PrefillArgs p = prefill_args(c, a, layer, x, T, topk_w, y);
    uint8_t* b = (uint8_t*)base;
    p.h = b + L.h;
    p.part = (float*)(b + L.part);
    p.inv = (int32_t*)(b + L.inv);
    p.sched_big = (int32_t*)(b + L.sched_big);
    p.sched_small = (int32_t*)(b + L.sched_small);
    p.sched_wide = (int32_t*)(b + L.sched_wide);
    p.n_tiles = (int32_t*)(b + L.n_tiles);
    p.cap_big = L.cap_big;
    p.cap_small = L.cap_small;
    p.cap_wide = L.cap_wide;
    HIP_TRY(c, moe::launch_ffn_prefill(p, prec, moe::PrefillStreams{s, c->aux, c->fork_ev, c->join_ev}));
    return MOE_OK;
}

moe_status moe_route_ffn(moe_ctx* c, int32_t layer, const void* x, int32_t x_dtype, const float* w_router,
                         const float* logits_in, int64_t T, int32_t* topk_ids, float* topk_w, const moe_plan* plan,
                         const void* shared_payload, int32_t prec, float* y, moe_stream stream) {
    if (moe_status st = need_device(c)) return st;
    const moe_config& cf = c->cfg;
    if (layer < 0 || layer >= cf.n_layers) return fail(c, MOE_EINVAL, "moe_route_ffn: bad layer");
    if (T < 1 || T > moe::kDecodeMaxT || T > cf.max_tokens)
        return fail(c, MOE_EINVAL, "moe_route_ffn: T=%lld outside [1, min(4, max_tokens)]", (long long)T);
    if (cf.n_experts > 256) return fail(c, MOE_EINVAL, "moe_route_ffn: more than 256 experts (route separately)");
    if (prec != MOE_PREC_F32 && prec != MOE_PREC_BF16) return fail(c, MOE_EINVAL, "moe_route_ffn: bad prec");
    if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return fail(c, MOE_EINVAL, "moe_route_ffn: bad x_dtype");
    if (!x || !topk_ids || !topk_w || !y || !plan || !plan->n_active || !plan->experts || !plan->offsets ||
        !plan->entries)
        return fail(c, MOE_EINVAL, "moe_route_ffn: null argument");
    if (!logits_in && !w_router) return fail(c, MOE_EINVAL, "moe_route_ffn: need logits_in or w_router");
    DeviceGuard dg(cf.device);
    hipStream_t s = (hipStream_t)stream;
    if (moe_status st = wait_pending_fills(c, s)) return st;
    moe::FfnArgs a = ffn_args(c, layer, x, x_dtype, T, plan, topk_w, shared_payload, y);
    a.route = logits_in ? moe::kRouteLogits : moe::kRouteRouter;
    a.logits_in = logits_in;
    a.w_router = w_router;
    a.ids_out = topk_ids;
    a.w_out = topk_w;
    a.o_n_active = plan->n_active;
    a.o_experts = plan->experts;
    a.o_offsets = plan->offsets;
    a.o_entries = plan->entries;
    if (a.route == moe::kRouteRouter && !c->split_route) {
        const hipError_t e = moe::launch_ffn_decode(c->g, a, prec, s);
        if (e == hipSuccess) return MOE_OK;
        (void)hipGetLastError();  // a refused cooperative launch enqueued nothing
    } else if (a.route != moe::kRouteRouter) {
        HIP_TRY(c, moe::launch_ffn_decode(c->g, a, prec, s));
        return MOE_OK;
    }
    // The router's logits in a launch of their own (with the top-k and the
    // union), then the experts on that plan: the same results bit for bit,
    // with no wait between workgroups of the routing.
    c->route_splits++;
    if (moe_status st = moe_route_union(c, x, x_dtype, w_router, nullptr, T, topk_ids, topk_w, nullptr, plan, stream))
        return st;
    moe::FfnArgs b = ffn_args(c, layer, x, x_dtype, T, plan, topk_w, shared_payload, y);
    HIP_TRY(c, moe::launch_ffn_decode(c->g, b, prec, s));
    return MOE_OK;
}

moe_status moe_route_splits(const moe_ctx* c, uint64_t* out) {
    if (!c || !out) return MOE_EINVAL;
    *out = c->route_splits;
    return MOE_OK;
}

moe_status moe_dequant(moe_ctx* c, const void* payload, int32_t prec, float* out, moe_stream stream) {
    if (moe_status st = need_device(c)) return st;
    if (!payload || !out) return fail(c, MOE_EINVAL, "moe_dequant: null argument");
    if (prec != MOE_PREC_F32 && prec != MOE_PREC_BF16) return fail(c, MOE_EINVAL, "moe_dequant: bad prec");
    DeviceGuard dg(c->cfg.device);
    HIP_TRY(c, moe::launch_dequant(c->g, (const uint8_t*)payload, prec, out, (hipStream_t)stream));
    return MOE_OK;
}

moe_status moe_stats(const moe_ctx* c, uint64_t out[5]) {
    if (!c || !out) return MOE_EINVAL;
    for (int i = 0; i < 5; i++) out[i] = c->stats[i];
    return MOE_OK;
}

moe_status moe_check(moe_ctx* c, moe_stream stream) {
    if (moe_status st = need_device(c)) return st;
    DeviceGuard dg(c->cfg.device);
    hipStream_t s = (hipStream_t)stream;
    HIP_TRY(c, hipStreamSynchronize(s));
    int w = 0;
    HIP_TRY(c, hipMemcpy(&w, c->err_word, sizeof(int), hipMemcpyDeviceToHost));
    if (!w) return MOE_OK;
    HIP_TRY(c, hipMemset(c->err_word, 0, sizeof(int)));
    if (w & moe::kErrSync) {
        // after a timed-out wait the workspace halves may hold rows of the wrong
        // launch: start both afresh (pending) with the count at zero
        HIP_TRY(c, hipMemset(c->sync, 0, sizeof(uint32_t) * moe::kSyncInts));
        HIP_TRY(c, hipMemset(c->hbuf, 0xFF, sizeof(float) * (size_t)moe::decode_h_floats(c->cfg.top_k, c->cfg.d_ff, c->cfg.n_experts, c->cfg.d_model)));
        HIP_TRY(c, hipDeviceSynchronize());
        return fail(c, MOE_ETIMEOUT, "a decode workgroup timed out waiting for the hidden rows or the logits (error word 0x%x)", w);
    }
    if (w & moe::kErrMiss) return fail(c, MOE_EMISS, "a kernel met an unmapped expert (error word 0x%x)", w);
    return fail(c, MOE_EINVAL, "a plan input held an expert id out of range (error word 0x%x)", w);
}

moe_status moe_probe_read(const void* src, int64_t bytes, int32_t workgroups, uint32_t* sink, moe_stream stream) {
    if (!src || !sink || bytes <= 0 || bytes % 16 || workgroups < 0) return MOE_EINVAL;
    const void* dsrc = nullptr;
    if (!device_view(src, &dsrc)) return MOE_EINVAL;
    return moe::launch_probe_read(dsrc, bytes, workgroups, sink, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_EHIP;
}

moe_status moe_probe_mfma(int32_t iters, int32_t grid, int32_t shape, float* sink, int64_t* flops, moe_stream stream) {
    if (iters < 1 || grid < 1 || shape < 0 || shape > 5 || !sink || !flops) return MOE_EINVAL;
    *flops = moe::probe_mfma_flops(iters, grid, shape);
    return moe::launch_probe_mfma(iters, grid, shape, sink, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_EHIP;
}

moe_status moe_probe_lds(int32_t iters, int32_t grid, uint32_t* sink, int64_t* bytes, moe_stream stream) {
    if (iters < 1 || grid < 1 || !sink || !bytes) return MOE_EINVAL;
    *bytes = (int64_t)grid * 256 * 8 * 16 * iters;
    return moe::launch_probe_lds(iters, grid, sink, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_EHIP;
}

moe_status moe_page_table(const moe_ctx* c, int32_t** out) {
    if (!c || !out || c->host_only) return MOE_EINVAL;
    *out = c->pt;
    return MOE_OK;
}

moe_status moe_hidden_rows(const moe_ctx* c, void** out, int32_t* elem_bytes) {
    if (!c || !out || !elem_bytes || c->host_only || !c->ph || c->last_prefill_prec < 0) return MOE_EINVAL;
    *out = c->ph;
    *elem_bytes = c->last_prefill_prec == MOE_PREC_BF16 ? 2 : 4;
    return MOE_OK;
}

}  // extern "C"
