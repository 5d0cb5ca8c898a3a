/* moe.h — C ABI of the routed mixture-of-experts FFN library (libmoe.so).
 *
 * One routed MoE layer step on an AMD Instinct MI355X (gfx950):
 *   moe_route       router logits, top-k, routing weights
 *   moe_plan_union  expert-major union of the routed tokens
 *   moe_route_union both of the above in one call (fewer launches for <= 4 tokens)
 *   moe_slot_map    host LRU over a bounded pool of expert slots
 *   moe_slot_fill   pinned-host -> slot copy on a side stream + page-table write
 *   moe_slot_stage  moe_slot_map and the fills of its misses in one call
 *   moe_slot_pull   moe_slot_map, then one kernel copies the misses in
 *   moe_route_pull  moe_route_union, then (host waits) moe_slot_pull of its experts
 *   moe_expert_ffn  quantised SwiGLU experts read through the page table,
 *                   shared expert, weighted combine
 *
 * Conventions for every entry point:
 *  - Pointers named "device" are HIP device (or managed) memory; "host" is
 *    ordinary host memory; "pinned" is host memory from hipHostMalloc.  All
 *    buffers belong to the caller and must outlive the work enqueued on them.
 *    The context owns only its page table, error word, workspace and events.
 *  - Streams are hipStream_t values passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously; nothing waits for the GPU unless stated.
 *  - Arguments are validated on the host before anything is enqueued: an
 *    invalid call returns MOE_EINVAL and enqueues nothing.  HIP failures
 *    return MOE_EHIP; moe_last_error() then holds the message.  Nothing
 *    aborts, prints or throws across this boundary.
 *  - Faults found on the device (an unmapped expert, an out-of-range id) set
 *    the context's error word and make the affected output rows quiet NaN;
 *    moe_check() reports them.
 *  - A context is used by one host thread, and its calls are ordered on one
 *    compute stream (plus side streams for fills); two calls that run at the
 *    same time on different streams share its workspace and race.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_ctx moe_ctx;
typedef void* moe_stream; /* hipStream_t */

typedef enum moe_status {
    MOE_OK = 0,
    MOE_EINVAL = -1,   /* invalid argument; nothing was enqueued */
    MOE_ENOMEM = -2,   /* device or host allocation failed */
    MOE_EHIP = -3,     /* HIP runtime error (moe_last_error has the text) */
    MOE_ENOSLOT = -4,  /* a step needs more slots than are free or unpinned */
    MOE_EMISS = -5,    /* a kernel met an unmapped (layer, expert) page-table entry */
    MOE_EBUSY = -6,    /* the slot is pinned by another (layer, expert) */
    MOE_ETIMEOUT = -7  /* a decode workgroup's bounded wait for the hidden rows ran out */
} moe_status;

enum { MOE_Q8_0 = 0, MOE_Q4_0 = 1 };          /* expert weight formats */
enum { MOE_F32 = 0, MOE_BF16 = 1 };           /* activation element types */
enum { MOE_PREC_F32 = 0, MOE_PREC_BF16 = 1 }; /* expert arithmetic modes (see moe_expert_ffn) */
enum { MOE_MAX_STAGE_STREAMS = 8 };           /* side streams one moe_slot_stage call may use */

typedef struct moe_config {
    int32_t n_layers;        /* routed layers sharing the slot pool (>= 1) */
    int32_t n_experts;       /* routed experts per layer, 1..1024 */
    int32_t top_k;           /* experts per token, 1..min(n_experts, 32) */
    int32_t d_model;         /* model width: 128, 256, 512, 1024 or 2048 */
    int32_t d_ff;            /* expert hidden width: a multiple of 128, at most 2048 */
    int32_t qtype;           /* MOE_Q8_0 or MOE_Q4_0 (routed and shared experts) */
    int32_t n_slots;         /* slots in slot_pool (>= 1) */
    int32_t max_tokens;      /* largest T of any call (sizes the workspace), 1..65536 */
    int32_t norm_topk;       /* 1: weights = softmax over the k selected logits;
                                0: weights = full softmax probability of each selected expert */
    int32_t gemm_min_tokens; /* calls of more than 4 tokens, PREC_BF16: buckets with at least
                                this many tokens run in 64-token MFMA tiles, smaller ones in
                                16-token tiles (default 16; 0 = 16) */
    int32_t device;          /* HIP device ordinal; -1 = host-only context (slot
                                bookkeeping only; device entry points return MOE_EINVAL) */
    int32_t reserved;        /* must be 0 */
    void* slot_pool;         /* device, caller-owned, n_slots * moe_payload_bytes() bytes,
                                256-byte aligned; NULL for a host-only context */
} moe_config;

/* Expert-major union ("Nanite for Experts", §5.3: experts are unioned across
 * the tokens of a window and each distinct expert is scheduled once).  All
 * device pointers, caller-owned; sizes from moe_plan_bytes(). */
typedef struct moe_plan {
    int32_t* n_active; /* [1]               number of distinct experts, A */
    int32_t* experts;  /* [n_experts]       experts[0..A) ascending */
    int32_t* offsets;  /* [n_experts + 1]   bucket a = entries[offsets[a] .. offsets[a+1]) */
    int32_t* entries;  /* [max_tokens*top_k] t*top_k + j, ascending within each bucket */
} moe_plan;

/* ---- sizes and formats ------------------------------------------------- */

/* Bytes of one expert's device payload (0 if cfg is invalid).  It equals the
 * expert's GGUF block bytes: 34 (Q8_0) or 18 (Q4_0) bytes per 32 weights of
 * gate [d_ff x d_model], up [d_ff x d_model] and down [d_model x d_ff].
 *
 * Payload layout (how slots hold an expert; "Nanite for Experts", §12 asks
 * for cache geometry chosen with the kernels): the 32-element blocks of each
 * matrix are grouped into tiles of 64 blocks.  Every tile is 16 rows x 4
 * column blocks (block (r, cb) at position 16 * (cb % 4) + r % 16), tiles in
 * order of row group, then column group, so 16 consecutive rows of a matrix
 * are one contiguous run of tiles.  A
 * Q8_0 tile stores the first 16 codes of each of its 64 blocks (64 x 16 B),
 * then the last 16 codes of each (64 x 16 B), then the 64 fp16 scales
 * (2176 B).  A Q4_0 tile stores each block's 16 nibble bytes in GGUF order
 * (64 x 16 B), then the 64 scales (1152 B).  The payload is gate tile 0, up
 * tile 0, gate tile 1, up tile 1, ..., then every down tile in order. */
size_t moe_payload_bytes(const moe_config* cfg);

/* Sizes in bytes of the moe_plan arrays for T tokens:
 * out[0] n_active, out[1] experts, out[2] offsets, out[3] entries. */
moe_status moe_plan_bytes(const moe_config* cfg, int64_t T, size_t out[4]);

/* Host-side repack of one expert between GGUF blocks (gate, up, down, each
 * row-major, blocks along rows: the per-(layer, expert) block of a split pack,
 * "MawForge", §IV-B) and the device payload layout above.  Both buffers are
 * host memory of moe_payload_bytes(cfg) bytes; nothing is enqueued. */
moe_status moe_pack_expert(const moe_config* cfg, const void* gguf_blocks, void* payload);
moe_status moe_unpack_expert(const moe_config* cfg, const void* payload, void* gguf_blocks);

/* ---- context ------------------------------------------------------------ */

/* Validates cfg, then (unless cfg->device == -1) allocates on that device the
 * page table [n_layers x n_experts] int32, every entry -1 (the sentinel for an
 * absent expert, "Nanite for Experts", §5.4), the error word and a workspace
 * for max_tokens.  The slot pool stays the caller's. */
moe_status moe_create(const moe_config* cfg, moe_ctx** out);
/* Waits for the device, frees what moe_create allocated.  NULL is ignored. */
void moe_destroy(moe_ctx* ctx);
/* Text of the last failure on ctx (empty string if none); valid until the next call. */
const char* moe_last_error(const moe_ctx* ctx);
const char* moe_status_string(int status);

/* ---- routing -------------------------------------------------------------- */

/* Router decisions pick the experts; nothing else may change them ("Nanite for
 * Experts", §3.1).  Per token t:
 *   logits[t,e] = sum_i x[t,i] * w_router[e,i]   (fp32, fixed summation order)
 *   ids[t,0..k) = the k largest logits, largest first, ties to the lower expert
 *                 index (+0 and -0 equal)
 *   w[t,j]      = exp(l_j - l_0) / sum_j' exp(l_j' - l_0) over the k selected
 *                 (norm_topk = 1), or over all experts (norm_topk = 0).
 * x: device [T, d_model] fp32 or bf16 (x_dtype).  w_router: device
 * [n_experts, d_model] fp32.  Pass logits_in (device [T, n_experts] fp32, all
 * finite) instead of x and w_router to route precomputed logits.
 * topk_ids: device [T, top_k] int32; topk_w: device [T, top_k] fp32;
 * logits_out: optional device [T, n_experts] fp32 (ignored with logits_in).
 * 0 <= T <= max_tokens. */
moe_status moe_route(moe_ctx* ctx, const void* x, int32_t x_dtype, const float* w_router,
                     const float* logits_in, int64_t T, int32_t* topk_ids, float* topk_w,
                     float* logits_out, moe_stream stream);

/* Expert-major union of topk_ids (device [T, top_k], values in [0, n_experts)):
 * a stable counting sort by expert id into *plan (device, caller-owned).
 * Out-of-range ids set the error word and are dropped. */
moe_status moe_plan_union(moe_ctx* ctx, const int32_t* topk_ids, int64_t T, const moe_plan* plan,
                          moe_stream stream);

/* moe_route followed by moe_plan_union on its topk_ids, with the same arguments
 * and bit-identical results.  The union is the step that turns the tokens'
 * routes into the expert-major set the experts run over ("Nanite for Experts",
 * §5.3); for T <= 4 the top-k and the union run in one single-workgroup launch
 * after the router logits, which saves the launch a decode step would otherwise
 * pay.  Calls on one context must not overlap (they share its logits workspace). */
moe_status moe_route_union(moe_ctx* ctx, const void* x, int32_t x_dtype, const float* w_router,
                           const float* logits_in, int64_t T, int32_t* topk_ids, float* topk_w,
                           float* logits_out, const moe_plan* plan, moe_stream stream);

/* ---- slots and page table ------------------------------------------------- */

/* Bounded expert slots with route-to-slot metadata; a miss materialises the
 * expert into a slot ("MawForge", §IV-C).  Entries stay pinned while their
 * layer is evaluated ("Paging the Experts", §3.2).
 *
 * moe_slot_map: host only, no device work.  experts: host [n], distinct and
 * ascending (e.g. the plan's experts copied back).  Each expert is touched
 * once in that order: a mapped one is a hit; an unmapped one takes the lowest
 * free slot, else the least recently touched slot that is unpinned and holds
 * none of the listed experts (evicted).  Every listed expert is then pinned to
 * `layer` until moe_slot_release(layer).
 * slots_out: host [n]; miss_out: host [n], 1 where the caller must now call
 * moe_slot_fill.  MOE_ENOSLOT (state unchanged) if misses exceed free plus
 * unpinned slots. */
moe_status moe_slot_map(moe_ctx* ctx, int32_t layer, const int32_t* experts, int32_t n,
                        int32_t* slots_out, uint8_t* miss_out);

/* Materialise a missed expert: on `side`, wait until every released reader of
 * the slot and every fill pending on another stream have finished (a pending
 * fill may target the slot being reused), mark the evicted expert's
 * page-table entry absent,
 * copy host_payload (pinned, moe_payload_bytes(), device payload layout) into
 * the slot with hipMemcpyAsync, then write page_table[layer, expert] = slot
 * and record a ready event ("Nanite for Experts", §3.4: asynchronous copies
 * from pinned memory on non-default streams).  The next moe_expert_ffn waits
 * for that event on its own stream.  (layer, expert) must be the slot's owner
 * from moe_slot_map. */
moe_status moe_slot_fill(moe_ctx* ctx, int32_t layer, int32_t expert, int32_t slot,
                         const void* host_payload, moe_stream side);

/* moe_slot_map followed by the fills of its misses, in one call (a miss
 * materialises the expert into its slot, "MawForge", §IV-C; copies from pinned
 * memory on non-default streams, "Nanite for Experts", §3.4).
 * host_payloads: host array of n_experts pointers indexed by expert id, each
 *   to that expert's pinned payload (as for moe_slot_fill); only the entries of
 *   experts that miss are read, the others may be NULL.
 * sides: host array of n_sides (1..MOE_MAX_STAGE_STREAMS) side streams.  Each
 *   stream that receives a copy first waits for every released reader (as in
 *   moe_slot_fill); the misses' copies alternate over the streams in list
 *   order.  Then sides[0] waits for the other streams, writes the page-table
 *   entries of the evicted experts (absent) and of the filled ones (their
 *   slots) in one launch, and records the ready event that the next
 *   moe_expert_ffn waits for.
 * experts, slots_out, miss_out and the mapping are those of moe_slot_map.  A
 * missing expert whose payload pointer is NULL, or a map that moe_slot_map
 * refuses, returns MOE_EINVAL / MOE_ENOSLOT with nothing mapped and nothing
 * enqueued. */
moe_status moe_slot_stage(moe_ctx* ctx, int32_t layer, const int32_t* experts, int32_t n,
                          const void* const* host_payloads, int32_t* slots_out, uint8_t* miss_out,
                          const moe_stream* sides, int32_t n_sides);

/* moe_slot_map, then the misses materialised by the GPU itself ("MawForge",
 * §IV-C: a miss brings the expert into its slot and updates the route-to-slot
 * metadata): kernels on `stream` read each missing expert's payload over the
 * host bus (or from device memory) and write it into its slot, and write the
 * page-table entries of the evicted experts (absent) and of the new ones
 * (their slots).  Work enqueued later on `stream` sees the experts resident
 * without waiting for a copy engine; other streams wait for the ready event
 * recorded on `stream` (moe_expert_ffn does).  Before its first write,
 * `stream` waits for every released reader and for fills still pending on
 * other streams.
 * payloads: host array of n_experts pointers indexed by expert id, each to
 *   that expert's payload (moe_payload_bytes(), device payload layout) in
 *   pinned host memory (hipHostMalloc) or device memory; only the entries of
 *   experts that miss are read, and each must be one of those two kinds, else
 *   MOE_EINVAL with nothing mapped and nothing enqueued.
 * experts, slots_out, miss_out and the mapping are those of moe_slot_map; a
 * refused map changes nothing. */
moe_status moe_slot_pull(moe_ctx* ctx, int32_t layer, const int32_t* experts, int32_t n,
                         const void* const* payloads, int32_t* slots_out, uint8_t* miss_out, moe_stream stream);

/* One demand-staged step of a layer for T <= 4 tokens, with the host in the
 * loop only where the mapping needs it: moe_route_union (same arguments and
 * results) on `stream`, whose union kernel also writes n_active and the
 * experts into the context's pinned memory; the host waits for that (a busy
 * wait on an event), then runs moe_slot_pull of those experts (same arguments
 * and results) on `stream`.  The experts a layer runs with are known only
 * after its routing ("MawForge", §IV-C: a miss materialises the expert into
 * a slot before the layer reads it).
 * n_out (host [1]), experts_out (host [n_experts]): the step's experts,
 * ascending; slots_out, miss_out (host [n_experts]): as moe_slot_map.
 * Blocks the calling thread until the routing is done.  MOE_EINVAL for T
 * outside [1, min(4, max_tokens)], a bad layer or a null argument. */
moe_status moe_route_pull(moe_ctx* ctx, int32_t layer, const void* x, int32_t x_dtype, const float* w_router,
                          const float* logits_in, int64_t T, int32_t* topk_ids, float* topk_w, float* logits_out,
                          const moe_plan* plan, const void* const* payloads, int32_t* n_out, int32_t* experts_out,
                          int32_t* slots_out, uint8_t* miss_out, moe_stream stream);

/* Lookahead staging ahead of demand ("Paging the Experts", §3.3: predicted
 * experts staged while the current layer computes; exact demand outranks
 * prediction).  Host only, no device work.  experts: host [n], distinct, in
 * priority order (e.g. highest routing weight first).  Each is mapped for
 * `layer` WITHOUT pinning: a mapped one is only touched; an unmapped one takes
 * the lowest free slot, else the least recently touched slot that no layer has
 * pinned, while the fills so far stay within max_bytes.  It stops at the first
 * expert that would exceed max_bytes or finds no such slot; *n_done (host)
 * receives how many were processed.  slots_out / fill_out (host [n]): the slot,
 * and 1 where the caller must now call moe_slot_fill (as for a miss).  A
 * prefetched expert that a later moe_slot_map finds counts as a hit and as
 * useful; one evicted before any use counts as wasted.  Demand counters keep
 * their meaning (bytes_staged = misses x payload); prefetch fills also count
 * in moe_stats' fills. */
moe_status moe_slot_prefetch(moe_ctx* ctx, int32_t layer, const int32_t* experts, int32_t n, int64_t max_bytes,
                             int32_t* slots_out, uint8_t* fill_out, int32_t* n_done);

/* Prefetch counters since moe_create: out[0] prefetch fills, out[1] used by a
 * later demand map, out[2] evicted unused, out[3] bytes prefetched. */
moe_status moe_prefetch_stats(const moe_ctx* ctx, uint64_t out[4]);

/* Lookahead for a layer stack, called after moe_route_pull of `layer`: predicts
 * the experts that layer next = (layer + 1) mod n_layers will route and stages
 * the missing ones on `side` while `layer` computes ("Paging the Experts",
 * §3.3: the previous step's highest-weight expert of the same layer at a
 * threshold; "Nanite for Experts", §3.3: staging ahead of need).  Candidates,
 * in this order, each once:
 *   1. the experts that the last moe_route_pull of `next` (the previous step)
 *      selected with weight >= min_weight, highest weight first;
 *   2. if min_transition > 0 and next == layer + 1: the experts e' with
 *      score(e') = sum over this step's entries (e, w) at `layer` of
 *      w * count(e -> e') / count(e -> any) >= min_transition, highest first
 *      (the scores sum to at most 1 over e'), where
 *      count(e -> e') is how often a token that selected e at `layer` selected
 *      e' at `next` in earlier steps (every moe_route_pull of `next` right
 *      after one of `layer` with as many tokens adds one per pair).
 * Candidates without a payload (null entry) are skipped.  A resident candidate
 * is left as it is (not touched); a missing one takes a free slot, else the
 * least recently touched slot that no moe_route_pull of the last n_layers
 * calls touched (a slot idle for a whole step) and no layer has pinned, and is
 * copied as moe_slot_fill copies it, on `side` (its page-table entry is written
 * after the copy; moe_expert_ffn of `next` waits for it).  The staging stops at
 * the first candidate that finds no such slot or would exceed max_bytes of
 * copies.  Counted as moe_slot_prefetch's fills (useful / wasted).
 * payloads: host array of n_experts pointers for layer `next`, each to a
 *   payload in pinned host memory, or null.
 * n_out (host [1]): candidates processed; experts_out (host [n_experts]) and
 *   fill_out (host [n_experts]): those candidates in order, and 1 where a copy
 *   was queued.  Nothing is predicted before the first moe_route_pull.
 * MOE_EINVAL: bad layer, max_bytes < 0, min_weight negative or not finite,
 *   min_transition NaN or infinite, or a null argument, with nothing mapped. */
moe_status moe_prefetch_next(moe_ctx* ctx, int32_t layer, const void* const* payloads, int64_t max_bytes,
                             float min_weight, float min_transition, moe_stream side, int32_t* n_out,
                             int32_t* experts_out, uint8_t* fill_out);

/* Unpin every slot pinned to `layer` and record, on `compute`, the point after
 * which their readers are done (later fills into them wait for it). */
moe_status moe_slot_release(moe_ctx* ctx, int32_t layer, moe_stream compute);

/* Set page_table[layer, expert] = slot (-1 = absent) on `stream`, outside the
 * LRU: the caller placed the payload itself.  MOE_EBUSY if the slot is pinned
 * by another (layer, expert). */
moe_status moe_slot_bind(moe_ctx* ctx, int32_t layer, int32_t expert, int32_t slot,
                         moe_stream stream);

/* ---- expert FFN ------------------------------------------------------------ */

/* For every token t of the step:
 *   y[t] = sum over its routed experts e (ascending e) of w[t,j] * FFN_e(x[t])
 *          + FFN_shared(x[t])
 *   FFN(x) = W_d (silu(W_g x) * (W_u x)),  silu(z) = z / (1 + exp(-z))
 * with each expert read from its slot through page_table[layer, e] and the
 * results merged into the tokens' own rows ("Nanite for Experts", §5.5), one
 * launch over all experts of the step ("Nanite for Experts", §12).  The
 * summation order depends only on expert ids and ranks, never on slots, so y
 * is bitwise identical under any slot assignment.
 * prec MOE_PREC_F32: weights dequantised exactly (d*q in fp32), fp32 hidden
 *   state, fp32 accumulation.
 * prec MOE_PREC_BF16: weights rounded to bf16 after dequantisation, x and the
 *   hidden state rounded to bf16, fp32 accumulation.
 * Calls of more than 4 tokens run every bucket on the matrix cores (bf16 MFMA,
 *   or fp32 MFMA in MOE_PREC_F32) in tiles of 16 tokens, or of 64 for buckets
 *   of at least gemm_min_tokens tokens in MOE_PREC_BF16; up to 4 tokens run
 *   the GEMV.
 * x: device [T, d_model] (x_dtype).  plan: from moe_plan_union on the same
 * topk ids.  topk_w: device [T, top_k] fp32.  shared_payload: device payload
 * of the always-on shared expert ("Nanite for Experts", §1) or NULL.
 * y: device [T, d_model] fp32.  Waits on `stream` for fills not yet awaited.
 * Rows of tokens routed to an unmapped expert become NaN (MOE_EMISS at
 * moe_check). */
moe_status moe_expert_ffn(moe_ctx* ctx, int32_t layer, const void* x, int32_t x_dtype, int64_t T,
                          const moe_plan* plan, const float* topk_w, const void* shared_payload,
                          int32_t prec, float* y, moe_stream stream);

/* Hit/miss split of a one-token step ("Nanite for Experts", §5.5: the experts
 * already resident run while the missing ones are still being copied in, and
 * the results are merged into the token's row).  Call it once after each
 * moe_route_pull, for the same layer and on the same stream (MOE_EINVAL
 * otherwise), with the experts that call copied in (its experts_out where
 * miss_out is 1):
 *   - `side` waits for that call's routing and for fills still pending on
 *     other streams, then runs the resident units (the shared expert too);
 *     x, topk_w and plan must be ready by the end of that routing (written on
 *     its stream before it, or by it);
 *   - `stream`, after the copies moe_route_pull queued on it, waits for
 *     `side` and runs the copied units, then merges.
 * With no miss, or with every unit a miss, or side == stream, it is one
 * launch on `stream`.  Either way
 *   y[t] = sum over the units in plan order, the shared expert last, of
 *          w * (W_d (silu(W_g x) * (W_u x)))
 * with each unit's term computed by the same code whichever launch takes it,
 * so y is bitwise the same for any split of the units (and any slot
 * assignment); it is moe_expert_ffn's result up to summation order, not bit
 * for bit.  Arguments as moe_expert_ffn, with T = 1 and
 * (top_k + 1) * d_ff / 128 <= 40 (every down tile of the step in registers),
 * else MOE_EINVAL.  miss_experts: host [n_miss] expert ids; every expert whose
 * copy may still be in flight must be listed.  Calls on one context must not
 * overlap. */
moe_status moe_expert_ffn_split(moe_ctx* ctx, int32_t layer, const void* x, int32_t x_dtype, int64_t T,
                                const moe_plan* plan, const float* topk_w, const void* shared_payload,
                                int32_t prec, const int32_t* miss_experts, int32_t n_miss, float* y,
                                moe_stream side, moe_stream stream);

/* Bytes of the device array behind moe_expert_ffn_static (one per GPU). */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* moe_expert_ffn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, kernels and results bit for bit, but a call of more
 * than 4 tokens keeps its scratch (hidden rows [T k + T, d_ff], partial rows
 * [T k + T, d_model] fp32, the entry inverse and the tile records) in a
 * fixed device array of MOE_STATIC_SCRATCH_BYTES per GPU that the library
 * holds until the process ends, not in the context's workspace; so T is not
 * limited by max_tokens but by that array: the call needs 256-byte-aligned
 * sections of (T k + T) d_ff (2 bytes in MOE_PREC_BF16, 4 in MOE_PREC_F32)
 * + (T k + T) d_model 4 + T k 4 + 16 bytes per tile record, and returns
 * MOE_EINVAL (nothing enqueued) when that exceeds the array (at d_model
 * 2048, d_ff 512, top-8 with a shared expert: T up to 808 in bf16 mode, 727
 * in fp32 mode).
 * Calls of up to 4 tokens run moe_expert_ffn itself (the decode kernel's
 * workspace belongs to the context, created with it).  Nothing in the call
 * allocates.  Every call on one GPU shares that GPU's array and leaves its
 * contents behind: calls that overlap on one GPU (other contexts, other
 * streams) race.  moe_hidden_rows does not show this call's hidden rows. */
moe_status moe_expert_ffn_static(moe_ctx* ctx, int32_t layer, const void* x, int32_t x_dtype, int64_t T,
                                 const moe_plan* plan, const float* topk_w, const void* shared_payload,
                                 int32_t prec, float* y, moe_stream stream);

/* The whole decode step of up to 4 tokens in ONE launch: moe_route_union and
 * then moe_expert_ffn, with the same results bit for bit ("Nanite for Experts",
 * §12, milestone 1: one expert-major operator for the step; §3.1: the router's
 * choice is authoritative).  Router workgroups compute the logits (from x and
 * w_router, as moe_route; or logits_in [T, n_experts] is taken as given) and
 * hand them to the expert workgroups through the context's workspace; each of
 * those selects the top-k and forms the union itself, and the shared expert's
 * work starts before routing ends.  Every expert the routing picks must already
 * be mapped (moe_slot_map / moe_slot_fill, or moe_slot_bind): one that is not
 * makes its tokens' rows NaN (MOE_EMISS at moe_check).
 * x: device [T, d_model] (x_dtype), also the router's input.  w_router: device
 * [n_experts, d_model] fp32, or NULL with logits_in.  Outputs: topk_ids [T,
 * top_k] int32, topk_w [T, top_k] fp32 and plan, as moe_route_union writes
 * them, and y [T, d_model] fp32 as moe_expert_ffn.  1 <= T <= min(4,
 * max_tokens) and n_experts <= 256, else MOE_EINVAL.  Waits on `stream` for
 * fills not yet awaited.  Calls on one context must not overlap.
 * Co-residency is not needed: workgroups wait only for workgroups of lower
 * index that wait for none of higher index (router rows on the first
 * workgroups, which exit; hidden rows from the gate/up workgroups), and
 * workgroups are dispatched in index order, so kernels running beside it on
 * other streams can delay the launch but not stall it.  If the launch itself
 * fails, the call routes in a launch of its own (moe_route_union) and then
 * runs the experts on that plan: the same results, two launches
 * (moe_route_splits counts such calls). */
moe_status moe_route_ffn(moe_ctx* ctx, int32_t layer, const void* x, int32_t x_dtype, const float* w_router,
                         const float* logits_in, int64_t T, int32_t* topk_ids, float* topk_w,
                         const moe_plan* plan, const void* shared_payload, int32_t prec, float* y,
                         moe_stream stream);

/* ---- inspection ------------------------------------------------------------- */

/* Dequantise one device payload into device out [3 * d_ff * d_model] fp32 in
 * logical order: gate rows, up rows, down rows, each row-major.  prec
 * MOE_PREC_F32 gives d*q exactly; MOE_PREC_BF16 gives it rounded to bf16. */
moe_status moe_dequant(moe_ctx* ctx, const void* payload, int32_t prec, float* out,
                       moe_stream stream);

/* Counters since moe_create: out[0] hits, out[1] misses, out[2] bytes staged
 * (= misses x payload bytes; "Paging the Experts", §4.2), out[3] evictions,
 * out[4] fills enqueued. */
moe_status moe_stats(const moe_ctx* ctx, uint64_t out[5]);

/* Synchronise `stream`, read and clear the error word: MOE_OK, MOE_EMISS,
 * MOE_ETIMEOUT (a decode launch's wait for its gate/up or router workgroups ran
 * out, about 200 ms; its rows are NaN; the counters are reset here), or MOE_EINVAL for an
 * out-of-range expert id met by moe_plan_union. */
moe_status moe_check(moe_ctx* ctx, moe_stream stream);

/* Peak references for measurement (not part of the routed path; no context).
 * moe_probe_read: one launch of `workgroups` workgroups (0: 512) of 512
 * threads, each reading its contiguous share of device src (bytes > 0, a
 * multiple of 16) once with 16-byte loads, 8 in flight per thread; sink:
 * device [1] uint32, written only on a value the caller cannot expect.  The
 * achievable streaming-read rate, to compare the expert kernels' bytes per
 * second with.
 * moe_probe_mfma: grid workgroups of 4 waves, each running iters rounds of
 * independent bf16 matrix-core products: shape % 2 selects the instruction
 * (0: 16x16x32, 1: 32x32x16), shape / 2 the accumulators per wave (0: 4,
 * 1: 8, 2: 16), shape 0..5;
 * *flops (host) receives the floating-point operations performed; sink:
 * device [1] fp32.  Both enqueue on `stream` and return MOE_EINVAL (nothing
 * enqueued) for bad arguments. */
moe_status moe_probe_read(const void* src, int64_t bytes, int32_t workgroups, uint32_t* sink, moe_stream stream);
moe_status moe_probe_mfma(int32_t iters, int32_t grid, int32_t shape, float* sink, int64_t* flops,
                          moe_stream stream);
/* moe_probe_lds: grid workgroups of 4 waves, each lane reading 16 bytes per
 * instruction from local data share memory (no bank conflicts), iters rounds
 * of 8 reads; *bytes (host) receives the bytes read; sink: device [1] uint32. */
moe_status moe_probe_lds(int32_t iters, int32_t grid, uint32_t* sink, int64_t* bytes, moe_stream stream);

/* Calls of moe_route_ffn with router weights since moe_create that took the
 * two-launch path (the one launch failed, or the MOE_SPLIT_ROUTE environment
 * variable was set when the context was created). */
moe_status moe_route_splits(const moe_ctx* ctx, uint64_t* out);

/* Device address of the page table ([n_layers x n_experts] int32), for tests. */
moe_status moe_page_table(const moe_ctx* ctx, int32_t** out);

/* Inspection of the chunk path's hidden state (calls of more than 4 tokens;
 * the SwiGLU hidden state h = silu(W_g x) * (W_u x) is the quantity that
 * MOE_PREC_BF16 rounds to bf16).  *out receives the device address of the
 * context's hidden-row workspace [max_tokens * top_k + max_tokens, d_ff] as
 * the last such moe_expert_ffn left it: row p < T * top_k is plan position p
 * (the entry plan.entries[p]), row T * top_k + t the shared expert on token t,
 * where T is that call's token count.  *elem_bytes receives 2 (bf16, the
 * codes of MOE_PREC_BF16) or 4 (fp32, MOE_PREC_F32) for the last call's mode.
 * Read it after that call completes and before the next one.  MOE_EINVAL for
 * a context whose max_tokens is at most 4 or that has not run such a call. */
moe_status moe_hidden_rows(const moe_ctx* ctx, void** out, int32_t* elem_bytes);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
