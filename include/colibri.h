/*
 * colibri.h -- C ABI of the MI355X (gfx950) MoE-layer library libcolibri.so.
 *
 * One mixture-of-experts layer forward on one GPU, in five steps:
 *   1. sigmoid router with a selection bias (DeepSeek-V3 style noaux_tc),
 *      top-k, renormalised weights times routed_scaling_factor;
 *   2. batched-union dispatch: the (token, slot) pairs are grouped by expert,
 *      so every expert present in the batch is read once for all its tokens;
 *   3. gated expert FFN (gate and up projections, SiLU, down projection) over
 *      packed int8 / int4 / int2 weights with per-row scales, multiplied on an
 *      integer dot-product path against Q8_0-style int8 activations;
 *   4. an always-on shared expert;
 *   5. the routing-weighted combine.
 *
 * Sources (web pages on the colibri runtime):
 *   [README] "Show HN: 如何在我的低配置电脑上运行 GLM-5.2" (translation of the
 *            colibri README), section "已实现的功能" (implemented features):
 *            sigmoid-router item, integer dot-product item (Q8_0-style int8
 *            activations), quantised-kernel item (int8 / packed int4 / packed
 *            int2, per-row scales, dequantised on use), batched-union MoE
 *            item; section "实验性 Metal 后端" (routed-expert SwiGLU); section
 *            "资源策略" (gate and up projections share one dispatch).
 *   [DIVE]   "colibrì 深度拆解" (deep dive), section 4.3 (shared expert plus
 *            routing-weighted sum of the selected experts) and section 5.1
 *            (int4 container, first element in the high nibble, per-row scale).
 *
 * Conventions for every call
 *   - Every pointer argument except the descriptor structs is DEVICE memory
 *     owned by the caller.  The library allocates nothing, frees nothing and
 *     keeps no pointer after a call returns.  Descriptor structs are host
 *     memory read during the call only.  (The tiered-residency objects at the
 *     end of this header are the exception; their section says what they
 *     own, keep and wait for.)
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  No call outside the tiered-residency section
 *     synchronises the host or copies to the host.
 *   - Scratch memory is the caller's workspace `ws` of `ws_bytes` bytes,
 *     256-byte aligned, sized by colibri_workspace_bytes().  Concurrent calls
 *     need distinct workspaces; workspace contents need no initialisation.
 *   - Arguments are validated before anything is enqueued: a call that returns
 *     an error has no device side effects.  A device fault surfaces at the
 *     caller's next synchronisation.  There is no CPU fallback.
 *   - Data preconditions that are documented but not checked: activations are
 *     finite, int8 weight codes lie in [-127, 127] (packed codes use their
 *     whole range), router weights and biases are finite, routed ids handed
 *     to colibri_moe_dispatch lie in [0, E).
 */
#ifndef COLIBRI_H
#define COLIBRI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t* coli_stream_t;

/* Status codes. */
enum {
    COLI_OK = 0,
    COLI_E_INVAL = 1,       /* null pointer, negative size, bad dimension, k > E, ... */
    COLI_E_UNSUPPORTED = 2, /* qtype, misaligned pointer, size beyond a limit below */
    COLI_E_WORKSPACE = 3,   /* ws_bytes smaller than colibri_workspace_bytes() */
    COLI_E_HIP = 4,         /* the HIP runtime reported an error at launch */
    COLI_E_SCRATCH = 5      /* colibri_moe_layer_forward_noalloc: the batch's workspace
                               exceeds COLI_NOALLOC_SCRATCH_BYTES */
};

/* Weight element width of a bank ([README] quantised-kernel item). */
enum { COLI_Q8 = 8, COLI_Q4 = 4, COLI_Q2 = 2 };

/* Limits checked by every call. */
#define COLI_MAX_EXPERTS 1024
#define COLI_MAX_TOPK 64
#define COLI_MAX_TOKENS 65536
#define COLI_MAX_PAIRS (1 << 20) /* S * top_k */
#define COLI_MAX_DIM 8192        /* hidden and inter */

/*
 * A bank of n_mat quantised matrices, each [rows][K] row-major, one fp32 scale
 * per row ([DIVE] 5.1), or with group > 0 one fp32 scale per `group`
 * consecutive columns of a row (group-wise scales: [README]'s
 * quality-benchmark paragraph names them as the likely priority).  Row r of
 * matrix m starts at byte (m*rows + r) * K * qtype / 8 of `data`; its scale is
 * row_scale[m*rows + r], or with groups its scales are row_scale[(m*rows + r)
 * * (K/group) + j] for column groups j = 0 .. K/group - 1.
 *   COLI_Q8: one two's-complement byte per weight.
 *   COLI_Q4: byte j of a row holds element 2j in bits 7..4 and element 2j+1 in
 *            bits 3..0, two's-complement nibbles in [-8, 7].
 *   COLI_Q2: byte j holds elements 4j..4j+3 in bits 7..6, 5..4, 3..2, 1..0,
 *            two's-complement values in [-2, 1].
 * Requirements: K % 32 == 0, rows >= 1, n_mat >= 1, `data` 16-byte aligned,
 * `row_scale` 4-byte aligned; group 0 or a multiple of 32 that divides K.
 */
typedef struct coli_qbank {
    const void* data;
    const float* row_scale;
    int32_t n_mat, rows, K;
    int32_t qtype; /* COLI_Q8, COLI_Q4 or COLI_Q2 */
    int32_t group; /* columns per scale; 0: one scale per row */
} coli_qbank;

/*
 * One layer.  gate/up: n_mat = n_experts, rows = inter, K = hidden; down:
 * n_mat = n_experts, rows = hidden, K = inter.  gate and up share a qtype and
 * a group.
 * The shared expert (has_shared != 0) has the same shapes with n_mat = 1.
 * router_w is fp32 [n_experts][hidden]; router_bias fp32 [n_experts] enters
 * expert selection only.  hidden % 32 == 0 and inter % 32 == 0.
 *
 * Router variants (zero-initialised fields, or n_group = topk_group = 1 and
 * top_p = 1, give the plain top-k of the sigmoid-router item):
 *   n_group > 1: group-limited selection, the group stage of DeepSeek-V3's
 *     noaux_tc routing.  Experts form n_group equal contiguous groups; a
 *     group's score is the sum of its two largest biased scores (fp32); the
 *     topk_group best groups are kept (ties to the lower group); the top-k
 *     runs over the kept groups' experts.  Requires n_experts % n_group == 0,
 *     n_experts / n_group >= 2, 1 <= topk_group <= n_group and
 *     top_k <= topk_group * n_experts / n_group.
 *   0 < top_p < 1: adaptive expert top-p ([README] practical-flags list:
 *     fewer expert reads per token).  The k selected slots are ordered by
 *     unbiased score (descending, ties in slot order); their shares s / sum s
 *     are accumulated in fp32 and the shortest prefix whose cumulative share
 *     reaches top_p is kept (at least one slot).  Kept slots keep their
 *     positions and weights rsf * s_j / sum over kept s; dropped slots get id
 *     -1 and weight 0 and are not computed.
 */
typedef struct coli_moe_layer {
    int32_t hidden, inter, n_experts, top_k;
    float routed_scaling_factor;
    const float* router_w;
    const float* router_bias;
    coli_qbank gate, up, down;
    int32_t has_shared;
    coli_qbank sh_gate, sh_up, sh_down;
    int32_t n_group;    /* 0 or 1: no group stage */
    int32_t topk_group; /* groups kept when n_group > 1 */
    float top_p;        /* 0 or >= 1: no top-p */
} coli_moe_layer;

/* Workspace bytes that every call below needs for layer L and up to S tokens
 * (0 if L is invalid). */
size_t colibri_workspace_bytes(const coli_moe_layer* L, int32_t S);

/* Workspace bytes colibri_expert_ffn_q needs for these banks, S tokens and k
 * pairs per token (0 if the banks are invalid). */
size_t colibri_expert_ffn_workspace_bytes(const coli_qbank* gate, const coli_qbank* down,
                                          int32_t S, int32_t k);

/*
 * Q8_0-style quantisation ([README] integer dot-product item) of x [rows][K]
 * fp32 (K % 32 == 0, 16-byte aligned): for every 32-element block, amax =
 * max |v|, d = amax / 127 (IEEE fp32 division), codes = clamp(round half away
 * from zero (v * (1/d)), -127, 127), with d = 0 and codes 0 for an all-zero
 * block.  Writes q [rows][K] int8 (16-byte aligned) and d [rows][K/32] fp32.
 * rows == 0 is a no-op.
 */
int colibri_quantize_q8_0(const float* x, int32_t rows, int32_t K, int8_t* q, float* d,
                          coli_stream_t stream);

/*
 * Router ([README] sigmoid-router item).  x: fp32 [S][hidden].  For each token:
 * logits l_e = x . router_w[e] (fp32), s_e = 1 / (1 + exp(-l_e)),
 * c_e = s_e + router_bias[e]; the top_k experts by c (ties to the lower id;
 * with n_group > 1 among the kept groups' experts) fill slots in that order;
 * topk_w[t][j] = routed_scaling_factor * s_(j) / sum_j' s_(j') from the
 * unbiased scores (with top_p, over the kept slots; dropped slots: id -1,
 * weight 0).  Writes topk_ids int32 [S][top_k] and topk_w fp32 [S][top_k].
 * S == 0 is a no-op.
 */
int colibri_route(const coli_moe_layer* L, const float* x, int32_t S, int32_t* topk_ids,
                  float* topk_w, void* ws, size_t ws_bytes, coli_stream_t stream);

/*
 * Batched-union dispatch ([README] batched-union MoE item).  Pairs p = t*k + j
 * of topk_ids [S][k] are stably grouped by expert id in [0, E); a negative id
 * (a slot dropped by top-p) is no pair and is left out of every output:
 *   expert_offsets int32 [E+1]: exclusive prefix of the per-expert counts;
 *   sorted_pairs   int32 [S*k]: pair indices ordered by (expert, p);
 *   active_experts int32 [E]  : experts with count > 0, ascending (entries
 *                               past *n_active are left untouched);
 *   n_active       int32 [1]  : their number (device memory).
 * Deterministic (no data-dependent atomics on positions).  S == 0 writes zero
 * offsets and *n_active = 0.
 */
int colibri_moe_dispatch(const int32_t* topk_ids, int32_t S, int32_t k, int32_t E,
                         int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* active_experts,
                         int32_t* n_active, void* ws, size_t ws_bytes, coli_stream_t stream);

/*
 * Gated expert FFN on the integer dot path ([README] integer dot-product and
 * quantised-kernel items; Metal section: SwiGLU; resource-policy section: gate
 * and up in one dispatch).  For every sorted position i < expert_offsets[n_mat]
 * with pair p = sorted_pairs[i], token t = p / k, expert e (the one whose
 * offset range holds i):
 *   g[r] = gate.row_scale[e][r] * F(gate row (e, r), xq[t], xd[t])   (r < I)
 *   u[r] likewise with up;  h[r] = silu(g[r]) * u[r];  h -> Q8_0 (hq, hd)
 *   y[i][n] = down.row_scale[e][n] * F(down row (e, n), hq, hd)       (n < H)
 * where F folds the exact int32 block partials S_b = sum over 32 elements of
 * weight code * activation code in one chain, acc = fmaf(d_b, (float)S_b,
 * acc) from +0 for b = 0 .. K/32 - 1 in ascending order (the pages leave the
 * order of the fp32 accumulation open; the sum as written is taken, and it
 * is the same in every kernel, so results are bit-exact across batch sizes
 * and kernels).  With group-wise scales s (bank group > 0)
 * block b's coefficient is the fp32 product s[32b/group] * d_b in place of
 * d_b, and the row-scale factor is absent.  silu(g) = g / (1 + exp(-g)) with exp by Cody-Waite
 * reduction and a degree-7 Taylor polynomial (+inf above 88, +0 below -87).
 * xq int8 [S][hidden] and xd fp32 [S][hidden/32] come from
 * colibri_quantize_q8_0; offsets / pairs from colibri_moe_dispatch (or, for a
 * one-matrix bank, {0, S} and the identity with k = 1).  Writes y fp32
 * [S*k][hidden] in sorted order (16-byte aligned); rows from
 * expert_offsets[n_mat] <= S*k on (fewer when slots were dropped) are left
 * untouched.
 */
int colibri_expert_ffn_q(const coli_qbank* gate, const coli_qbank* up, const coli_qbank* down,
                         const int8_t* xq, const float* xd, int32_t S,
                         const int32_t* expert_offsets, const int32_t* sorted_pairs, int32_t k,
                         float* y, void* ws, size_t ws_bytes, coli_stream_t stream);

/*
 * Whole layer ([DIVE] 4.3): out[t] = y_shared[t] + sum_j topk_w[t][j] *
 * y_routed[t][j] (fp32, slot order, dropped slots skipped), with the steps
 * above.  x and out are fp32
 * [S][hidden], 16-byte aligned.  S == 0 is a no-op.
 */
int colibri_moe_layer_forward(const coli_moe_layer* L, const float* x, int32_t S, float* out,
                              void* ws, size_t ws_bytes, coli_stream_t stream);

/*
 * The same layer forward, with stage timing for profiling callers:
 * stage_events holds COLI_N_STAGE_EVENTS hipEvent_t handles created by the
 * caller; event 0 is recorded on `stream` before the first kernel and event i
 * after stage i: 1 quantise + router, 2 dispatch, 3 gate/up + SiLU + requant,
 * 4 down projection, 5 combine.  Results are identical to
 * colibri_moe_layer_forward.  stage_events == NULL behaves like it.
 */
#define COLI_N_STAGE_EVENTS 6
int colibri_moe_layer_forward_staged(const coli_moe_layer* L, const float* x, int32_t S, float* out,
                                     void* ws, size_t ws_bytes, coli_stream_t stream,
                                     void* const* stage_events);

/*
 * The same layer forward without a caller workspace and without any
 * allocation, for callers that cannot allocate device memory around the call
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The workspace is a static device array of
 * COLI_NOALLOC_SCRATCH_BYTES in the library, one per GPU, held until the
 * process ends; its address on the current device is looked up once, on the
 * first call on that device.  The call allocates nothing and frees nothing.
 * x, out and the layer's tensors are as for colibri_moe_layer_forward and
 * results are identical to it.
 *   COLI_E_SCRATCH: colibri_workspace_bytes(L, S) > COLI_NOALLOC_SCRATCH_BYTES
 *                   (a batch that large needs colibri_moe_layer_forward); the
 *                   check happens before anything is enqueued.
 *   COLI_E_HIP:     the current device or the array's address could not be
 *                   obtained.
 * Every call on one GPU uses that GPU's one array, which keeps the last
 * call's contents (no call needs it cleared): calls that may overlap on one
 * GPU -- on different streams, or from different host threads -- race and
 * must be serialised by the caller.
 */
#define COLI_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int colibri_moe_layer_forward_noalloc(const coli_moe_layer* L, const float* x, int32_t S, float* out,
                                      coli_stream_t stream);

/* ===========================================================================
 * Tiered expert residency ([README] section "思路" (idea): the routed experts
 * live in a slow tier and stream in on demand through a per-layer LRU cache
 * with an optional pinned hot store; its learned-cache paragraph: the experts
 * routed most often are pinned; its deferred cold-expert pipeline paragraph:
 * resident experts compute while the missing ones load in the background and
 * their results join before the layer ends).  On one MI355X the fast tier is
 * a bank of n_slots expert slots in HBM and the slow tier is pinned host
 * memory, which kernels read over PCIe.
 *
 * Two objects:
 *   coli_expert_cache  the slot-cache policy as a host object (no GPU
 *                      calls): the reference that the tier's device planner
 *                      follows step for step, usable on its own.
 *   coli_tier          one layer whose routed experts live in the slow tier,
 *                      with its cache state in HBM, its slot bank, a copy
 *                      stream and events.
 * Unlike the calls above, these objects own host memory and (coli_tier) HIP
 * objects; which calls wait for the host is stated with each.
 * ========================================================================= */

typedef struct coli_expert_cache coli_expert_cache;

/* Pair codes written by colibri_cache_plan: pass << COLI_PLAN_SLOT_BITS | slot. */
#define COLI_PLAN_SLOT_BITS 11

/* One expert load: `expert` into `slot`, needed by pass `pass`.  When
 * after >= 0 the load may start only once pass `after` of the same plan has
 * finished (that pass still reads the slot's previous occupant). */
typedef struct coli_cache_load {
    int32_t expert, slot, pass, after;
} coli_cache_load;

typedef struct coli_cache_plan {
    int32_t n_pass; /* passes; pass 0 computes the experts found resident */
    int32_t n_load; /* loads written (one per miss) */
    int32_t n_hit;  /* distinct routed experts found resident */
    int32_t n_miss; /* distinct routed experts that have to be loaded */
} coli_cache_plan;

typedef struct coli_cache_stats {
    uint64_t plans;     /* successful plans */
    uint64_t pairs;     /* routed pairs planned (dropped slots excluded) */
    uint64_t hits;      /* per plan: distinct experts found resident, summed */
    uint64_t misses;    /* per plan: distinct experts loaded, summed */
    uint64_t pin_loads; /* loads made by pinning */
    uint64_t passes;    /* summed over plans */
    uint64_t prefetches;     /* successful look-ahead prefetches */
    uint64_t prefetch_loads; /* loads made by them */
    int32_t resident;   /* slots holding an expert now */
    int32_t pinned;     /* slots pinned now */
} coli_cache_stats;

/* A cache of n_slots empty slots for n_experts experts (1 <= n_slots <=
 * n_experts <= COLI_MAX_EXPERTS). */
int colibri_cache_create(int32_t n_experts, int32_t n_slots, coli_expert_cache** out);
void colibri_cache_destroy(coli_expert_cache* c);

/*
 * Pins n distinct experts in [0, n_experts) for good (the hot store): a
 * resident one keeps its slot; any other takes a victim slot (empty first,
 * then least recently used, ties to the lower slot) and is listed in loads
 * (host, n entries; pass 1, after -1), *n_load of them.  The pinned set may
 * hold at most n_slots - 1 experts unless it holds all of them (n_slots ==
 * n_experts), so that a miss always finds a slot: COLI_E_UNSUPPORTED
 * otherwise.  Invalid or refused calls change nothing.
 */
int colibri_cache_pin(coli_expert_cache* c, const int32_t* experts, int32_t n,
                      coli_cache_load* loads, int32_t* n_load);

/* Unpins every expert; they stay resident. */
void colibri_cache_unpin(coli_expert_cache* c);

/*
 * Plans one batch.  ids [P] (host) are routed expert ids, -1 for a dropped
 * slot.  The distinct experts are taken in order of first appearance; those
 * resident (hits) run in pass 0 from their slots.  Misses take slots from a
 * ring: first the slots neither pinned nor holding a hit (empty first, then
 * least recently used, ties to the lower slot), then the unpinned hit slots
 * (reusable after pass 0).  With R ring slots, misses that fit (n_miss <= R)
 * all run in pass 1; otherwise they run in chunks of c = max(1, R/2) per
 * pass, miss i taking ring slot i mod R, so that (for R >= 2) one chunk's
 * loads overlap the previous chunk's compute.  Each ring slot ends up with
 * its last miss; what it held before is evicted.  Every expert of the batch
 * becomes most recently used; usage counts grow by its pairs.  Host
 * outputs: pair_code [P] (pass << COLI_PLAN_SLOT_BITS | slot, -1 for a
 * dropped slot), loads [min(P, n_experts)] in pass order, pass_pairs
 * [min(P, n_experts) + 1] (pairs per pass), *plan.  An id >= n_experts is
 * COLI_E_INVAL and changes nothing.
 */
int colibri_cache_plan(coli_expert_cache* c, const int32_t* ids, int32_t P, int32_t* pair_code,
                       coli_cache_load* loads, int32_t* pass_pairs, coli_cache_plan* plan);

/*
 * Look-ahead prefetch ([README] router look-ahead paragraph: the next
 * layer's experts are predicted from the current layer's state and read
 * ahead while the current layer computes).  ids [P] (host) are predicted
 * routed ids.  As colibri_cache_plan, except: the ring is only the slots
 * neither pinned nor holding a predicted expert, the misses beyond it are
 * not loaded, and usage is not counted.  Writes loads [min(P, n_experts)]
 * (pass 1, after -1) and *plan (n_pass 2 if anything is loaded, else 1;
 * n_miss = n_load = loads made).  Counted in prefetches / prefetch_loads.
 */
int colibri_cache_prefetch(coli_expert_cache* c, const int32_t* ids, int32_t P, coli_cache_load* loads,
                           coli_cache_plan* plan);

int colibri_cache_stats(const coli_expert_cache* c, coli_cache_stats* st);

/* Host copies of the state: slot_of [n_experts] (slot or -1) and usage
 * [n_experts] (routed pairs so far); either may be NULL. */
int colibri_cache_state(const coli_expert_cache* c, int32_t* slot_of, uint64_t* usage);

typedef struct coli_tier coli_tier;

/* Device bytes that colibri_tier_create needs for n_slots experts of layer
 * L: the slot bank (gate, up and down codes and scales) and the cache state,
 * each region 256-byte aligned (0 if L is invalid or n_slots is outside
 * [1, n_experts]). */
size_t colibri_tier_slot_bytes(const coli_moe_layer* L, int32_t n_slots);

/*
 * A tiered layer on the current device.  L is a complete layer descriptor
 * whose routed banks (gate, up, down with n_mat = n_experts) are the slow
 * tier: pinned host memory (hipHostMalloc) or device memory, row scales
 * 16-byte aligned; pageable host memory is COLI_E_UNSUPPORTED.  Router and
 * shared expert are device memory as for colibri_moe_layer_forward.
 * slot_mem is device memory of slot_bytes >= colibri_tier_slot_bytes(L,
 * n_slots) bytes, 256-byte aligned, that the tier owns until
 * colibri_tier_destroy, as it keeps L's pointers.  Creates a non-blocking
 * copy stream (default priority) and events, and waits for the state's
 * initialisation: all slots empty, nothing pinned.
 */
int colibri_tier_create(const coli_moe_layer* L, int32_t n_slots, void* slot_mem, size_t slot_bytes,
                        coli_tier** out);

/* Waits for the tier's copy stream, then frees its host state and HIP objects. */
void colibri_tier_destroy(coli_tier* t);

/*
 * Pins experts (the policy of colibri_cache_pin, same limit): the pin
 * kernel and the loads run on `stream`, and the call waits for them.
 */
int colibri_tier_pin(coli_tier* t, const int32_t* experts, int32_t n, coli_stream_t stream);

/* Workspace bytes of colibri_tier_forward for up to S tokens (0 if invalid). */
size_t colibri_tier_workspace_bytes(const coli_tier* t, int32_t S);

/*
 * colibri_moe_layer_forward with the routed experts taken from the slot
 * bank.  On `stream`: route, then the plan kernel (the policy of
 * colibri_cache_plan on the routed ids, on the state in device memory),
 * then pass 0 (the resident experts and the shared expert) while the fetch
 * kernel on the tier's copy stream reads the misses from the slow tier into
 * their slots; pass 1 waits for that fetch; one combine ends the call.
 * When n_slots minus the pinned experts is at least min(S * top_k,
 * n_experts), every plan has at most these two passes and the call returns
 * without waiting for the device; with every expert pinned, pass 0 alone,
 * and for one token the resident one-token kernels themselves, reading the
 * experts through the slot map (then the plan, all hits, updates the
 * cache's counters).  Otherwise a plan may need more passes:
 * the call then waits once for the plan to reach the host (pass 0 is
 * already running) and enqueues each later pass after its own fetch.  The
 * output is bit-identical to colibri_moe_layer_forward on the same weights.
 * Calls on one tier must be ordered on one stream and made with the tier's
 * device current; pinned host staging is allocated the first time a
 * many-pass call needs more than any call before it.  After a HIP error the
 * tier's state is unspecified: destroy it.
 */
int colibri_tier_forward(coli_tier* t, const float* x, int32_t S, float* out, void* ws,
                         size_t ws_bytes, coli_stream_t stream);

/*
 * Look-ahead prefetch of the tier's experts for activations x fp32
 * [S][hidden] (S <= 8) that predict this layer's input, for instance the
 * previous layer's input ([README] router look-ahead paragraph).  Everything
 * runs on the tier's copy stream after the work enqueued on `stream` so far:
 * route x with this layer's router (into the tier's own scratch), plan a
 * prefetch on the state (colibri_cache_prefetch's policy), load the
 * predicted misses.  Returns without waiting; the caller's stream is not
 * delayed.  The tier's next forward waits for the prefetch before it plans.
 * x must not be changed by work on `stream` enqueued before that forward.
 */
int colibri_tier_prefetch(coli_tier* t, const float* x, int32_t S, coli_stream_t stream);

/*
 * One step of batched verification through a stack of tiered layers: the
 * S positions of one step (for speculative decoding, the last accepted
 * token and its drafts, checked in one batched forward: "Show HN:
 * 如何在我的低配置电脑上运行 GLM-5.2", section 已实现的功能, the native MTP
 * item) pass through tiers[0 .. n_layers - 1] in order, each layer's
 * forward being colibri_tier_forward's.
 *   x    device fp32 [n_layers][S][hidden]: layer l's input.  The attention
 *        and norms between the layers are not part of this library, so the
 *        caller supplies every layer's input (recorded or synthetic
 *        activations).
 *   out  device fp32 [n_layers][S][hidden]: layer l's output, bit-identical
 *        to colibri_tier_forward's and the resident forward's on x_l.
 *   lookahead  nonzero: the router look-ahead of the same section (the
 *        next layer's experts predicted from the current layer's input and
 *        read while it computes): before layer l runs, layer l + 1's
 *        router routes x_l on layer l + 1's copy stream and plans a
 *        prefetch there (colibri_tier_prefetch's policy); its loads are
 *        queued behind layer l's own misses, and layer l + 1's forward uses
 *        them as colibri_tier_forward uses any prefetch.  Requires S <= 8.
 *   union_mask, stats  both null (no statistics), or: union_mask device
 *        uint32 [n_layers][(n_experts + 31) / 32], per layer the set of
 *        experts the previous step routed to (zero it before the first
 *        step; each step replaces it with its own), and stats device int32
 *        [n_layers][2], per layer the number of distinct routed experts of
 *        this step (the union its batched forward reads once) and how many
 *        of them the previous step's set held.
 *   ws   workspace of colibri_tier_workspace_bytes(tiers[0], S).
 * Every tier has the same hidden, inter, n_experts, top_k and shared
 * expert, appears once, and lives on the current device.  Calls are ordered
 * on `stream` like colibri_tier_forward's and return without waiting for
 * the device when every layer's misses fit two passes; work enqueued on
 * `stream` after the call follows every read of x.  x and out are 16-byte
 * aligned.  Returns COLI_E_INVAL for a null or repeated tier, differing
 * shapes, null buffers (or one of union_mask and stats null) or another
 * current device, COLI_E_UNSUPPORTED for misaligned buffers or look-ahead
 * with S > 8, COLI_E_WORKSPACE for a short workspace; after COLI_E_HIP the
 * tiers' states are unspecified.
 */
int colibri_tier_verify_step(coli_tier* const* tiers, int32_t n_layers, const float* x, int32_t S,
                             float* out, int32_t lookahead, void* ws, size_t ws_bytes,
                             uint32_t* union_mask, int32_t* stats, coli_stream_t stream);

/* Statistics of the tier's cache (as colibri_cache_stats); waits for `stream`. */
int colibri_tier_stats(const coli_tier* t, coli_cache_stats* st, coli_stream_t stream);

/* Host copies of the tier's state (as colibri_cache_state); waits for `stream`. */
int colibri_tier_state(const coli_tier* t, int32_t* slot_of, uint64_t* usage, coli_stream_t stream);

/* Static text for a status code. */
const char* colibri_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif
