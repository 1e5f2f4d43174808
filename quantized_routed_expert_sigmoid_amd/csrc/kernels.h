/*
 * kernels.h -- internal launch interface of libcolibri's gfx950 kernels.
 * Host-side argument validation lives in api.hip; every launcher here assumes
 * validated shapes and returns the HIP launch status.
 */
#ifndef COLI_KERNELS_H
#define COLI_KERNELS_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

/* Tokens that one GEMV work unit applies an expert's rows to.  Experts with
 * more tokens are split into several units. */
constexpr int kUnitTokens = 4;

/* Experts holding at least a threshold of tokens of a batch run on the int8
 * matrix cores (ffn_mfma.hip) in units of up to kMfmaUnitTokens tokens;
 * experts with fewer run on the GEMV kernels (ffn_gemv.hip).  The threshold
 * is kMfmaMinTokens, except in a layer's routed batch (layer_mfma_min). */
constexpr int kMfmaMinTokens = 8;
constexpr int kMfmaUnitTokens = 32;

/* Most (token, slot) pairs of one call (the ABI's limit). */
constexpr int32_t kPairLimit = 1 << 20;

/* Batches of at most this many tokens use the small-batch router kernels
 * (a workgroup per router row; selection and dispatch in one workgroup). */
constexpr int kSmallS = 8;

/* Pair codes of a tiered forward: pass << kPassSlotBits | slot (slots below
 * 2^kPassSlotBits, which the expert limit of 1024 keeps); the same width as
 * COLI_PLAN_SLOT_BITS of the C ABI. */
constexpr int kPassSlotBits = 11;

/* Most expert groups of group-limited selection. */
constexpr int kMaxGroups = 64;

/* Router variants (n_group <= 1 and top_p outside (0, 1): plain top-k). */
struct RouteOpts {
    int32_t n_group, topk_group;
    float top_p;
};

/* A work unit: expert e applied to sorted positions [pos0, pos0 + ntok). */
struct Unit {
    int32_t e, pos0, ntok, pad;
};

/* Device unit lists written by the dispatch (or schedule) kernel. */
struct UnitLists {
    Unit* units;       /* GEMV units (experts with < mfma_min tokens) */
    int32_t* n_units;
    int32_t max_units;
    Unit* munits;      /* MFMA units */
    int32_t* n_munits;
    int32_t max_munits;
    int32_t mfma_min;  /* fewest tokens of an expert on the matrix cores */
};

/* One group of experts run by the FFN kernels.  A group with units ==
 * munits == nullptr is one expert applied to positions [0, S) in order (the
 * shared expert); its max_units / max_munits select which kernels take it. */
struct FfnSeg {
    const uint8_t* gate_w;
    const float* gate_s;
    const uint8_t* up_w;
    const float* up_s;
    const uint8_t* down_w;
    const float* down_s;
    const int32_t* sorted;   /* pair index per sorted position; nullptr: identity */
    const Unit* units;       /* GEMV unit list (device) */
    const int32_t* n_units;
    const Unit* munits;      /* MFMA unit list (device) */
    const int32_t* n_munits;
    int32_t k;               /* token of pair p is p / k */
    int32_t out_base;        /* first row of this group in hq / hd / y */
    int32_t max_units;       /* grid bounds of the two kernel families */
    int32_t max_munits;
    int32_t S;               /* tokens of the batch */
    int32_t rows;            /* sorted positions of this group (S*k, or S for identity) */
    int32_t n_mat;           /* matrices in the group's banks */
    int32_t gu_gb, d_gb;     /* Q8_0 blocks per weight scale of gate/up and of down; 0: per-row
                                scales (row r's K/32/gb scales at scale + (e*rows + r) * K/32/gb) */
};

/* Coefficient of block b with group-wise weight scales: the row's scale of
 * b's group times the activation block scale (one fp32 multiply). */
__device__ __forceinline__ float group_coef(const float* ws, int gb, int b, float d)
{
    return ws[b / gb] * d;
}

/* Test-only build (COLI_DEBUG_PARTIALS): the FFN kernels also store the
 * exact int32 block partials they compute for one slice -- matrix kind
 * (kDbgGate, kDbgUp, kDbgDown), output rows [o0, o1) of hq / y (sorted
 * positions, or units of a one-token batch), weight rows [r0, r1), blocks
 * below nb -- at out[((o - o0) * (r1 - r0) + (r - r0)) * nb + b].  In the
 * product build FfnArgs carries no slice and the hook is empty. */
enum { kDbgGate = 0, kDbgUp = 1, kDbgDown = 2 };

struct DebugSlice {
    int32_t* out; /* device; null: off */
    int32_t kind, o0, o1, r0, r1, nb;
};

struct FfnArgs {
#ifdef COLI_DEBUG_PARTIALS
    DebugSlice dbg;
#endif
    FfnSeg seg[2];
    int32_t nseg;
    int32_t unit_tokens; /* most tokens any GEMV unit holds: 1 or kUnitTokens */
    int32_t H, I;
    const int8_t* xq; /* [S][H]   */
    const float* xd;  /* [S][H/32] */
    int8_t* hq;       /* [rows][I] */
    float* hd;        /* [rows][I/32] */
    float* y;         /* [rows][H] */
};

/* Stores partial s of (kind, output row o, weight row r, block b) when the
 * slice holds it (test-only build). */
__device__ __forceinline__ void dbg_partial(const FfnArgs& a, int kind, int64_t o, int r, int b, int32_t s)
{
#ifdef COLI_DEBUG_PARTIALS
    const DebugSlice& d = a.dbg;
    if (d.out && kind == d.kind && o >= d.o0 && o < d.o1 && r >= d.r0 && r < d.r1 && b >= 0 && b < d.nb)
        d.out[((o - d.o0) * (int64_t)(d.r1 - d.r0) + (r - d.r0)) * d.nb + b] = s;
#else
    (void)a; (void)kind; (void)o; (void)r; (void)b; (void)s;
#endif
}

/* The slot cache's state of a tiered layer (tier_kernels.hip). */
struct TierHdr {
    uint32_t tick; /* plans, prefetches and pins so far (the LRU clock) */
    int32_t pad;
    unsigned long long plans, pairs, hits, misses, pin_loads, passes, prefetches, prefetch_loads;
};

struct TierState {
    TierHdr* hdr;
    int32_t* slot_of;          /* [E]: slot or -1 */
    int32_t* expert_in;        /* [n]: expert or -1 */
    uint32_t* last_use;        /* [n]: tick of the last use */
    int32_t* pinned;           /* [n] */
    int32_t* inflight;         /* [n]: loaded by a prefetch that no plan has consumed */
    unsigned long long* usage; /* [E]: routed pairs */
    int32_t E, n;
};

/* One-token batch (decode): selection inside the gate/up kernel.  f.seg[0]
 * is the routed bank (n_mat = E), f.seg[1] the shared expert when
 * f.nseg == 2; hq / hd / y hold one row per unit (slot order, shared last). */
struct DecodeArgs {
    FfnArgs f;
    const float* logits; /* [E] */
    const float* bias;   /* [E] */
    int32_t E, k;
    float rsf;
    RouteOpts opt;
    int32_t* ids;        /* [k] selected experts, slot order (-1: dropped) */
    float* w;            /* [k] routing weights */
    float* out;          /* [H] layer output (down + combine launch) */
    /* nullptr: the shared expert's gate/up runs as whole jobs into hq / hd.
     * Otherwise its gate/up runs as I / 8 one-wave jobs of 8 gate and 8 up
     * rows that write h (fp32, [I]) here, and the fused down + combine
     * quantises it while staging (per-row scales, I <= 2048 and the fused
     * launch only). */
    float* hs;
    /* nullptr: a routed expert's matrices are at its id in seg[0]'s banks.
     * Otherwise at slot_of[id] (a tiered layer's slot map, [E], every
     * routed expert resident). */
    const int32_t* slot_of;
    /* nonzero: a tiered forward with every expert resident; the fused
     * down + combine also leaves the slot cache's state `ts` as the plan
     * kernel leaves it after an all-hit batch */
    int32_t note_hits;
    TierState ts;
};

/* The matrix-core threshold of a layer's batch of S tokens (P pairs over E
 * experts).  Small batches (S <= kSmallS) stay on the GEMV kernels, so they
 * launch no matrix-core kernel at all.  A batch with at least kMfmaMinTokens
 * pairs per expert on average runs every expert on the matrix cores and
 * launches no GEMV kernel: its few small experts cost less there than the
 * GEMV launches' worst-case grids.  In between, kMfmaMinTokens. */
inline int32_t layer_mfma_min(int64_t P, int32_t E, int32_t S)
{
    if (S <= kSmallS)
        return kSmallS + 1;
    if (P >= (int64_t)kMfmaMinTokens * E)
        return 1;
    return kMfmaMinTokens;
}

/* Bounds on the unit counts of a routed group with P pairs over E experts
 * (n_e pairs each, sum P) and threshold mmin.  GEMV: experts with n_e < mmin
 * give ceil(n_e / kUnitTokens) units each, at most ceil((mmin - 1) /
 * kUnitTokens).  MFMA: experts with n_e >= mmin give ceil(n_e / 32) <=
 * n_e / 32 + 1 units each; none when the batch has fewer than mmin tokens
 * per expert at most (S < mmin, S = the most pairs one expert can hold). */
inline int32_t max_gemv_units(int64_t P, int32_t E, int32_t mmin)
{
    const int64_t per = (mmin - 1 + kUnitTokens - 1) / kUnitTokens;
    const int64_t active = P < E ? P : E;
    const int64_t a = (P + (kUnitTokens - 1) * active) / kUnitTokens;
    const int64_t b = per * active;
    return (int32_t)(a < b ? a : b);
}

inline int32_t max_mfma_units(int64_t P, int32_t E, int32_t S, int32_t mmin)
{
    if (S < mmin)
        return 0;
    const int64_t big = P / mmin < E ? P / mmin : E;
    return (int32_t)(P / kMfmaUnitTokens + big + 1);
}

/* Units of a one-expert identity group over S tokens. */
inline int32_t identity_gemv_units(int32_t S, int32_t mmin)
{
    return S >= mmin ? 0 : (S + kUnitTokens - 1) / kUnitTokens;
}

inline int32_t identity_mfma_units(int32_t S, int32_t mmin)
{
    return S >= mmin ? (S + kMfmaUnitTokens - 1) / kMfmaUnitTokens : 0;
}

/* Tile edge of the many-token router logits (tokens x experts per
 * workgroup of four waves): 128 (waves of 64 x 64) when the batch has at
 * least 32 such tiles, else 64 (waves of 32 x 32). */
inline int32_t router_tile(int32_t S, int32_t E)
{
    const int64_t t128 = (int64_t)((S + 127) / 128) * ((E + 127) / 128);
    return t128 >= 32 ? 128 : 64;
}

/* K slices of the many-token router logits (S > kSmallS): enough tiles
 * times slices for about 512 workgroups, at most 16 slices and one 16-wide k
 * chunk per slice; 1 for small batches.  The logits buffer holds
 * router_parts * S * E floats. */
inline int32_t router_parts(int32_t S, int32_t E, int32_t H)
{
    if (S <= kSmallS)
        return 1;
    const int32_t T = router_tile(S, E);
    const int64_t tiles = (int64_t)((S + T - 1) / T) * ((E + T - 1) / T);
    int64_t p = (512 + tiles - 1) / tiles;
    if (p > 16)
        p = 16;
    if (p > H / 16)
        p = H / 16;
    return (int32_t)(p < 1 ? 1 : p);
}

hipError_t launch_quantize_q8_0(const float* x, int64_t n_blocks, int8_t* q, float* d,
                                hipStream_t st);

/* Writes router_parts(S, E, H) partial logit slices [part][S][E]. */
hipError_t launch_router_logits(const float* x, int32_t S, int32_t H, int32_t E,
                                const float* w, float* logits, hipStream_t st);

/* Selection from n_parts partial logit slices (added in slice order). */
hipError_t launch_router_select(const float* logits, int32_t n_parts, const float* bias, int32_t S,
                                int32_t E, int32_t k, float rsf, const RouteOpts& opt, int32_t* ids,
                                float* weights, hipStream_t st);

/* Router logits (router_parts slices for S > kSmallS) and Q8_0 quantisation
 * of x in one launch, for any S. */
hipError_t launch_route_prep(const float* x, int32_t S, int32_t H, int32_t E, const float* w, float* logits,
                             int8_t* xq, float* xd, hipStream_t st);

/* S <= kSmallS: router logits and Q8_0 quantisation of x in one launch. */
hipError_t launch_route_prep_small(const float* x, int32_t S, int32_t H, int32_t E, const float* w,
                                   float* logits, int8_t* xq, float* xd, hipStream_t st);

/* S <= kSmallS: selection, union dispatch and unit lists in one workgroup. */
hipError_t launch_select_dispatch_small(const float* logits, const float* bias, int32_t S, int32_t E,
                                        int32_t k, float rsf, const RouteOpts& opt, int32_t* ids,
                                        float* weights, int32_t* offsets, int32_t* sorted, int32_t* inv,
                                        int32_t* active, int32_t* n_active, const UnitLists& ul,
                                        hipStream_t st);

/* Union dispatch; `ul` may be null (then no unit lists). */
hipError_t launch_dispatch(const int32_t* ids, int32_t S, int32_t k, int32_t E,
                           int32_t* offsets, int32_t* sorted, int32_t* inv, int32_t* active,
                           int32_t* n_active, const UnitLists* ul, hipStream_t st);

/* Union dispatch of one pass of a tiered forward over n_slots slot matrices:
 * the pairs whose code names `pass` (see kPassSlotBits); they get inv =
 * inv_base + sorted position.  Pass 0 also sets inv = -1 for every other
 * pair; later passes leave those entries alone. */
hipError_t launch_dispatch_pass(const int32_t* codes, int32_t pass, int32_t inv_base, int32_t S,
                                int32_t k, int32_t n_slots, int32_t* offsets, int32_t* sorted,
                                int32_t* inv, int32_t* active, int32_t* n_active, const UnitLists& ul,
                                hipStream_t st);

/* Unit lists from expert offsets (for a caller-provided dispatch), bounded
 * by ul.max_units / ul.max_munits. */
hipError_t launch_schedule(const int32_t* offsets, int32_t n_mat, const UnitLists& ul,
                           hipStream_t st);

/* GEMV and MFMA kernel families; each launches nothing when its units are
 * impossible for the batch. */
hipError_t launch_ffn_gate_up(const FfnArgs& a, int32_t bits, hipStream_t st);
hipError_t launch_ffn_down(const FfnArgs& a, int32_t bits, hipStream_t st);
hipError_t launch_ffn_gate_up_mfma(const FfnArgs& a, int32_t bits, hipStream_t st);
hipError_t launch_ffn_down_mfma(const FfnArgs& a, int32_t bits, hipStream_t st);

/* ---- tiered expert store (tier_kernels.hip) ------------------------------
 * The slot cache's state lives in device memory next to the slot bank; the
 * plan kernel follows the policy of the host planner (expert_cache.cpp)
 * step for step. */
constexpr int kTierMaxE = 1024; /* experts and slots */

/* info[] fields written by the plan and pin kernels. */
enum { kInfoPass = 0, kInfoLoad, kInfoHit, kInfoMiss, kInfoChunk, kInfoRing, kInfoError, kInfoN = 8 };

/* Per-expert regions of the slow tier and the slot bank, in 16-byte units:
 * gate codes, gate scales, up codes, up scales, down codes, down scales.
 * Expert e's region r starts at src[r] + e * len[r]; slot s's at dst[r] +
 * s * len[r]. */
struct TierBanks {
    const uint4* src[6];
    uint4* dst[6];
    int64_t len[6];
};

hipError_t launch_tier_init(const TierState& st, hipStream_t s);

/* Plans P routed ids (ids >= E or < 0 count as dropped): codes [P], loads
 * [min(P, E)] {expert, slot, pass, after}, info [kInfoN], pass_pairs
 * [min(P, E) + 1]; updates the state.  With `prefetch` set it plans a
 * look-ahead instead: the misses that fit the free slots are loaded in pass
 * 1, usage is not counted, and codes / pass_pairs are not written (may be
 * null). */
hipError_t launch_tier_plan(const int32_t* ids, int32_t P, const TierState& st, int32_t* codes,
                            int4* loads, int32_t* info, int32_t* pass_pairs, bool prefetch,
                            hipStream_t s);

/* Pins n experts (validated by the host): loads [n] and info as for a plan
 * whose single miss pass is pass 1. */
hipError_t launch_tier_pin(const int32_t* experts, int32_t n, const TierState& st, int4* loads,
                           int32_t* info, hipStream_t s);

/* Copies the loads of `pass` (from info's chunk and load count) from the slow
 * tier into their slots. */
hipError_t launch_tier_fetch(const int4* loads, const int32_t* info, int32_t pass, const TierBanks& b,
                             hipStream_t s);

/* Draft-union statistics of P routed ids (E <= kTierMaxE): stats[0] =
 * distinct experts, stats[1] = how many of them the bit set mask
 * [(E + 31) / 32] held; mask <- this set. */
hipError_t launch_verify_union(const int32_t* ids, int32_t P, int32_t E, uint32_t* mask, int32_t* stats,
                               hipStream_t s);

hipError_t launch_ffn_gate_up_decode(const DecodeArgs& d, int32_t bits, hipStream_t st);
hipError_t launch_ffn_down_decode(const DecodeArgs& d, int32_t bits, hipStream_t st);

/* Down projection and combine in one launch (writes out, not y); usable
 * when H is a multiple of 16 and all units' h fit the workgroup's LDS. */
bool down_combine_decode_fits(const DecodeArgs& d);
hipError_t launch_ffn_down_combine_decode(const DecodeArgs& d, int32_t bits, hipStream_t st);

/* out[t] = y[shared_row0 + t] (if shared_row0 >= 0) + sum_j w[t*k+j] * y[row(t*k+j)],
 * row(p) = inv[p], or p when inv is null; slots with inv[p] < 0 (inv null:
 * ids[p] < 0) were dropped and are skipped. */
hipError_t launch_combine(const float* y, const int32_t* inv, const int32_t* ids, const float* w,
                          int32_t S, int32_t k, int32_t H, int32_t shared_row0, float* out,
                          hipStream_t st);

} // namespace coli

#endif
