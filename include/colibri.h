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
 *     memory read during the call only.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  No call synchronises the host or copies to the host.
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
    COLI_E_HIP = 4          /* the HIP runtime reported an error at launch */
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
 * per row ([DIVE] 5.1).  Row r of matrix m starts at byte (m*rows + r) * K *
 * qtype / 8 of `data`; its scale is row_scale[m*rows + r].
 *   COLI_Q8: one two's-complement byte per weight.
 *   COLI_Q4: byte j of a row holds element 2j in bits 7..4 and element 2j+1 in
 *            bits 3..0, two's-complement nibbles in [-8, 7].
 *   COLI_Q2: byte j holds elements 4j..4j+3 in bits 7..6, 5..4, 3..2, 1..0,
 *            two's-complement values in [-2, 1].
 * Requirements: K % 32 == 0, rows >= 1, n_mat >= 1, `data` 16-byte aligned,
 * `row_scale` 4-byte aligned.
 */
typedef struct coli_qbank {
    const void* data;
    const float* row_scale;
    int32_t n_mat, rows, K;
    int32_t qtype; /* COLI_Q8, COLI_Q4 or COLI_Q2 */
} coli_qbank;

/*
 * One layer.  gate/up: n_mat = n_experts, rows = inter, K = hidden; down:
 * n_mat = n_experts, rows = hidden, K = inter.  gate and up share a qtype.
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
 * weight code * activation code: the nb = K/32 blocks form four consecutive
 * groups (group g: blocks floor(g*nb/4) .. floor((g+1)*nb/4)-1), each folded
 * acc = fmaf(d_b, (float)S_b, acc) in ascending block order from +0, and the
 * four group sums are added left to right (the pages leave the order of the
 * fp32 accumulation open; this one is fixed so that results are bit-exact
 * across batch sizes and kernels).  silu(g) = g / (1 + exp(-g)) with exp by Cody-Waite
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

/* Static text for a status code. */
const char* colibri_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif
