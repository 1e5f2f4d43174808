/*
 * coli_ref.h -- the oracle: a plain, slow, single-threaded C11 reference of
 * one sigmoid-routed, quantised mixture-of-experts layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library never
 * includes, links or calls it, and this file shares no code with it.
 *
 * Sources (web pages on the colibri runtime):
 *   [README]  "Show HN: 如何在我的低配置电脑上运行 GLM-5.2" (Chinese translation
 *             of the colibri README), section "已实现的功能" (implemented
 *             features): the sigmoid-router item (DeepSeek-V3 style, noaux_tc,
 *             routed_scaling_factor, shared expert), the integer dot-product
 *             item (Q8_0-style int8 activations), the quantised-kernel item
 *             (int8 / packed int4 / packed int2, per-row scales, dequantised
 *             on use, packing bit-identical to the int8 container) and the
 *             batched-union MoE item; section "实验性 Metal 后端" (the routed
 *             expert work is a SwiGLU).
 *   [DIVE]    "colibrì 深度拆解" (deep dive), section 4.3 (per-token routing:
 *             shared expert plus routing-weighted sum of the top-8 experts)
 *             and section 5.1 (int4 container: two values per byte, first
 *             element in the high nibble, one fp32 scale per row).
 *
 * Where the pages are silent the oracle follows one stated reading; every
 * reading is listed in the repository's design notes.  Precision: every step
 * that decides an integer (an activation code, a routed expert id) is taken
 * in fp32, the precision of the GPU kernels; the routing weights and the
 * final combine are carried in fp64.
 */
#ifndef COLI_REF_H
#define COLI_REF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by the oracle's layer-level calls. */
#define REF_OK 0
#define REF_E_INVAL 1     /* bad dimension / null pointer */
#define REF_E_MISSING 2   /* a matrix the computation needs was not supplied */

/*
 * A bank of n_mat quantised matrices, each [rows][K], row-major, with one
 * fp32 scale per row ([DIVE] 5.1; [README] quantised-kernel item) or, with
 * group > 0, one fp32 scale per `group` consecutive columns of a row (the
 * group-wise scaling that [README]'s quality-benchmark paragraph names as
 * the likely priority; the pages give no layout, see ref_qdot_grouped).
 *   bits = 8: one two's-complement byte per weight.
 *   bits = 4: byte j of a row holds element 2j in bits 7..4 and element 2j+1
 *             in bits 3..0, each a two's-complement nibble in [-8, 7].
 *   bits = 2: byte j holds elements 4j..4j+3 in bits 7..6, 5..4, 3..2, 1..0,
 *             each a two's-complement 2-bit value in [-2, 1].
 * mat_data[m] / mat_scale[m] point at matrix m's rows / scales (rows floats,
 * or rows * K/group floats, row r's at r * K/group); a NULL entry means "not
 * supplied" (lets a caller hand over only the experts a computation
 * touches).  group: 0, or a multiple of 32 that divides K.
 */
typedef struct ref_bank {
    const uint8_t* const* mat_data;
    const float* const* mat_scale;
    int32_t n_mat, rows, K, bits;
    int32_t group;
} ref_bank;

/* Router variants.  n_group > 1: group-limited selection (experts in n_group
 * equal contiguous groups; a group's score is the sum of its two largest
 * biased scores; the topk_group best groups are kept, ties to the lower
 * group; top-k runs over the kept groups' experts).  0 < top_p < 1: adaptive
 * expert top-p (the k slots ordered by unbiased score, descending, ties in
 * slot order; shares s / sum s accumulated in fp32; the shortest prefix whose
 * cumulative share reaches top_p is kept, at least one slot; dropped slots get
 * id -1 and weight 0, kept weights are renormalised over the kept slots). */
typedef struct ref_route_opts {
    int32_t n_group;
    int32_t topk_group;
    float top_p;
} ref_route_opts;

typedef struct ref_layer {
    int32_t hidden, inter, n_experts, top_k;
    float routed_scaling_factor;
    const float* router_w;     /* [E][H] fp32 */
    const float* router_bias;  /* [E]    fp32, selection only */
    ref_bank gate, up, down;   /* routed: gate/up [I][H], down [H][I] per expert */
    int32_t has_shared;
    ref_bank sh_gate, sh_up, sh_down; /* one matrix each */
    ref_route_opts route;      /* n_group 0 or 1 and top_p 0 or >= 1: plain top-k */
} ref_layer;

/* ---- activation quantisation (Q8_0 style, blocks of 32, fp32 scale) ---- */
float ref_round_half_away(float v);
/* v: n values (n % 32 == 0) -> q: n int8 codes, d: n/32 fp32 block scales. */
void ref_quantize_q8_0(const float* v, int64_t n, int8_t* q, float* d);

/* ---- weight containers ---- */
int32_t ref_row_bytes(int32_t K, int32_t bits);
/* Decode weight element `col` of a packed row. */
int32_t ref_weight_code(const uint8_t* row, int32_t bits, int32_t col);
/* Pack K codes (already in range for `bits`) into a row of ref_row_bytes. */
void ref_pack_row(const int8_t* codes, int32_t K, int32_t bits, uint8_t* out);

/* ---- integer dot path ---- */
/* Exact int32 partial of block b: sum over 32 elements of weight * code. */
int32_t ref_block_partial(const uint8_t* row, int32_t bits, const int8_t* q, int32_t b);
/* Canonical quantised row dot: the nb = K/32 block partials are folded in
 * one chain, acc = fmaf(d_b, (float)S_b, acc) from acc = +0 for b = 0, 1,
 * ..., nb-1 in ascending order; then one multiply by the row scale. */
float ref_qdot(const uint8_t* row, int32_t bits, float row_scale,
               const int8_t* q, const float* d, int32_t K);
/* The same quantity, unblocked, in fp64 (used to bound the fp32 fold). */
double ref_qdot_f64(const uint8_t* row, int32_t bits, float row_scale,
                    const int8_t* q, const float* d, int32_t K);
/* Row dot with group-wise scales s [K/group]: the weight of column c is
 * s[c / group] times its code, so block b contributes
 * s[32b / group] * d_b * S_b.  Canonical form: the coefficient
 * t_b = s[32b / group] * d_b is one fp32 multiply, and t_b takes the place of
 * d_b in the fold of ref_qdot (the same ascending chain); there is no row
 * scale. */
float ref_qdot_grouped(const uint8_t* row, int32_t bits, const float* s, int32_t group,
                       const int8_t* q, const float* d, int32_t K);
/* The same quantity, unblocked, in fp64. */
double ref_qdot_grouped_f64(const uint8_t* row, int32_t bits, const float* s, int32_t group,
                            const int8_t* q, const float* d, int32_t K);

/* ---- SwiGLU nonlinearity ---- */
/* exp by Cody-Waite reduction and a degree-7 Taylor polynomial; saturates to
 * +inf above 88 and to +0 below -87. */
float ref_cexp(float z);
float ref_silu(float g);
/* Element-wise loops over the two functions above (for sweeps). */
void ref_cexp_array(const float* z, float* out, int64_t n);
void ref_silu_array(const float* g, float* out, int64_t n);

/* ---- one expert on one token ----
 * gate/up/down rows of matrix e; xq/xd: the token's Q8_0 codes and scales.
 * Fills (when non-NULL) g, u, h [I], hq [I], hd [I/32]; always fills y [H]. */
int ref_expert_ffn(const ref_bank* gate, const ref_bank* up, const ref_bank* down,
                   int32_t e, const int8_t* xq, const float* xd,
                   float* g, float* u, float* h, int8_t* hq, float* hd, float* y);

/* ---- router, one token ----
 * logits in fp64 rounded to fp32; s = sigmoid (fp32, libm expf); c = s + bias
 * (fp32).  Selection: the k largest c under (c descending, expert ascending);
 * slot j holds the j-th selected expert.  w_j = rsf * s_j / sum_j' s_j' (fp64,
 * denominator summed in slot order).  Optional outputs: s[E], c[E], and gap =
 * c of the k-th selected minus the largest unselected c (+inf if k == E). */
int ref_route_token(const float* x, int32_t H, int32_t E, int32_t k,
                    const float* router_w, const float* bias, float rsf,
                    int32_t* ids, double* w, float* s, float* c, float* gap);
/* The same with the router variants of ref_route_opts (NULL: none).  gap is
 * the smallest decision margin: the expert gap above among the eligible
 * experts, with n_group > 1 also the topk_group-th kept group score minus the
 * best dropped one, with top-p also the distances of top_p from the
 * cumulative shares just before and at the cut. */
int ref_route_token_opt(const float* x, int32_t H, int32_t E, int32_t k,
                        const float* router_w, const float* bias, float rsf,
                        const ref_route_opts* opt, int32_t* ids, double* w, float* s, float* c,
                        float* gap);

/* ---- union dispatch ----
 * pairs p = t*k + j.  counts -> exclusive offsets[E+1]; sorted[] = pairs
 * stably ordered by expert; inv[p] = position of p in sorted[]; active[] =
 * experts with count > 0 ascending, *n_active their number.  A negative id
 * (a slot dropped by top-p) is no pair: it is not counted and inv[p] = -1. */
void ref_dispatch(const int32_t* ids, int32_t S, int32_t k, int32_t E,
                  int32_t* offsets, int32_t* sorted, int32_t* inv,
                  int32_t* active, int32_t* n_active);

/* ---- whole layer ----
 * out [S][H] in fp64.  Optional traces (NULL to skip): xq [S][H], xd
 * [S][H/32], ids [S][k], w [S][k] (fp64), y_routed [S*k][H] in pair order
 * (p = t*k + j), y_shared [S][H]. */
int ref_moe_layer_forward(const ref_layer* L, const float* x, int32_t S, double* out,
                          int8_t* xq, float* xd, int32_t* ids, double* w,
                          float* y_routed, float* y_shared);

#ifdef __cplusplus
}
#endif
#endif
