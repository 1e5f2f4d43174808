/*
 * coli_ref.c -- the oracle (see coli_ref.h).  TEST INFRASTRUCTURE ONLY.
 *
 * Plain C11, one thread, scalar loops in the order the method states them.
 * Built with -O2 -std=c11 -ffp-contract=off so that every fused multiply-add
 * is the explicit fmaf() written here and nothing else is contracted.
 */
#include "coli_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Activation quantisation: Q8_0 style, blocks of 32, one fp32 scale each    */
/* ([README] integer dot-product item).  Per block: amax = max |v|;           */
/* d = amax / 127 (IEEE fp32 division); id = 1/d (0 for an all-zero block);  */
/* code = clamp(round-half-away-from-zero(v * id), -127, 127).               */
/* ------------------------------------------------------------------------ */

float ref_round_half_away(float v)
{
    float t = truncf(v);
    float frac = v - t; /* exact for |v| < 2^23 */
    if (fabsf(frac) >= 0.5f)
        t += (v > 0.0f) ? 1.0f : -1.0f;
    return t;
}

void ref_quantize_q8_0(const float* v, int64_t n, int8_t* q, float* d)
{
    for (int64_t b = 0; b < n / 32; ++b) {
        const float* blk = v + 32 * b;
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
            float a = fabsf(blk[i]);
            if (a > amax)
                amax = a;
        }
        float scale = amax / 127.0f;
        float inv = (amax == 0.0f) ? 0.0f : 1.0f / scale;
        d[b] = scale;
        for (int i = 0; i < 32; ++i) {
            float r = ref_round_half_away(blk[i] * inv);
            if (r > 127.0f)
                r = 127.0f;
            if (r < -127.0f)
                r = -127.0f;
            q[32 * b + i] = (int8_t)r;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Weight containers ([DIVE] 5.1 for int4; int2 by the same MSB-first rule)  */
/* ------------------------------------------------------------------------ */

int32_t ref_row_bytes(int32_t K, int32_t bits)
{
    return (int32_t)(((int64_t)K * bits) / 8);
}

int32_t ref_weight_code(const uint8_t* row, int32_t bits, int32_t col)
{
    if (bits == 8)
        return (int32_t)(int8_t)row[col];
    if (bits == 4) {
        uint8_t byte = row[col / 2];
        int32_t nib = (col % 2 == 0) ? (byte >> 4) : (byte & 0x0F);
        return nib >= 8 ? nib - 16 : nib;
    }
    /* bits == 2 */
    uint8_t byte = row[col / 4];
    int32_t shift = 6 - 2 * (col % 4);
    int32_t v = (byte >> shift) & 0x03;
    return v >= 2 ? v - 4 : v;
}

void ref_pack_row(const int8_t* codes, int32_t K, int32_t bits, uint8_t* out)
{
    int32_t nbytes = ref_row_bytes(K, bits);
    memset(out, 0, (size_t)nbytes);
    for (int32_t col = 0; col < K; ++col) {
        int32_t c = codes[col];
        if (bits == 8) {
            out[col] = (uint8_t)(int8_t)c;
        } else if (bits == 4) {
            uint8_t nib = (uint8_t)(c & 0x0F);
            out[col / 2] |= (col % 2 == 0) ? (uint8_t)(nib << 4) : nib;
        } else {
            uint8_t v = (uint8_t)(c & 0x03);
            out[col / 4] |= (uint8_t)(v << (6 - 2 * (col % 4)));
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Integer dot path ([README] integer dot-product and quantised-kernel items) */
/* ------------------------------------------------------------------------ */

int32_t ref_block_partial(const uint8_t* row, int32_t bits, const int8_t* q, int32_t b)
{
    int32_t sum = 0;
    for (int32_t i = 0; i < 32; ++i) {
        int32_t col = 32 * b + i;
        sum += ref_weight_code(row, bits, col) * (int32_t)q[col];
    }
    return sum;
}

float ref_qdot(const uint8_t* row, int32_t bits, float row_scale,
               const int8_t* q, const float* d, int32_t K)
{
    /* The pages do not fix the order of the fp32 accumulation; the plain
     * reading is the sum written out: one fused multiply-add per block, in
     * ascending block order, starting from +0, then the row scale. */
    float acc = 0.0f;
    for (int32_t b = 0; b < K / 32; ++b) {
        int32_t part = ref_block_partial(row, bits, q, b);
        acc = fmaf(d[b], (float)part, acc);
    }
    return row_scale * acc;
}

float ref_qdot_grouped(const uint8_t* row, int32_t bits, const float* s, int32_t group,
                       const int8_t* q, const float* d, int32_t K)
{
    /* Group-wise weight scales, as ref_qdot but with block b's coefficient
     * s[32b / group] * d_b (one fp32 multiply) and no row scale.  The pages
     * name group-wise scaling without fixing its layout or where the scale
     * enters; this reading puts it where the activation block scale already
     * enters, so that a group of 32 columns is exactly a Q8_0 block. */
    float acc = 0.0f;
    for (int32_t b = 0; b < K / 32; ++b) {
        int32_t part = ref_block_partial(row, bits, q, b);
        float t = s[(b * 32) / group] * d[b];
        acc = fmaf(t, (float)part, acc);
    }
    return acc;
}

double ref_qdot_grouped_f64(const uint8_t* row, int32_t bits, const float* s, int32_t group,
                            const int8_t* q, const float* d, int32_t K)
{
    double acc = 0.0;
    for (int32_t col = 0; col < K; ++col)
        acc += (double)s[col / group] * (double)ref_weight_code(row, bits, col) * (double)q[col] *
               (double)d[col / 32];
    return acc;
}

double ref_qdot_f64(const uint8_t* row, int32_t bits, float row_scale,
                    const int8_t* q, const float* d, int32_t K)
{
    double acc = 0.0;
    for (int32_t col = 0; col < K; ++col)
        acc += (double)ref_weight_code(row, bits, col) * (double)q[col] * (double)d[col / 32];
    return (double)row_scale * acc;
}

/* ------------------------------------------------------------------------ */
/* exp and SiLU ([README] Metal section: the routed-expert work is a SwiGLU) */
/* exp(z) = 2^n * exp(r), n = nearest integer to z/ln2, r = z - n*ln2 taken  */
/* in two steps (Cody & Waite 1980) with ln2 split into a 16-significant-bit */
/* head (so n*head is exact for |n| <= 128) and an fp32 tail; exp(r) by the  */
/* degree-7 Taylor polynomial, coefficients 1/j! rounded to fp32, Horner     */
/* with fmaf.                                                                */
/* ------------------------------------------------------------------------ */

float ref_cexp(float z)
{
    if (z > 88.0f)
        return INFINITY;
    if (z < -87.0f)
        return 0.0f;
    const double ln2 = 0.69314718055994530942;
    const float log2e = (float)(1.0 / ln2);
    const float ln2_hi = (float)(floor(ln2 * 65536.0 + 0.5) / 65536.0);
    const float ln2_lo = (float)(ln2 - (double)ln2_hi);
    float n = rintf(z * log2e);
    float r = fmaf(-n, ln2_hi, z);
    r = fmaf(-n, ln2_lo, r);
    double fact = 1.0;
    float coef[8];
    for (int j = 0; j < 8; ++j) {
        if (j > 0)
            fact *= (double)j;
        coef[j] = (float)(1.0 / fact);
    }
    float p = coef[7];
    for (int j = 6; j >= 0; --j)
        p = fmaf(p, r, coef[j]);
    return ldexpf(p, (int)n);
}

float ref_silu(float g)
{
    return g / (1.0f + ref_cexp(-g));
}

void ref_cexp_array(const float* z, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = ref_cexp(z[i]);
}

void ref_silu_array(const float* g, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = ref_silu(g[i]);
}

/* ------------------------------------------------------------------------ */
/* One expert applied to one token: g = gate.x, u = up.x, h = silu(g) * u,   */
/* h re-quantised Q8_0 along I, y = down.h.                                  */
/* ------------------------------------------------------------------------ */

static const uint8_t* bank_row(const ref_bank* B, int32_t m, int32_t r)
{
    return B->mat_data[m] + (int64_t)r * ref_row_bytes(B->K, B->bits);
}

/* Row r of matrix m dotted with Q8_0 activations, per-row or group-wise
 * scales as the bank holds them. */
static float bank_dot(const ref_bank* B, int32_t m, int32_t r, const int8_t* q, const float* d)
{
    if (B->group > 0)
        return ref_qdot_grouped(bank_row(B, m, r), B->bits, B->mat_scale[m] + (int64_t)r * (B->K / B->group),
                                B->group, q, d, B->K);
    return ref_qdot(bank_row(B, m, r), B->bits, B->mat_scale[m][r], q, d, B->K);
}

int ref_expert_ffn(const ref_bank* gate, const ref_bank* up, const ref_bank* down,
                   int32_t e, const int8_t* xq, const float* xd,
                   float* g_out, float* u_out, float* h_out, int8_t* hq_out, float* hd_out,
                   float* y)
{
    if (e < 0 || e >= gate->n_mat || e >= up->n_mat || e >= down->n_mat)
        return REF_E_INVAL;
    if (!gate->mat_data[e] || !up->mat_data[e] || !down->mat_data[e] ||
        !gate->mat_scale[e] || !up->mat_scale[e] || !down->mat_scale[e])
        return REF_E_MISSING;
    const ref_bank* banks[3] = {gate, up, down};
    for (int32_t j = 0; j < 3; ++j)
        if (banks[j]->group < 0 || (banks[j]->group > 0 && (banks[j]->group % 32 || banks[j]->K % banks[j]->group)))
            return REF_E_INVAL;
    int32_t I = gate->rows, H = gate->K;
    float* h = (float*)malloc(sizeof(float) * (size_t)I);
    int8_t* hq = (int8_t*)malloc((size_t)I);
    float* hd = (float*)malloc(sizeof(float) * (size_t)(I / 32));
    for (int32_t i = 0; i < I; ++i) {
        float g = bank_dot(gate, e, i, xq, xd);
        float u = bank_dot(up, e, i, xq, xd);
        h[i] = ref_silu(g) * u;
        if (g_out)
            g_out[i] = g;
        if (u_out)
            u_out[i] = u;
    }
    ref_quantize_q8_0(h, I, hq, hd);
    for (int32_t n = 0; n < H; ++n)
        y[n] = bank_dot(down, e, n, hq, hd);
    if (h_out)
        memcpy(h_out, h, sizeof(float) * (size_t)I);
    if (hq_out)
        memcpy(hq_out, hq, (size_t)I);
    if (hd_out)
        memcpy(hd_out, hd, sizeof(float) * (size_t)(I / 32));
    free(h);
    free(hq);
    free(hd);
    return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Router ([README] sigmoid-router item: DeepSeek-V3 style sigmoid scores,    */
/* noaux_tc selection bias, routed_scaling_factor).  One group (the configs  */
/* give no group parameters), bias used for selection only.                  */
/* ------------------------------------------------------------------------ */

/* Group stage of group-limited selection (DeepSeek-V3's noaux_tc routing,
 * restated): marks eligible[e] for the experts of the topk_group groups with
 * the largest top-2 sums of c; returns the kept/dropped group-score margin
 * (+inf when every group is kept). */
static float group_stage(const float* c, int32_t E, int32_t n_group, int32_t topk_group, char* eligible)
{
    const int32_t gsz = E / n_group;
    float* score = (float*)malloc(sizeof(float) * (size_t)n_group);
    char* kept = (char*)calloc((size_t)n_group, 1);
    for (int32_t g = 0; g < n_group; ++g) {
        /* the two largest c of the group (a repeated maximum counts twice) */
        float first = -INFINITY, second = -INFINITY;
        for (int32_t e = g * gsz; e < (g + 1) * gsz; ++e) {
            if (c[e] > first) {
                second = first;
                first = c[e];
            } else if (c[e] > second) {
                second = c[e];
            }
        }
        score[g] = first + second;
    }
    for (int32_t r = 0; r < topk_group; ++r) {
        int32_t best = -1;
        for (int32_t g = 0; g < n_group; ++g)
            if (!kept[g] && (best < 0 || score[g] > score[best]))
                best = g; /* strict '>' keeps the lower group on ties */
        kept[best] = 1;
    }
    float worst_kept = INFINITY, best_dropped = -INFINITY;
    for (int32_t g = 0; g < n_group; ++g) {
        if (kept[g] && score[g] < worst_kept)
            worst_kept = score[g];
        if (!kept[g] && score[g] > best_dropped)
            best_dropped = score[g];
    }
    for (int32_t e = 0; e < E; ++e)
        eligible[e] = kept[e / gsz];
    free(score);
    free(kept);
    return topk_group == n_group ? INFINITY : worst_kept - best_dropped;
}

int ref_route_token(const float* x, int32_t H, int32_t E, int32_t k,
                    const float* router_w, const float* bias, float rsf,
                    int32_t* ids, double* w, float* s_out, float* c_out, float* gap)
{
    return ref_route_token_opt(x, H, E, k, router_w, bias, rsf, NULL, ids, w, s_out, c_out, gap);
}

int ref_route_token_opt(const float* x, int32_t H, int32_t E, int32_t k,
                        const float* router_w, const float* bias, float rsf,
                        const ref_route_opts* opt, int32_t* ids, double* w, float* s_out,
                        float* c_out, float* gap)
{
    const int32_t n_group = (opt && opt->n_group > 1) ? opt->n_group : 1;
    const int32_t topk_group = n_group > 1 ? opt->topk_group : 1;
    const float top_p = (opt && opt->top_p > 0.0f && opt->top_p < 1.0f) ? opt->top_p : 1.0f;
    if (k < 1 || k > E)
        return REF_E_INVAL;
    if (n_group > 1 && (E % n_group || E / n_group < 2 || topk_group < 1 || topk_group > n_group ||
                        k > topk_group * (E / n_group)))
        return REF_E_INVAL;
    float* s = (float*)malloc(sizeof(float) * (size_t)E);
    float* c = (float*)malloc(sizeof(float) * (size_t)E);
    char* taken = (char*)calloc((size_t)E, 1);
    char* eligible = (char*)malloc((size_t)E);
    for (int32_t e = 0; e < E; ++e) {
        double acc = 0.0;
        for (int32_t i = 0; i < H; ++i)
            acc += (double)x[i] * (double)router_w[(int64_t)e * H + i];
        float logit = (float)acc;
        s[e] = 1.0f / (1.0f + expf(-logit));
        c[e] = s[e] + bias[e];
        eligible[e] = 1;
    }
    float margin = INFINITY;
    if (n_group > 1)
        margin = group_stage(c, E, n_group, topk_group, eligible);
    for (int32_t j = 0; j < k; ++j) {
        int32_t best = -1;
        for (int32_t e = 0; e < E; ++e) {
            if (taken[e] || !eligible[e])
                continue;
            if (best < 0 || c[e] > c[best])
                best = e; /* strict '>' keeps the lower id on ties */
        }
        taken[best] = 1;
        ids[j] = best;
    }
    {
        float best_rest = -INFINITY;
        for (int32_t e = 0; e < E; ++e)
            if (eligible[e] && !taken[e] && c[e] > best_rest)
                best_rest = c[e];
        const float g = c[ids[k - 1]] - best_rest; /* +inf when nothing is left */
        if (g < margin)
            margin = g;
    }
    /* adaptive top-p: decisions in fp32 */
    char* kept = (char*)malloc((size_t)k);
    for (int32_t j = 0; j < k; ++j)
        kept[j] = 1;
    if (top_p < 1.0f) {
        float den = 0.0f;
        for (int32_t j = 0; j < k; ++j)
            den = den + s[ids[j]];
        int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
        for (int32_t j = 0; j < k; ++j) {
            /* insertion by s descending; equal s keep slot order */
            int32_t i = j;
            while (i > 0 && s[ids[order[i - 1]]] < s[ids[j]]) {
                order[i] = order[i - 1];
                --i;
            }
            order[i] = j;
        }
        float cum = 0.0f, prev = 0.0f;
        int32_t m = 0;
        while (m < k) {
            prev = cum;
            cum = cum + s[ids[order[m]]] / den;
            ++m;
            if (cum >= top_p)
                break;
        }
        for (int32_t j = 0; j < k; ++j)
            kept[j] = 0;
        for (int32_t i = 0; i < m; ++i)
            kept[order[i]] = 1;
        /* margins: one slot fewer stays below top_p; the cut slot reaches it */
        float mp = top_p - prev;
        if (cum >= top_p && cum - top_p < mp)
            mp = cum - top_p;
        if (mp < margin)
            margin = mp;
        free(order);
    }
    if (gap)
        *gap = margin;
    double denom = 0.0;
    for (int32_t j = 0; j < k; ++j)
        if (kept[j])
            denom += (double)s[ids[j]];
    for (int32_t j = 0; j < k; ++j) {
        if (kept[j]) {
            w[j] = (double)rsf * ((double)s[ids[j]] / denom);
        } else {
            w[j] = 0.0;
            ids[j] = -1;
        }
    }
    free(kept);
    free(eligible);
    if (s_out)
        memcpy(s_out, s, sizeof(float) * (size_t)E);
    if (c_out)
        memcpy(c_out, c, sizeof(float) * (size_t)E);
    free(s);
    free(c);
    free(taken);
    return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Union dispatch ([README] batched-union MoE item: each expert present in   */
/* the batch is read once and applied to every position routed to it).      */
/* ------------------------------------------------------------------------ */

void ref_dispatch(const int32_t* ids, int32_t S, int32_t k, int32_t E,
                  int32_t* offsets, int32_t* sorted, int32_t* inv,
                  int32_t* active, int32_t* n_active)
{
    int32_t P = S * k;
    int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    for (int32_t e = 0; e <= E; ++e)
        offsets[e] = 0;
    for (int32_t p = 0; p < P; ++p)
        if (ids[p] >= 0)
            offsets[ids[p] + 1] += 1;
    for (int32_t e = 0; e < E; ++e)
        offsets[e + 1] += offsets[e];
    for (int32_t p = 0; p < P; ++p) {
        int32_t e = ids[p];
        if (e < 0) {
            if (inv)
                inv[p] = -1;
            continue;
        }
        int32_t pos = offsets[e] + fill[e];
        fill[e] += 1;
        sorted[pos] = p;
        if (inv)
            inv[p] = pos;
    }
    int32_t na = 0;
    for (int32_t e = 0; e < E; ++e)
        if (offsets[e + 1] > offsets[e])
            active[na++] = e;
    *n_active = na;
    free(fill);
}

/* ------------------------------------------------------------------------ */
/* Whole layer ([DIVE] 4.3: shared expert output plus the routing-weighted   */
/* sum of the selected experts' outputs).                                    */
/* ------------------------------------------------------------------------ */

int ref_moe_layer_forward(const ref_layer* L, const float* x, int32_t S, double* out,
                          int8_t* xq_tr, float* xd_tr, int32_t* ids_tr, double* w_tr,
                          float* y_routed, float* y_shared)
{
    int32_t H = L->hidden, I = L->inter, E = L->n_experts, k = L->top_k;
    if (S < 0 || H <= 0 || I <= 0 || H % 32 || I % 32 || k < 1 || k > E)
        return REF_E_INVAL;
    int8_t* xq = (int8_t*)malloc((size_t)H);
    float* xd = (float*)malloc(sizeof(float) * (size_t)(H / 32));
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    double* w = (double*)malloc(sizeof(double) * (size_t)k);
    float* y = (float*)malloc(sizeof(float) * (size_t)H);
    int status = REF_OK;
    for (int32_t t = 0; t < S && status == REF_OK; ++t) {
        const float* xt = x + (int64_t)t * H;
        double* ot = out + (int64_t)t * H;
        ref_quantize_q8_0(xt, H, xq, xd);
        status = ref_route_token_opt(xt, H, E, k, L->router_w, L->router_bias,
                                     L->routed_scaling_factor, &L->route, ids, w, NULL, NULL, NULL);
        if (status != REF_OK)
            break;
        for (int32_t n = 0; n < H; ++n)
            ot[n] = 0.0;
        if (L->has_shared) {
            status = ref_expert_ffn(&L->sh_gate, &L->sh_up, &L->sh_down, 0, xq, xd,
                                    NULL, NULL, NULL, NULL, NULL, y);
            if (status != REF_OK)
                break;
            for (int32_t n = 0; n < H; ++n)
                ot[n] = (double)y[n];
            if (y_shared)
                memcpy(y_shared + (int64_t)t * H, y, sizeof(float) * (size_t)H);
        }
        for (int32_t j = 0; j < k && status == REF_OK; ++j) {
            if (ids[j] < 0) { /* slot dropped by top-p */
                if (y_routed)
                    memset(y_routed + ((int64_t)t * k + j) * H, 0, sizeof(float) * (size_t)H);
                continue;
            }
            status = ref_expert_ffn(&L->gate, &L->up, &L->down, ids[j], xq, xd,
                                    NULL, NULL, NULL, NULL, NULL, y);
            if (status != REF_OK)
                break;
            for (int32_t n = 0; n < H; ++n)
                ot[n] += w[j] * (double)y[n];
            if (y_routed)
                memcpy(y_routed + ((int64_t)t * k + j) * H, y, sizeof(float) * (size_t)H);
        }
        if (xq_tr)
            memcpy(xq_tr + (int64_t)t * H, xq, (size_t)H);
        if (xd_tr)
            memcpy(xd_tr + (int64_t)t * (H / 32), xd, sizeof(float) * (size_t)(H / 32));
        if (ids_tr)
            memcpy(ids_tr + (int64_t)t * k, ids, sizeof(int32_t) * (size_t)k);
        if (w_tr)
            memcpy(w_tr + (int64_t)t * k, w, sizeof(double) * (size_t)k);
    }
    free(xq);
    free(xd);
    free(ids);
    free(w);
    free(y);
    return status;
}
