/*
 * layer.h -- host-side helpers shared by the C ABI's entry points (api.hip,
 * tier.hip): argument validation, workspace layout and FFN group set-up.
 */
#ifndef COLI_LAYER_H
#define COLI_LAYER_H

#include "../../include/colibri.h"
#include "kernels.h"

#include <stdint.h>

namespace coli {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v)
{
    return (v + kAlign - 1) & ~(kAlign - 1);
}

inline bool aligned(const void* p, size_t a)
{
    return ((uintptr_t)p % a) == 0;
}

inline int check_bank(const coli_qbank* b, int32_t n_mat, int32_t rows, int32_t K)
{
    if (!b || !b->data || !b->row_scale)
        return COLI_E_INVAL;
    if (b->n_mat != n_mat || b->rows != rows || b->K != K)
        return COLI_E_INVAL;
    if (b->qtype != COLI_Q8 && b->qtype != COLI_Q4 && b->qtype != COLI_Q2)
        return COLI_E_UNSUPPORTED;
    if (b->group < 0 || (b->group > 0 && (b->group % 32 != 0 || K % b->group != 0)))
        return COLI_E_INVAL;
    if (!aligned(b->data, 16) || !aligned(b->row_scale, 4))
        return COLI_E_UNSUPPORTED;
    return COLI_OK;
}

inline int check_dims(int32_t H, int32_t I)
{
    if (H <= 0 || I <= 0 || H % 32 != 0 || I % 32 != 0)
        return COLI_E_INVAL;
    if (H > COLI_MAX_DIM || I > COLI_MAX_DIM)
        return COLI_E_UNSUPPORTED;
    return COLI_OK;
}

inline int check_layer(const coli_moe_layer* L)
{
    if (!L)
        return COLI_E_INVAL;
    int st = check_dims(L->hidden, L->inter);
    if (st)
        return st;
    if (L->n_experts < 1 || L->top_k < 1 || L->top_k > L->n_experts)
        return COLI_E_INVAL;
    if (L->n_experts > COLI_MAX_EXPERTS || L->top_k > COLI_MAX_TOPK)
        return COLI_E_UNSUPPORTED;
    if (!L->router_w || !L->router_bias)
        return COLI_E_INVAL;
    if (!aligned(L->router_w, 16) || !aligned(L->router_bias, 4))
        return COLI_E_UNSUPPORTED;
    const int32_t H = L->hidden, I = L->inter, E = L->n_experts;
    if ((st = check_bank(&L->gate, E, I, H)) || (st = check_bank(&L->up, E, I, H)) ||
        (st = check_bank(&L->down, E, H, I)))
        return st;
    if (L->gate.qtype != L->up.qtype || L->gate.group != L->up.group)
        return COLI_E_UNSUPPORTED;
    if (L->n_group < 0 || !(L->top_p >= 0.0f)) /* also rejects a NaN top_p */
        return COLI_E_INVAL;
    if (L->n_group > 1) {
        const int32_t G = L->n_group;
        if (G > kMaxGroups || E % G || E / G < 2 || L->topk_group < 1 || L->topk_group > G ||
            L->top_k > L->topk_group * (E / G))
            return COLI_E_INVAL;
    }
    if (L->has_shared) {
        if ((st = check_bank(&L->sh_gate, 1, I, H)) || (st = check_bank(&L->sh_up, 1, I, H)) ||
            (st = check_bank(&L->sh_down, 1, H, I)))
            return st;
        if (L->sh_gate.qtype != L->sh_up.qtype || L->sh_gate.group != L->sh_up.group)
            return COLI_E_UNSUPPORTED;
    }
    return COLI_OK;
}

inline int check_tokens(int32_t S, int32_t k)
{
    if (S < 0)
        return COLI_E_INVAL;
    if (S > COLI_MAX_TOKENS || (int64_t)S * k > COLI_MAX_PAIRS)
        return COLI_E_UNSUPPORTED;
    return COLI_OK;
}

inline RouteOpts route_opts(const coli_moe_layer* L)
{
    RouteOpts o;
    o.n_group = L->n_group > 1 ? L->n_group : 1;
    o.topk_group = L->n_group > 1 ? L->topk_group : 1;
    o.top_p = L->top_p;
    return o;
}

/* Byte offsets of the workspace regions. */
struct Layout {
    size_t logits, units, n_units, munits, n_munits, hq, hd, xq, xd, ids, w, offsets, sorted, inv,
        active, n_active, y;
    size_t total;
};

struct Bump {
    size_t at = 0;
    size_t take(size_t bytes)
    {
        size_t r = at;
        at += align_up(bytes);
        return r;
    }
};

/* extra_rows: rows of hq / hd / y beyond the P routed rows, before the S
 * shared-expert rows. */
inline Layout layer_layout(int32_t H, int32_t I, int32_t E, int32_t k, int32_t S, bool shared,
                           int64_t extra_rows = 0)
{
    const int64_t P = (int64_t)S * k;
    const int64_t rows = P + extra_rows + (shared ? S : 0);
    const int32_t mmin = layer_mfma_min(P, E, S);
    Bump b;
    Layout L;
    L.logits = b.take((size_t)router_parts(S, E, H) * S * E * 4);
    L.units = b.take((size_t)max_gemv_units(P, E, mmin) * sizeof(Unit));
    L.n_units = b.take(16);
    L.munits = b.take((size_t)max_mfma_units(P, E, S, mmin) * sizeof(Unit));
    L.n_munits = b.take(16);
    L.hq = b.take((size_t)rows * I);
    L.hd = b.take((size_t)rows * (I / 32) * 4);
    L.xq = b.take((size_t)S * H);
    L.xd = b.take((size_t)S * (H / 32) * 4);
    L.ids = b.take((size_t)P * 4);
    L.w = b.take((size_t)P * 4);
    L.offsets = b.take((size_t)(E + 1) * 4);
    L.sorted = b.take((size_t)P * 4);
    L.inv = b.take((size_t)P * 4);
    L.active = b.take((size_t)E * 4);
    L.n_active = b.take(16);
    L.y = b.take((size_t)rows * H * 4);
    L.total = b.at;
    return L;
}

struct FfnLayout {
    size_t units, n_units, munits, n_munits, hq, hd, total;
};

/* Caller offsets may give one expert several pairs of the same token, so
 * every expert may reach the MFMA threshold: bound with the largest S. */
inline int32_t ffn_max_munits(int64_t rows, int32_t n_mat)
{
    return max_mfma_units(rows, n_mat, kMfmaMinTokens, kMfmaMinTokens);
}

inline FfnLayout ffn_layout(int32_t H, int32_t I, int32_t n_mat, int32_t S, int32_t k)
{
    (void)H;
    const int64_t rows = (int64_t)S * k;
    Bump b;
    FfnLayout L;
    L.units = b.take((size_t)max_gemv_units(rows, n_mat, kMfmaMinTokens) * sizeof(Unit));
    L.n_units = b.take(16);
    L.munits = b.take((size_t)ffn_max_munits(rows, n_mat) * sizeof(Unit));
    L.n_munits = b.take(16);
    L.hq = b.take((size_t)rows * I);
    L.hd = b.take((size_t)rows * (I / 32) * 4);
    L.total = b.at;
    return L;
}

template <typename T>
inline T* at(void* ws, size_t off)
{
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

/* The unit lists of a layer's routed batch (P pairs of S tokens over E
 * experts) in a workspace laid out by layer_layout. */
inline UnitLists layer_unit_lists(void* ws, const Layout& Lo, int64_t P, int32_t E, int32_t S)
{
    UnitLists ul;
    ul.units = at<Unit>(ws, Lo.units);
    ul.n_units = at<int32_t>(ws, Lo.n_units);
    ul.munits = at<Unit>(ws, Lo.munits);
    ul.n_munits = at<int32_t>(ws, Lo.n_munits);
    ul.mfma_min = layer_mfma_min(P, E, S);
    ul.max_units = max_gemv_units(P, E, ul.mfma_min);
    ul.max_munits = max_mfma_units(P, E, S, ul.mfma_min);
    return ul;
}

#ifdef COLI_DEBUG_PARTIALS
/* The slice of block partials the FFN kernels store (test-only build; set by
 * colibri_debug_partials). */
extern DebugSlice g_debug_slice;
#endif

/* Hands the test-only build's partial slice to a launch (nothing otherwise). */
inline void debug_attach(FfnArgs& a)
{
#ifdef COLI_DEBUG_PARTIALS
    a.dbg = g_debug_slice;
#else
    (void)a;
#endif
}

inline int hip_status(hipError_t e)
{
    return e == hipSuccess ? COLI_OK : COLI_E_HIP;
}

/* A routed group (ul != nullptr: unit lists from the dispatch or schedule
 * kernel) or the identity group of the shared expert (ul == nullptr), which
 * runs on the matrix cores when S >= mmin (the routed batch's threshold). */
inline FfnSeg make_seg(const coli_qbank* g, const coli_qbank* u, const coli_qbank* d, const int32_t* sorted,
                const UnitLists* ul, int32_t k, int32_t S, int32_t rows, int32_t out_base, int32_t mmin)
{
    FfnSeg s;
    s.gate_w = static_cast<const uint8_t*>(g->data);
    s.gate_s = g->row_scale;
    s.up_w = static_cast<const uint8_t*>(u->data);
    s.up_s = u->row_scale;
    s.down_w = static_cast<const uint8_t*>(d->data);
    s.down_s = d->row_scale;
    s.sorted = sorted;
    s.units = ul ? ul->units : nullptr;
    s.n_units = ul ? ul->n_units : nullptr;
    s.munits = ul ? ul->munits : nullptr;
    s.n_munits = ul ? ul->n_munits : nullptr;
    s.max_units = ul ? ul->max_units : identity_gemv_units(S, mmin);
    s.max_munits = ul ? ul->max_munits : identity_mfma_units(S, mmin);
    s.k = k;
    s.out_base = out_base;
    s.S = S;
    s.rows = rows;
    s.n_mat = g->n_mat;
    s.gu_gb = g->group / 32;
    s.d_gb = d->group / 32;
    return s;
}

/* gate/up then down, each with both kernel families (a family with no
 * possible unit launches nothing). */
inline hipError_t run_ffn(const FfnArgs& a, int32_t bits_gu, int32_t bits_d, hipStream_t s)
{
    hipError_t e = launch_ffn_gate_up(a, bits_gu, s);
    if (e == hipSuccess)
        e = launch_ffn_gate_up_mfma(a, bits_gu, s);
    if (e == hipSuccess)
        e = launch_ffn_down(a, bits_d, s);
    if (e == hipSuccess)
        e = launch_ffn_down_mfma(a, bits_d, s);
    return e;
}

/* The one-token forward (S = 1; a: the FFN arguments, the shared expert if
 * any in its second segment): quantise + router logits, selection with
 * gate/up, down with the combine.  slot_of: as DecodeArgs::slot_of.
 * stage_events (may be null): events 0..5 as the staged forward records
 * them.  note_hits (may be null): the slot cache of a tiered layer whose
 * experts are all resident; when the launch fuses down and combine it also
 * keeps that state as the plan kernel would for this all-hit batch, and
 * *noted says so (the caller launches the plan kernel otherwise). */
hipError_t one_token_forward(const coli_moe_layer* L, const FfnArgs& a, const float* x, int8_t* xq, float* xd,
                             float* logits, int32_t* ids, float* w, float* out, const int32_t* slot_of,
                             void* const* stage_events, hipStream_t s, const TierState* note_hits = nullptr,
                             bool* noted = nullptr);

} // namespace coli

#endif
