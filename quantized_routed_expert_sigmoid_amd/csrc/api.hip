/*
 * api.hip -- the C ABI of libcolibri (declared in include/colibri.h): argument
 * validation, workspace layout and launch sequencing on the caller's stream.
 * Validation happens before anything is enqueued; nothing here synchronises
 * or allocates.
 */
#include "../../include/colibri.h"
#include "kernels.h"

#include <stdint.h>

using namespace coli;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v)
{
    return (v + kAlign - 1) & ~(kAlign - 1);
}

bool aligned(const void* p, size_t a)
{
    return ((uintptr_t)p % a) == 0;
}

int check_bank(const coli_qbank* b, int32_t n_mat, int32_t rows, int32_t K)
{
    if (!b || !b->data || !b->row_scale)
        return COLI_E_INVAL;
    if (b->n_mat != n_mat || b->rows != rows || b->K != K)
        return COLI_E_INVAL;
    if (b->qtype != COLI_Q8 && b->qtype != COLI_Q4 && b->qtype != COLI_Q2)
        return COLI_E_UNSUPPORTED;
    if (!aligned(b->data, 16) || !aligned(b->row_scale, 4))
        return COLI_E_UNSUPPORTED;
    return COLI_OK;
}

int check_dims(int32_t H, int32_t I)
{
    if (H <= 0 || I <= 0 || H % 32 != 0 || I % 32 != 0)
        return COLI_E_INVAL;
    if (H > COLI_MAX_DIM || I > COLI_MAX_DIM)
        return COLI_E_UNSUPPORTED;
    return COLI_OK;
}

int check_layer(const coli_moe_layer* L)
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
    if (L->gate.qtype != L->up.qtype)
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
        if (L->sh_gate.qtype != L->sh_up.qtype)
            return COLI_E_UNSUPPORTED;
    }
    return COLI_OK;
}

int check_tokens(int32_t S, int32_t k)
{
    if (S < 0)
        return COLI_E_INVAL;
    if (S > COLI_MAX_TOKENS || (int64_t)S * k > COLI_MAX_PAIRS)
        return COLI_E_UNSUPPORTED;
    return COLI_OK;
}

RouteOpts route_opts(const coli_moe_layer* L)
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

Layout layer_layout(int32_t H, int32_t I, int32_t E, int32_t k, int32_t S, bool shared)
{
    const int64_t P = (int64_t)S * k;
    const int64_t rows = P + (shared ? S : 0);
    Bump b;
    Layout L;
    L.logits = b.take((size_t)router_parts(S, E, H) * S * E * 4);
    L.units = b.take((size_t)max_gemv_units(P, E) * sizeof(Unit));
    L.n_units = b.take(16);
    L.munits = b.take((size_t)max_mfma_units(P, E, S) * sizeof(Unit));
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
int32_t ffn_max_munits(int64_t rows, int32_t n_mat)
{
    return max_mfma_units(rows, n_mat, kMfmaMinTokens);
}

FfnLayout ffn_layout(int32_t H, int32_t I, int32_t n_mat, int32_t S, int32_t k)
{
    (void)H;
    const int64_t rows = (int64_t)S * k;
    Bump b;
    FfnLayout L;
    L.units = b.take((size_t)max_gemv_units(rows, n_mat) * sizeof(Unit));
    L.n_units = b.take(16);
    L.munits = b.take((size_t)ffn_max_munits(rows, n_mat) * sizeof(Unit));
    L.n_munits = b.take(16);
    L.hq = b.take((size_t)rows * I);
    L.hd = b.take((size_t)rows * (I / 32) * 4);
    L.total = b.at;
    return L;
}

template <typename T>
T* at(void* ws, size_t off)
{
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int hip_status(hipError_t e)
{
    return e == hipSuccess ? COLI_OK : COLI_E_HIP;
}

/* A routed group (ul != nullptr: unit lists from the dispatch or schedule
 * kernel) or the identity group of the shared expert (ul == nullptr). */
FfnSeg make_seg(const coli_qbank* g, const coli_qbank* u, const coli_qbank* d, const int32_t* sorted,
                const UnitLists* ul, int32_t k, int32_t S, int32_t rows, int32_t out_base)
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
    s.max_units = ul ? ul->max_units : identity_gemv_units(S);
    s.max_munits = ul ? ul->max_munits : identity_mfma_units(S);
    s.k = k;
    s.out_base = out_base;
    s.S = S;
    s.rows = rows;
    s.n_mat = g->n_mat;
    return s;
}

/* gate/up then down, each with both kernel families (a family with no
 * possible unit launches nothing). */
hipError_t run_ffn(const FfnArgs& a, int32_t bits_gu, int32_t bits_d, hipStream_t s)
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

} // namespace

extern "C" {

const char* colibri_status_string(int status)
{
    switch (status) {
    case COLI_OK: return "ok";
    case COLI_E_INVAL: return "invalid argument";
    case COLI_E_UNSUPPORTED: return "unsupported argument (qtype, alignment or size limit)";
    case COLI_E_WORKSPACE: return "workspace too small";
    case COLI_E_HIP: return "HIP launch error";
    default: return "unknown status";
    }
}

size_t colibri_workspace_bytes(const coli_moe_layer* L, int32_t S)
{
    if (check_layer(L) || check_tokens(S, L->top_k))
        return 0;
    return layer_layout(L->hidden, L->inter, L->n_experts, L->top_k, S, L->has_shared != 0).total;
}

size_t colibri_expert_ffn_workspace_bytes(const coli_qbank* gate, const coli_qbank* down, int32_t S,
                                          int32_t k)
{
    if (!gate || !down || k < 1 || check_tokens(S, k))
        return 0;
    const int32_t H = gate->K, I = gate->rows;
    if (check_dims(H, I) || down->rows != H || down->K != I || gate->n_mat < 1 ||
        gate->n_mat > COLI_MAX_EXPERTS)
        return 0;
    return ffn_layout(H, I, gate->n_mat, S, k).total;
}

int colibri_quantize_q8_0(const float* x, int32_t rows, int32_t K, int8_t* q, float* d,
                          coli_stream_t stream)
{
    if (rows < 0 || K <= 0 || K % 32 != 0)
        return COLI_E_INVAL;
    if (rows == 0)
        return COLI_OK;
    if (!x || !q || !d)
        return COLI_E_INVAL;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(d, 4))
        return COLI_E_UNSUPPORTED;
    const int64_t nblk = (int64_t)rows * (K / 32);
    return hip_status(launch_quantize_q8_0(x, nblk, q, d, (hipStream_t)stream));
}

int colibri_route(const coli_moe_layer* L, const float* x, int32_t S, int32_t* topk_ids,
                  float* topk_w, void* ws, size_t ws_bytes, coli_stream_t stream)
{
    int st = check_layer(L);
    if (st || (st = check_tokens(S, L->top_k)))
        return st;
    if (S == 0)
        return COLI_OK;
    if (!x || !topk_ids || !topk_w || !ws)
        return COLI_E_INVAL;
    if (!aligned(x, 16) || !aligned(ws, kAlign))
        return COLI_E_UNSUPPORTED;
    const Layout Lo = layer_layout(L->hidden, L->inter, L->n_experts, L->top_k, S, L->has_shared != 0);
    if (ws_bytes < Lo.total)
        return COLI_E_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    float* logits = at<float>(ws, Lo.logits);
    hipError_t e = launch_router_logits(x, S, L->hidden, L->n_experts, L->router_w, logits, s);
    if (e == hipSuccess)
        e = launch_router_select(logits, router_parts(S, L->n_experts, L->hidden), L->router_bias, S,
                                 L->n_experts, L->top_k, L->routed_scaling_factor, route_opts(L), topk_ids,
                                 topk_w, s);
    return hip_status(e);
}

int colibri_moe_dispatch(const int32_t* topk_ids, int32_t S, int32_t k, int32_t E,
                         int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* active_experts,
                         int32_t* n_active, void* ws, size_t ws_bytes, coli_stream_t stream)
{
    (void)ws;
    (void)ws_bytes;
    if (S < 0 || k < 1 || E < 1 || k > E)
        return COLI_E_INVAL;
    if (E > COLI_MAX_EXPERTS || k > COLI_MAX_TOPK)
        return COLI_E_UNSUPPORTED;
    int st = check_tokens(S, k);
    if (st)
        return st;
    if (!expert_offsets || !active_experts || !n_active || (S > 0 && (!topk_ids || !sorted_pairs)))
        return COLI_E_INVAL;
    return hip_status(launch_dispatch(topk_ids, S, k, E, expert_offsets, sorted_pairs, nullptr,
                                      active_experts, n_active, nullptr, (hipStream_t)stream));
}

int colibri_expert_ffn_q(const coli_qbank* gate, const coli_qbank* up, const coli_qbank* down,
                         const int8_t* xq, const float* xd, int32_t S, const int32_t* expert_offsets,
                         const int32_t* sorted_pairs, int32_t k, float* y, void* ws, size_t ws_bytes,
                         coli_stream_t stream)
{
    if (!gate || !up || !down || k < 1)
        return COLI_E_INVAL;
    if (k > COLI_MAX_TOPK)
        return COLI_E_UNSUPPORTED;
    int st = check_tokens(S, k);
    if (st)
        return st;
    const int32_t H = gate->K, I = gate->rows, n_mat = gate->n_mat;
    if ((st = check_dims(H, I)))
        return st;
    if (n_mat < 1)
        return COLI_E_INVAL;
    if (n_mat > COLI_MAX_EXPERTS)
        return COLI_E_UNSUPPORTED;
    if ((st = check_bank(gate, n_mat, I, H)) || (st = check_bank(up, n_mat, I, H)) ||
        (st = check_bank(down, n_mat, H, I)))
        return st;
    if (gate->qtype != up->qtype)
        return COLI_E_UNSUPPORTED;
    if (S == 0)
        return COLI_OK;
    if (!xq || !xd || !expert_offsets || !sorted_pairs || !y || !ws)
        return COLI_E_INVAL;
    if (!aligned(xq, 16) || !aligned(xd, 4) || !aligned(y, 16) || !aligned(ws, kAlign))
        return COLI_E_UNSUPPORTED;
    const FfnLayout Lo = ffn_layout(H, I, n_mat, S, k);
    if (ws_bytes < Lo.total)
        return COLI_E_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    const int32_t rows = S * k;
    UnitLists ul;
    ul.units = at<Unit>(ws, Lo.units);
    ul.n_units = at<int32_t>(ws, Lo.n_units);
    ul.max_units = max_gemv_units(rows, n_mat);
    ul.munits = at<Unit>(ws, Lo.munits);
    ul.n_munits = at<int32_t>(ws, Lo.n_munits);
    ul.max_munits = ffn_max_munits(rows, n_mat);
    hipError_t e = launch_schedule(expert_offsets, n_mat, ul, s);
    FfnArgs a;
    a.seg[0] = make_seg(gate, up, down, sorted_pairs, &ul, k, S, rows, 0);
    a.seg[1] = a.seg[0];
    a.nseg = 1;
    a.unit_tokens = kUnitTokens; /* caller offsets: units may hold several tokens */
    a.H = H;
    a.I = I;
    a.xq = xq;
    a.xd = xd;
    a.hq = at<int8_t>(ws, Lo.hq);
    a.hd = at<float>(ws, Lo.hd);
    a.y = y;
    if (e == hipSuccess)
        e = run_ffn(a, gate->qtype, down->qtype, s);
    return hip_status(e);
}

int colibri_moe_layer_forward(const coli_moe_layer* L, const float* x, int32_t S, float* out,
                              void* ws, size_t ws_bytes, coli_stream_t stream)
{
    return colibri_moe_layer_forward_staged(L, x, S, out, ws, ws_bytes, stream, nullptr);
}

int colibri_moe_layer_forward_staged(const coli_moe_layer* L, const float* x, int32_t S, float* out,
                                     void* ws, size_t ws_bytes, coli_stream_t stream,
                                     void* const* stage_events)
{
    int st = check_layer(L);
    if (st || (st = check_tokens(S, L->top_k)))
        return st;
    if (S == 0)
        return COLI_OK;
    if (!x || !out || !ws)
        return COLI_E_INVAL;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(ws, kAlign))
        return COLI_E_UNSUPPORTED;
    const int32_t H = L->hidden, I = L->inter, E = L->n_experts, k = L->top_k;
    const bool shared = L->has_shared != 0;
    const Layout Lo = layer_layout(H, I, E, k, S, shared);
    if (ws_bytes < Lo.total)
        return COLI_E_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    const int32_t P = S * k;

    int8_t* xq = at<int8_t>(ws, Lo.xq);
    float* xd = at<float>(ws, Lo.xd);
    float* logits = at<float>(ws, Lo.logits);
    int32_t* ids = at<int32_t>(ws, Lo.ids);
    float* w = at<float>(ws, Lo.w);
    int32_t* offsets = at<int32_t>(ws, Lo.offsets);
    int32_t* sorted = at<int32_t>(ws, Lo.sorted);
    int32_t* inv = at<int32_t>(ws, Lo.inv);
    int32_t* active = at<int32_t>(ws, Lo.active);
    int32_t* n_active = at<int32_t>(ws, Lo.n_active);
    UnitLists ul;
    ul.units = at<Unit>(ws, Lo.units);
    ul.n_units = at<int32_t>(ws, Lo.n_units);
    ul.max_units = max_gemv_units(P, E);
    ul.munits = at<Unit>(ws, Lo.munits);
    ul.n_munits = at<int32_t>(ws, Lo.n_munits);
    ul.max_munits = max_mfma_units(P, E, S);
    float* y = at<float>(ws, Lo.y);

    auto mark = [&](int i, hipError_t prev) -> hipError_t {
        if (prev != hipSuccess || !stage_events)
            return prev;
        return hipEventRecord((hipEvent_t)stage_events[i], s);
    };
    FfnArgs a;
    a.seg[0] = make_seg(&L->gate, &L->up, &L->down, sorted, &ul, k, S, P, 0);
    a.nseg = 1;
    a.unit_tokens = S == 1 ? 1 : kUnitTokens; /* distinct experts per token */
    a.H = H;
    a.I = I;
    a.xq = xq;
    a.xd = xd;
    a.hq = at<int8_t>(ws, Lo.hq);
    a.hd = at<float>(ws, Lo.hd);
    a.y = y;
    FfnArgs b = a; /* shared expert, when it cannot share the routed launch */
    if (shared) {
        FfnSeg sh = make_seg(&L->sh_gate, &L->sh_up, &L->sh_down, nullptr, nullptr, 1, S, S, P);
        if (L->sh_gate.qtype == L->gate.qtype && L->sh_down.qtype == L->down.qtype) {
            a.seg[1] = sh;
            a.nseg = 2;
            b.nseg = 0;
        } else {
            b.seg[0] = sh;
            b.nseg = 1;
        }
    } else {
        b.nseg = 0;
    }

    /* One token whose shared expert (if any) runs in the routed launches:
     * router logits with quantisation, selection with gate/up, down, combine. */
    const bool one_token = S == 1 && b.nseg == 0;

    hipError_t e = mark(0, hipSuccess);
    if (e == hipSuccess)
        e = S <= kSmallS
                ? launch_route_prep_small(x, S, H, E, L->router_w, logits, xq, xd, s)
                : launch_quantize_q8_0(x, (int64_t)S * (H / 32), xq, xd, s);
    if (e == hipSuccess && S > kSmallS)
        e = launch_router_logits(x, S, H, E, L->router_w, logits, s);
    if (e == hipSuccess && S > kSmallS)
        e = launch_router_select(logits, router_parts(S, E, H), L->router_bias, S, E, k,
                                 L->routed_scaling_factor, route_opts(L), ids, w, s);
    e = mark(1, e);
    if (one_token) {
        DecodeArgs dd;
        dd.f = a;
        dd.logits = logits;
        dd.bias = L->router_bias;
        dd.E = E;
        dd.k = k;
        dd.rsf = L->routed_scaling_factor;
        dd.opt = route_opts(L);
        dd.ids = ids;
        dd.w = w;
        dd.out = out;
        e = mark(2, e);
        if (e == hipSuccess)
            e = launch_ffn_gate_up_decode(dd, L->gate.qtype, s);
        e = mark(3, e);
        if (down_combine_decode_fits(dd)) {
            /* down and combine in one launch: the combine stage is empty */
            if (e == hipSuccess)
                e = launch_ffn_down_combine_decode(dd, L->down.qtype, s);
            e = mark(4, e);
        } else {
            if (e == hipSuccess)
                e = launch_ffn_down_decode(dd, L->down.qtype, s);
            e = mark(4, e);
            if (e == hipSuccess)
                e = launch_combine(y, nullptr, ids, w, 1, k, H, shared ? k : -1, out, s);
        }
        e = mark(5, e);
        return hip_status(e);
    }
    if (e == hipSuccess)
        e = S <= kSmallS
                ? launch_select_dispatch_small(logits, L->router_bias, S, E, k, L->routed_scaling_factor,
                                               route_opts(L), ids, w, offsets, sorted, inv, active,
                                               n_active, ul, s)
                : launch_dispatch(ids, S, k, E, offsets, sorted, inv, active, n_active, &ul, s);
    e = mark(2, e);

    if (e == hipSuccess)
        e = launch_ffn_gate_up(a, L->gate.qtype, s);
    if (e == hipSuccess)
        e = launch_ffn_gate_up_mfma(a, L->gate.qtype, s);
    if (e == hipSuccess && b.nseg)
        e = launch_ffn_gate_up(b, L->sh_gate.qtype, s);
    if (e == hipSuccess && b.nseg)
        e = launch_ffn_gate_up_mfma(b, L->sh_gate.qtype, s);
    e = mark(3, e);
    if (e == hipSuccess)
        e = launch_ffn_down(a, L->down.qtype, s);
    if (e == hipSuccess)
        e = launch_ffn_down_mfma(a, L->down.qtype, s);
    if (e == hipSuccess && b.nseg)
        e = launch_ffn_down(b, L->sh_down.qtype, s);
    if (e == hipSuccess && b.nseg)
        e = launch_ffn_down_mfma(b, L->sh_down.qtype, s);
    e = mark(4, e);
    if (e == hipSuccess)
        e = launch_combine(y, inv, ids, w, S, k, H, shared ? P : -1, out, s);
    e = mark(5, e);
    return hip_status(e);
}

} // extern "C"
