/*
 * api.hip -- the C ABI of libcolibri (declared in include/colibri.h): argument
 * validation, workspace layout and launch sequencing on the caller's stream.
 * Validation happens before anything is enqueued; nothing here synchronises
 * or allocates.
 */
#include "layer.h"

#include <mutex>
#include <stdint.h>

using namespace coli;

namespace {

/* Workspace of colibri_moe_layer_forward_noalloc: one static array per GPU
 * (each device holds its own copy).  In host code `scratch` names a host-side
 * stand-in, not device memory: only the address that hipGetSymbolAddress
 * returns for the current device may reach a kernel or a copy. */
static __device__ __align__(256) uint8_t scratch[COLI_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_at[kMaxDevices]; /* the array's address on each device, once looked up */

/* The array's address on the current device (looked up on the first call
 * there, with that device current), or null. */
void* scratch_address()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_at[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return nullptr;
        g_scratch_at[dev] = p;
    }
    return g_scratch_at[dev];
}

} // namespace

#ifdef COLI_DEBUG_PARTIALS
namespace coli {
DebugSlice g_debug_slice = {nullptr, 0, 0, 0, 0, 0, 0};
}
#endif

namespace coli {

hipError_t one_token_forward(const coli_moe_layer* L, const FfnArgs& a, const float* x, int8_t* xq, float* xd,
                             float* logits, int32_t* ids, float* w, float* out, const int32_t* slot_of,
                             void* const* stage_events, hipStream_t s, const TierState* note_hits, bool* noted)
{
    const int32_t H = L->hidden, I = L->inter, E = L->n_experts, k = L->top_k;
    const bool shared = a.nseg > 1;
    auto mark = [&](int i, hipError_t prev) -> hipError_t {
        if (prev != hipSuccess || !stage_events)
            return prev;
        return hipEventRecord((hipEvent_t)stage_events[i], s);
    };
    hipError_t e = mark(0, hipSuccess);
    if (e == hipSuccess)
        e = launch_route_prep_small(x, 1, H, E, L->router_w, logits, xq, xd, s);
    e = mark(1, e);
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
    dd.hs = nullptr;
    dd.slot_of = slot_of;
    dd.note_hits = 0;
    dd.ts = TierState{};
    const bool fused = down_combine_decode_fits(dd);
    if (note_hits && fused) {
        dd.note_hits = 1;
        dd.ts = *note_hits;
    }
    if (noted)
        *noted = dd.note_hits != 0;
    /* With the fused down + combine (which writes no y rows), the shared
     * expert's gate/up runs as one-wave jobs spread over every CU, its fp32 h
     * in the y region: the routed jobs then give each CU the same share.
     * Per-row scales only. */
    if (fused && shared && a.seg[1].gu_gb == 0 && I % 8 == 0 && I <= 2048 && (int64_t)(k + 1) * H >= I)
        dd.hs = a.y;
    e = mark(2, e);
    if (e == hipSuccess)
        e = launch_ffn_gate_up_decode(dd, L->gate.qtype, s);
    e = mark(3, e);
    if (fused) {
        /* down and combine in one launch: the combine stage is empty */
        if (e == hipSuccess)
            e = launch_ffn_down_combine_decode(dd, L->down.qtype, s);
        e = mark(4, e);
    } else {
        if (e == hipSuccess)
            e = launch_ffn_down_decode(dd, L->down.qtype, s);
        e = mark(4, e);
        if (e == hipSuccess)
            e = launch_combine(a.y, nullptr, ids, w, 1, k, H, shared ? k : -1, out, s);
    }
    return mark(5, e);
}

} // namespace coli

extern "C" {

const char* colibri_status_string(int status)
{
    switch (status) {
    case COLI_OK: return "ok";
    case COLI_E_INVAL: return "invalid argument";
    case COLI_E_UNSUPPORTED: return "unsupported argument (qtype, alignment or size limit)";
    case COLI_E_WORKSPACE: return "workspace too small";
    case COLI_E_HIP: return "HIP launch error";
    case COLI_E_SCRATCH: return "batch workspace exceeds the static scratch of the allocation-free forward";
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
    if (gate->qtype != up->qtype || gate->group != up->group)
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
    ul.max_units = max_gemv_units(rows, n_mat, kMfmaMinTokens);
    ul.munits = at<Unit>(ws, Lo.munits);
    ul.n_munits = at<int32_t>(ws, Lo.n_munits);
    ul.max_munits = ffn_max_munits(rows, n_mat);
    ul.mfma_min = kMfmaMinTokens;
    hipError_t e = launch_schedule(expert_offsets, n_mat, ul, s);
    FfnArgs a;
    debug_attach(a);
    a.seg[0] = make_seg(gate, up, down, sorted_pairs, &ul, k, S, rows, 0, ul.mfma_min);
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
    const UnitLists ul = layer_unit_lists(ws, Lo, P, E, S);
    float* y = at<float>(ws, Lo.y);

    auto mark = [&](int i, hipError_t prev) -> hipError_t {
        if (prev != hipSuccess || !stage_events)
            return prev;
        return hipEventRecord((hipEvent_t)stage_events[i], s);
    };
    FfnArgs a;
    debug_attach(a);
    a.seg[0] = make_seg(&L->gate, &L->up, &L->down, sorted, &ul, k, S, P, 0, ul.mfma_min);
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
        FfnSeg sh = make_seg(&L->sh_gate, &L->sh_up, &L->sh_down, nullptr, nullptr, 1, S, S, P, ul.mfma_min);
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
    if (one_token)
        return hip_status(one_token_forward(L, a, x, xq, xd, logits, ids, w, out, nullptr, stage_events, s));

    hipError_t e = mark(0, hipSuccess);
    if (e == hipSuccess)
        e = launch_route_prep(x, S, H, E, L->router_w, logits, xq, xd, s);
    if (e == hipSuccess && S > kSmallS)
        e = launch_router_select(logits, router_parts(S, E, H), L->router_bias, S, E, k,
                                 L->routed_scaling_factor, route_opts(L), ids, w, s);
    e = mark(1, e);
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

int colibri_moe_layer_forward_noalloc(const coli_moe_layer* L, const float* x, int32_t S, float* out,
                                      coli_stream_t stream)
{
    int st = check_layer(L);
    if (st || (st = check_tokens(S, L->top_k)))
        return st;
    if (S == 0)
        return COLI_OK;
    if (!x || !out)
        return COLI_E_INVAL;
    const size_t need =
        layer_layout(L->hidden, L->inter, L->n_experts, L->top_k, S, L->has_shared != 0).total;
    if (need > COLI_NOALLOC_SCRATCH_BYTES)
        return COLI_E_SCRATCH;
    void* ws = scratch_address();
    if (!ws)
        return COLI_E_HIP;
    return colibri_moe_layer_forward(L, x, S, out, ws, COLI_NOALLOC_SCRATCH_BYTES, stream);
}

#ifdef COLI_DEBUG_PARTIALS
int colibri_debug_partials(int32_t* out, int32_t kind, int32_t o0, int32_t o1, int32_t r0, int32_t r1, int32_t nb)
{
    if (out && (kind < kDbgGate || kind > kDbgDown || o1 < o0 || r1 < r0 || nb < 0))
        return COLI_E_INVAL;
    g_debug_slice = DebugSlice{out, kind, o0, o1, r0, r1, nb};
    return COLI_OK;
}
#endif

} // extern "C"
