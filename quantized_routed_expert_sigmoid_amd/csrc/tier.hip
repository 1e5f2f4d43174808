/*
 * tier.hip -- tiered expert residency (colibri_tier_* of the C ABI): the
 * routed experts of one layer live in pinned host memory, a slot bank in HBM
 * caches some of them, and the layer forward streams the misses in over PCIe
 * while the resident experts compute.
 *
 * The placement follows "Show HN: 如何在我的低配置电脑上运行 GLM-5.2",
 * section "思路" (idea: a per-layer LRU cache over a slower store, with an
 * optional pinned hot set) and its paragraph on the deferred cold-expert
 * pipeline (resident experts run while the missing ones load in the
 * background; the late results join before the layer completes).  There the
 * tiers are RAM over disk; here they are HBM over pinned host memory, and the
 * loads are copy-engine transfers on a stream of their own.
 *
 * One forward:
 *   1. quantise + router + selection on the caller's stream (the kernels of
 *      the resident forward); the routed ids go to pinned host staging and
 *      the host waits for the stream;
 *   2. the slot cache plans the batch (expert_cache.cpp): pair codes (pass,
 *      slot), loads and passes; the codes go back to the device;
 *   3. pass 0 -- dispatch of the resident experts' pairs over the slot bank,
 *      FFN over those pairs and the shared expert -- runs on the caller's
 *      stream at once; the copy stream loads the misses, each load waiting
 *      only for the pass that still reads its slot's previous occupant;
 *   4. pass j >= 1 waits for its loads, dispatches its pairs (inv continues
 *      where the previous passes stopped) and runs the FFN;
 *   5. one combine over every pass's rows, in slot order as in the resident
 *      forward, so the output is the resident forward's bit for bit.
 */
#include "expert_cache.h"
#include "layer.h"

#include <new>
#include <vector>

using namespace coli;

static_assert(kPassSlotBits == COLI_PLAN_SLOT_BITS, "pair code layouts differ");

namespace {

/* Bytes of one row of K weights of `qtype` bits. */
size_t row_bytes(int32_t K, int32_t qtype)
{
    return (size_t)K * qtype / 8;
}

struct SlotLayout {
    size_t gate, gate_s, up, up_s, down, down_s, total;
};

SlotLayout slot_layout(const coli_moe_layer* L, int32_t n_slots)
{
    const int32_t H = L->hidden, I = L->inter;
    Bump b;
    SlotLayout s;
    s.gate = b.take((size_t)n_slots * I * row_bytes(H, L->gate.qtype));
    s.gate_s = b.take((size_t)n_slots * I * 4);
    s.up = b.take((size_t)n_slots * I * row_bytes(H, L->up.qtype));
    s.up_s = b.take((size_t)n_slots * I * 4);
    s.down = b.take((size_t)n_slots * H * row_bytes(I, L->down.qtype));
    s.down_s = b.take((size_t)n_slots * H * 4);
    s.total = b.at;
    return s;
}

/* Pinned host memory or device memory: what a copy engine reads
 * asynchronously. */
bool transferable(const void* p)
{
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError(); /* clear the sticky error of a pageable pointer */
        return false;
    }
    return a.type == hipMemoryTypeHost || a.type == hipMemoryTypeDevice ||
           a.type == hipMemoryTypeManaged;
}

struct TierLayout {
    Layout l;
    size_t codes, total;
};

TierLayout tier_layout(const coli_moe_layer* L, int32_t S)
{
    TierLayout t;
    t.l = layer_layout(L->hidden, L->inter, L->n_experts, L->top_k, S, L->has_shared != 0);
    Bump b;
    b.at = t.l.total;
    t.codes = b.take((size_t)S * L->top_k * 4);
    t.total = b.at;
    return t;
}

} // namespace

struct coli_tier {
    coli_moe_layer L;          /* slow-tier routed banks, device router and shared expert */
    coli_qbank slot[3];        /* gate, up, down slot banks (n_mat = n_slots) */
    coli_expert_cache cache;
    int device = -1;
    hipStream_t copy = nullptr;
    std::vector<hipEvent_t> ev_pass, ev_load;
    int32_t* h_ids = nullptr;  /* pinned staging, h_cap pairs */
    int32_t* h_codes = nullptr;
    int64_t h_cap = 0;
    std::vector<coli_cache_load> loads;
    std::vector<int32_t> pass_pairs;

    coli_tier(const coli_moe_layer& l, int32_t n_slots) : L(l), cache(l.n_experts, n_slots) {}

    /* Grows staging, plan arrays and event pools for P pairs. */
    hipError_t reserve(int64_t P, hipStream_t s)
    {
        const int64_t m = P < L.n_experts ? P : L.n_experts;
        if ((int64_t)loads.size() < m)
            loads.resize(m);
        if ((int64_t)pass_pairs.size() < m + 1)
            pass_pairs.resize(m + 1);
        while ((int64_t)ev_pass.size() < m + 1) {
            hipEvent_t a, b;
            hipError_t e = hipEventCreateWithFlags(&a, hipEventDisableTiming);
            if (e != hipSuccess)
                return e;
            e = hipEventCreateWithFlags(&b, hipEventDisableTiming);
            if (e != hipSuccess) {
                (void)hipEventDestroy(a);
                return e;
            }
            ev_pass.push_back(a);
            ev_load.push_back(b);
        }
        if (P <= h_cap)
            return hipSuccess;
        /* the previous call's transfers from the old staging may be pending */
        hipError_t e = hipStreamSynchronize(s);
        if (e != hipSuccess)
            return e;
        free_staging();
        if ((e = hipHostMalloc((void**)&h_ids, (size_t)P * 4, hipHostMallocDefault)) != hipSuccess)
            return e;
        if ((e = hipHostMalloc((void**)&h_codes, (size_t)P * 4, hipHostMallocDefault)) != hipSuccess)
            return e;
        h_cap = P;
        return hipSuccess;
    }

    void free_staging()
    {
        if (h_ids)
            (void)hipHostFree(h_ids);
        if (h_codes)
            (void)hipHostFree(h_codes);
        h_ids = h_codes = nullptr;
        h_cap = 0;
    }

    /* Copies expert e's gate, up and down codes and scales into slot s. */
    hipError_t load(int32_t e, int32_t s, hipStream_t st) const
    {
        const coli_qbank* src[3] = {&L.gate, &L.up, &L.down};
        for (int m = 0; m < 3; ++m) {
            const coli_qbank& a = *src[m];
            const coli_qbank& d = slot[m];
            const size_t rb = row_bytes(a.K, a.qtype) * a.rows;
            hipError_t r = hipMemcpyAsync((char*)d.data + (size_t)s * rb,
                                          (const char*)a.data + (size_t)e * rb, rb, hipMemcpyDefault, st);
            if (r == hipSuccess)
                r = hipMemcpyAsync((float*)d.row_scale + (size_t)s * a.rows,
                                   a.row_scale + (size_t)e * a.rows, (size_t)a.rows * 4,
                                   hipMemcpyDefault, st);
            if (r != hipSuccess)
                return r;
        }
        return hipSuccess;
    }
};

namespace {

int check_current_device(const coli_tier* t)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return COLI_E_HIP;
    return dev == t->device ? COLI_OK : COLI_E_INVAL;
}

/* The routed and shared FFN of one pass; `shared` only in pass 0. */
hipError_t run_pass(const coli_tier* t, const TierLayout& Lo, void* ws, const int32_t* codes, int32_t pass,
                    int32_t base, int32_t S, bool with_routed, bool with_shared, hipStream_t s)
{
    const coli_moe_layer* L = &t->L;
    const int32_t H = L->hidden, I = L->inter, E = L->n_experts, k = L->top_k;
    const int32_t P = S * k;
    const int32_t n_slots = t->cache.n_slots();
    int32_t* offsets = at<int32_t>(ws, Lo.l.offsets);
    int32_t* sorted = at<int32_t>(ws, Lo.l.sorted);
    UnitLists ul;
    ul.units = at<Unit>(ws, Lo.l.units);
    ul.n_units = at<int32_t>(ws, Lo.l.n_units);
    ul.max_units = max_gemv_units(P, E);
    ul.munits = at<Unit>(ws, Lo.l.munits);
    ul.n_munits = at<int32_t>(ws, Lo.l.n_munits);
    ul.max_munits = max_mfma_units(P, E, S);

    hipError_t e = launch_dispatch_pass(codes, pass, base, S, k, n_slots, offsets, sorted,
                                        at<int32_t>(ws, Lo.l.inv), at<int32_t>(ws, Lo.l.active),
                                        at<int32_t>(ws, Lo.l.n_active), ul, s);
    FfnArgs a;
    a.seg[0] = make_seg(&t->slot[0], &t->slot[1], &t->slot[2], sorted, &ul, k, S, P, base);
    a.nseg = with_routed ? 1 : 0;
    a.unit_tokens = S == 1 ? 1 : kUnitTokens;
    a.H = H;
    a.I = I;
    a.xq = at<int8_t>(ws, Lo.l.xq);
    a.xd = at<float>(ws, Lo.l.xd);
    a.hq = at<int8_t>(ws, Lo.l.hq);
    a.hd = at<float>(ws, Lo.l.hd);
    a.y = at<float>(ws, Lo.l.y);
    FfnArgs b = a;
    b.nseg = 0;
    if (with_shared) {
        const FfnSeg sh = make_seg(&L->sh_gate, &L->sh_up, &L->sh_down, nullptr, nullptr, 1, S, S, P);
        if (L->sh_gate.qtype == t->slot[0].qtype && L->sh_down.qtype == t->slot[2].qtype) {
            if (a.nseg == 1) {
                a.seg[1] = sh;
                a.nseg = 2;
            } else {
                a.seg[0] = sh;
                a.nseg = 1;
            }
        } else {
            b.seg[0] = sh;
            b.nseg = 1;
        }
    }
    if (e == hipSuccess && a.nseg)
        e = run_ffn(a, t->slot[0].qtype, t->slot[2].qtype, s);
    if (e == hipSuccess && b.nseg)
        e = run_ffn(b, L->sh_gate.qtype, L->sh_down.qtype, s);
    return e;
}

} // namespace

extern "C" {

size_t colibri_tier_slot_bytes(const coli_moe_layer* L, int32_t n_slots)
{
    if (check_layer(L) || n_slots < 1 || n_slots > L->n_experts)
        return 0;
    return slot_layout(L, n_slots).total;
}

int colibri_tier_create(const coli_moe_layer* L, int32_t n_slots, void* slot_mem, size_t slot_bytes,
                        coli_tier** out)
{
    if (!out)
        return COLI_E_INVAL;
    *out = nullptr;
    int st = check_layer(L);
    if (st)
        return st;
    if (n_slots < 1 || n_slots > L->n_experts || !slot_mem)
        return COLI_E_INVAL;
    if (!aligned(slot_mem, kAlign))
        return COLI_E_UNSUPPORTED;
    const SlotLayout sl = slot_layout(L, n_slots);
    if (slot_bytes < sl.total)
        return COLI_E_WORKSPACE;
    const void* slow[6] = {L->gate.data, L->gate.row_scale, L->up.data,
                           L->up.row_scale, L->down.data, L->down.row_scale};
    for (const void* p : slow)
        if (!transferable(p))
            return COLI_E_UNSUPPORTED;

    coli_tier* t = new (std::nothrow) coli_tier(*L, n_slots);
    if (!t)
        return COLI_E_INVAL;
    const coli_qbank* src[3] = {&L->gate, &L->up, &L->down};
    const size_t off[3][2] = {{sl.gate, sl.gate_s}, {sl.up, sl.up_s}, {sl.down, sl.down_s}};
    for (int m = 0; m < 3; ++m) {
        t->slot[m] = *src[m];
        t->slot[m].n_mat = n_slots;
        t->slot[m].data = at<uint8_t>(slot_mem, off[m][0]);
        t->slot[m].row_scale = at<float>(slot_mem, off[m][1]);
    }
    if (hipGetDevice(&t->device) != hipSuccess ||
        hipStreamCreateWithFlags(&t->copy, hipStreamNonBlocking) != hipSuccess) {
        t->copy = nullptr;
        colibri_tier_destroy(t);
        return COLI_E_HIP;
    }
    *out = t;
    return COLI_OK;
}

void colibri_tier_destroy(coli_tier* t)
{
    if (!t)
        return;
    if (t->copy) {
        (void)hipStreamSynchronize(t->copy);
        (void)hipStreamDestroy(t->copy);
    }
    for (hipEvent_t e : t->ev_pass)
        (void)hipEventDestroy(e);
    for (hipEvent_t e : t->ev_load)
        (void)hipEventDestroy(e);
    t->free_staging();
    delete t;
}

const coli_expert_cache* colibri_tier_cache(const coli_tier* t)
{
    return t ? &t->cache : nullptr;
}

int colibri_tier_pin(coli_tier* t, const int32_t* experts, int32_t n, coli_stream_t stream)
{
    if (!t)
        return COLI_E_INVAL;
    int st = check_current_device(t);
    if (st)
        return st;
    std::vector<coli_cache_load> loads(n > 0 ? n : 0);
    int32_t n_load = 0;
    if ((st = t->cache.pin(experts, n, loads.data(), &n_load)))
        return st;
    hipError_t e = hipSuccess;
    for (int32_t i = 0; i < n_load && e == hipSuccess; ++i)
        e = t->load(loads[i].expert, loads[i].slot, (hipStream_t)stream);
    if (e != hipSuccess) {
        t->cache.reset();
        return COLI_E_HIP;
    }
    return COLI_OK;
}

size_t colibri_tier_workspace_bytes(const coli_tier* t, int32_t S)
{
    if (!t || check_tokens(S, t->L.top_k))
        return 0;
    return tier_layout(&t->L, S).total;
}

int colibri_tier_forward(coli_tier* t, const float* x, int32_t S, float* out, void* ws, size_t ws_bytes,
                         coli_stream_t stream)
{
    if (!t)
        return COLI_E_INVAL;
    const coli_moe_layer* L = &t->L;
    int st = check_tokens(S, L->top_k);
    if (st)
        return st;
    if (S == 0)
        return COLI_OK;
    if (!x || !out || !ws)
        return COLI_E_INVAL;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(ws, kAlign))
        return COLI_E_UNSUPPORTED;
    if ((st = check_current_device(t)))
        return st;
    const TierLayout Lo = tier_layout(L, S);
    if (ws_bytes < Lo.total)
        return COLI_E_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    const int32_t H = L->hidden, E = L->n_experts, k = L->top_k;
    const int32_t P = S * k;
    int8_t* xq = at<int8_t>(ws, Lo.l.xq);
    float* xd = at<float>(ws, Lo.l.xd);
    float* logits = at<float>(ws, Lo.l.logits);
    int32_t* ids = at<int32_t>(ws, Lo.l.ids);
    float* w = at<float>(ws, Lo.l.w);
    int32_t* codes = at<int32_t>(ws, Lo.codes);

    hipError_t e = t->reserve(P, s);
    if (e != hipSuccess)
        return COLI_E_HIP;

    /* 1. route */
    e = S <= kSmallS ? launch_route_prep_small(x, S, H, E, L->router_w, logits, xq, xd, s)
                     : launch_quantize_q8_0(x, (int64_t)S * (H / 32), xq, xd, s);
    if (e == hipSuccess && S > kSmallS)
        e = launch_router_logits(x, S, H, E, L->router_w, logits, s);
    if (e == hipSuccess)
        e = launch_router_select(logits, router_parts(S, E, H), L->router_bias, S, E, k,
                                 L->routed_scaling_factor, route_opts(L), ids, w, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(t->h_ids, ids, (size_t)P * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipStreamSynchronize(s);
    if (e != hipSuccess)
        return COLI_E_HIP;

    /* 2. plan */
    coli_cache_plan plan;
    if ((st = t->cache.plan(t->h_ids, P, t->h_codes, t->loads.data(), t->pass_pairs.data(), &plan)))
        return st; /* ids out of range cannot come from the router; nothing was enqueued */
    e = hipMemcpyAsync(codes, t->h_codes, (size_t)P * 4, hipMemcpyHostToDevice, s);

    /* 3. pass 0 at once */
    const bool shared = L->has_shared != 0;
    if (e == hipSuccess)
        e = run_pass(t, Lo, ws, codes, 0, 0, S, t->pass_pairs[0] > 0, shared, s);
    if (e == hipSuccess)
        e = hipEventRecord(t->ev_pass[0], s);

    /* 4. later passes, each after its loads */
    int32_t li = 0, waited = -1, base = t->pass_pairs[0];
    for (int32_t j = 1; j < plan.n_pass && e == hipSuccess; ++j) {
        for (; li < plan.n_load && t->loads[li].pass == j && e == hipSuccess; ++li) {
            const coli_cache_load& ld = t->loads[li];
            if (ld.after > waited) {
                e = hipStreamWaitEvent(t->copy, t->ev_pass[ld.after], 0);
                waited = ld.after;
            }
            if (e == hipSuccess)
                e = t->load(ld.expert, ld.slot, t->copy);
        }
        if (e == hipSuccess)
            e = hipEventRecord(t->ev_load[j], t->copy);
        if (e == hipSuccess)
            e = hipStreamWaitEvent(s, t->ev_load[j], 0);
        if (e == hipSuccess)
            e = run_pass(t, Lo, ws, codes, j, base, S, true, false, s);
        if (e == hipSuccess)
            e = hipEventRecord(t->ev_pass[j], s);
        base += t->pass_pairs[j];
    }

    /* 5. combine over every pass's rows */
    if (e == hipSuccess)
        e = launch_combine(at<float>(ws, Lo.l.y), at<int32_t>(ws, Lo.l.inv), ids, w, S, k, H,
                           shared ? P : -1, out, s);
    if (e != hipSuccess) {
        t->cache.reset();
        return COLI_E_HIP;
    }
    return COLI_OK;
}

} // extern "C"
