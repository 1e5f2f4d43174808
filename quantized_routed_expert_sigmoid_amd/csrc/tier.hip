/*
 * tier.hip -- tiered expert residency (colibri_tier_* of the C ABI): the
 * routed experts of one layer live in pinned host memory, a slot bank in HBM
 * caches some of them, and the layer forward pulls the misses in over PCIe
 * while the resident experts compute.
 *
 * The placement follows "Show HN: 如何在我的低配置电脑上运行 GLM-5.2",
 * section "思路" (idea: a per-layer LRU cache over a slower store, with an
 * optional pinned hot set) and its paragraph on the deferred cold-expert
 * pipeline (resident experts run while the missing ones load in the
 * background; the late results join before the layer completes).  There the
 * tiers are RAM over disk and the planner runs on the CPU; here they are HBM
 * over pinned host memory, the cache state lives in HBM, and both the plan
 * and the loads are kernels, so a forward needs nothing from the host.
 *
 * One forward:
 *   1. quantise + router + selection (the kernels of the resident forward);
 *   2. the plan kernel (tier_kernels.hip) gives every pair a pass and a
 *      slot, lists the loads and updates the cache state;
 *   3. pass 0 -- dispatch of the resident experts' pairs over the slot bank,
 *      FFN over those pairs and the shared expert -- runs on the caller's
 *      stream while the fetch kernel, on the tier's copy stream, pulls the
 *      misses from pinned host memory into their slots;
 *   4. pass 1 waits for the fetch.  When the unpinned slots cannot hold
 *      every expert a batch may route to, a plan may need more passes: the
 *      plan is then read back to the host once, and each later pass waits
 *      for its own fetch, which waits for the pass that last read its slots;
 *   5. one combine over every pass's rows, in slot order as in the resident
 *      forward, so the output is the resident forward's bit for bit.
 */
#include "layer.h"

#include <new>
#include <vector>

using namespace coli;

static_assert(kPassSlotBits == COLI_PLAN_SLOT_BITS, "pair code layouts differ");
static_assert(kTierMaxE == COLI_MAX_EXPERTS, "planner sized for the expert limit");

namespace {

/* Bytes of one row of K weights of `qtype` bits. */
size_t row_bytes(int32_t K, int32_t qtype)
{
    return (size_t)K * qtype / 8;
}

/* Scales per row of a bank: one, or one per column group. */
size_t scales_per_row(const coli_qbank& b)
{
    return b.group > 0 ? (size_t)(b.K / b.group) : 1;
}

/* slot_mem: the six slot-bank regions, then the cache state and the pin
 * scratch. */
struct SlotLayout {
    size_t reg[6];
    size_t hdr, slot_of, expert_in, last_use, pinned, inflight, usage, pin_experts, pin_loads, pin_info, pf_loads,
        pf_info, pf_logits, pf_xq, pf_xd, pf_ids, pf_w, total;
};

SlotLayout slot_layout(const coli_moe_layer* L, int32_t n)
{
    const int32_t H = L->hidden, I = L->inter, E = L->n_experts;
    Bump b;
    SlotLayout s;
    s.reg[0] = b.take((size_t)n * I * row_bytes(H, L->gate.qtype));
    s.reg[1] = b.take((size_t)n * I * scales_per_row(L->gate) * 4);
    s.reg[2] = b.take((size_t)n * I * row_bytes(H, L->up.qtype));
    s.reg[3] = b.take((size_t)n * I * scales_per_row(L->up) * 4);
    s.reg[4] = b.take((size_t)n * H * row_bytes(I, L->down.qtype));
    s.reg[5] = b.take((size_t)n * H * scales_per_row(L->down) * 4);
    s.hdr = b.take(sizeof(TierHdr));
    s.slot_of = b.take((size_t)E * 4);
    s.expert_in = b.take((size_t)n * 4);
    s.last_use = b.take((size_t)n * 4);
    s.pinned = b.take((size_t)n * 4);
    s.inflight = b.take((size_t)n * 4);
    s.usage = b.take((size_t)E * 8);
    s.pin_experts = b.take((size_t)kTierMaxE * 4);
    s.pin_loads = b.take((size_t)kTierMaxE * 16);
    s.pin_info = b.take((size_t)kInfoN * 4);
    s.pf_loads = b.take((size_t)kTierMaxE * 16);
    s.pf_info = b.take((size_t)kInfoN * 4);
    /* the prefetch's own routing scratch, up to kSmallS tokens */
    s.pf_logits = b.take((size_t)kSmallS * E * 4);
    s.pf_xq = b.take((size_t)kSmallS * H);
    s.pf_xd = b.take((size_t)kSmallS * (H / 32) * 4);
    s.pf_ids = b.take((size_t)kSmallS * L->top_k * 4);
    s.pf_w = b.take((size_t)kSmallS * L->top_k * 4);
    s.total = b.at;
    return s;
}

/* Per-expert bytes of the six regions (gate, gate scales, up, up scales,
 * down, down scales). */
void region_bytes(const coli_moe_layer* L, size_t out[6])
{
    const int32_t H = L->hidden, I = L->inter;
    out[0] = (size_t)I * row_bytes(H, L->gate.qtype);
    out[1] = (size_t)I * scales_per_row(L->gate) * 4;
    out[2] = (size_t)I * row_bytes(H, L->up.qtype);
    out[3] = (size_t)I * scales_per_row(L->up) * 4;
    out[4] = (size_t)H * row_bytes(I, L->down.qtype);
    out[5] = (size_t)H * scales_per_row(L->down) * 4;
}

/* The device address of slow-tier memory: pinned host memory (mapped into
 * the device's address space) or device memory; nullptr otherwise. */
const void* device_view(const void* p)
{
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError(); /* clear the error a pageable pointer leaves */
        return nullptr;
    }
    if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged)
        return p;
    if (a.type == hipMemoryTypeHost)
        return a.devicePointer ? a.devicePointer : p;
    return nullptr;
}

/* Workspace of a tiered forward: the resident layout with P more rows of
 * hq / hd / y (pass 1 writes rows P .. 2P-1, the shared expert 2P ..), then
 * the plan. */
struct TierLayout {
    Layout l;
    size_t codes, loads, info, pass_pairs, total;
};

TierLayout tier_layout(const coli_moe_layer* L, int32_t S)
{
    const int64_t P = (int64_t)S * L->top_k;
    const int64_t m = P < L->n_experts ? P : L->n_experts;
    TierLayout t;
    t.l = layer_layout(L->hidden, L->inter, L->n_experts, L->top_k, S, L->has_shared != 0, P);
    Bump b;
    b.at = t.l.total;
    t.codes = b.take((size_t)P * 4);
    t.loads = b.take((size_t)m * 16);
    t.info = b.take((size_t)kInfoN * 4);
    t.pass_pairs = b.take((size_t)(m + 1) * 4);
    t.total = b.at;
    return t;
}

} // namespace

struct coli_tier {
    coli_moe_layer L;        /* slow-tier routed banks, device router and shared expert */
    coli_qbank slot[3];      /* gate, up, down slot banks (n_mat = n_slots) */
    TierState st;
    TierBanks banks;
    size_t expert_bytes = 0;
    int32_t n_slots = 0;
    int device = -1;
    hipStream_t copy = nullptr;
    hipEvent_t ev_plan = nullptr, ev_d2h = nullptr;
    std::vector<hipEvent_t> ev_pass, ev_fetch;
    std::vector<uint8_t> pinned_e; /* host mirror of the pinned set */
    int32_t n_pinned = 0;
    int32_t* pin_experts = nullptr; /* device */
    int4* pin_loads = nullptr;
    int32_t* pin_info = nullptr;
    int4* pf_loads = nullptr;       /* device: the last prefetch's plan */
    int32_t* pf_info = nullptr;
    float* pf_logits = nullptr;     /* device: the prefetch's routing scratch */
    int8_t* pf_xq = nullptr;
    float* pf_xd = nullptr;
    int32_t* pf_ids = nullptr;
    float* pf_w = nullptr;
    hipEvent_t ev_issue = nullptr;    /* the caller's stream when a prefetch was issued */
    hipEvent_t ev_pfplan = nullptr;   /* after the last prefetch's plan */
    hipEvent_t ev_prefetch = nullptr; /* after the last prefetch's fetch */
    hipEvent_t ev_copy_tail = nullptr; /* the copy stream's work so far (verify steps) */
    bool prefetch_pending = false;    /* a prefetch fetch no forward has waited for */
    int32_t* h_buf = nullptr;       /* pinned host staging */
    size_t h_cap = 0;               /* int32 entries */

    ~coli_tier()
    {
        if (copy) {
            (void)hipStreamSynchronize(copy);
            (void)hipStreamDestroy(copy);
        }
        for (hipEvent_t e : ev_pass)
            (void)hipEventDestroy(e);
        for (hipEvent_t e : ev_fetch)
            (void)hipEventDestroy(e);
        if (ev_plan)
            (void)hipEventDestroy(ev_plan);
        if (ev_d2h)
            (void)hipEventDestroy(ev_d2h);
        if (ev_prefetch)
            (void)hipEventDestroy(ev_prefetch);
        if (ev_issue)
            (void)hipEventDestroy(ev_issue);
        if (ev_pfplan)
            (void)hipEventDestroy(ev_pfplan);
        if (ev_copy_tail)
            (void)hipEventDestroy(ev_copy_tail);
        if (h_buf)
            (void)hipHostFree(h_buf);
    }

    hipError_t events(size_t n)
    {
        while (ev_pass.size() < n) {
            hipEvent_t a, b;
            hipError_t e = hipEventCreateWithFlags(&a, hipEventDisableTiming);
            if (e != hipSuccess)
                return e;
            if ((e = hipEventCreateWithFlags(&b, hipEventDisableTiming)) != hipSuccess) {
                (void)hipEventDestroy(a);
                return e;
            }
            ev_pass.push_back(a);
            ev_fetch.push_back(b);
        }
        return hipSuccess;
    }

    /* Pinned host staging of at least n int32 entries.  Every earlier use
     * of the staging has completed when this is called. */
    hipError_t staging(size_t n)
    {
        if (n <= h_cap)
            return hipSuccess;
        if (h_buf)
            (void)hipHostFree(h_buf);
        h_buf = nullptr;
        h_cap = 0;
        hipError_t e = hipHostMalloc((void**)&h_buf, n * 4, hipHostMallocDefault);
        if (e == hipSuccess)
            h_cap = n;
        return e;
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
                    int32_t base, int32_t S, bool with_shared, hipStream_t s)
{
    const coli_moe_layer* L = &t->L;
    const int32_t H = L->hidden, I = L->inter, E = L->n_experts, k = L->top_k;
    const int32_t P = S * k;
    int32_t* sorted = at<int32_t>(ws, Lo.l.sorted);
    const UnitLists ul = layer_unit_lists(ws, Lo.l, P, E, S);

    hipError_t e = launch_dispatch_pass(codes, pass, base, S, k, t->n_slots, at<int32_t>(ws, Lo.l.offsets),
                                        sorted, at<int32_t>(ws, Lo.l.inv), at<int32_t>(ws, Lo.l.active),
                                        at<int32_t>(ws, Lo.l.n_active), ul, s);
    FfnArgs a;
    debug_attach(a);
    a.seg[0] = make_seg(&t->slot[0], &t->slot[1], &t->slot[2], sorted, &ul, k, S, P, base, ul.mfma_min);
    a.nseg = 1;
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
        const FfnSeg sh = make_seg(&L->sh_gate, &L->sh_up, &L->sh_down, nullptr, nullptr, 1, S, S, 2 * P, ul.mfma_min);
        if (L->sh_gate.qtype == t->slot[0].qtype && L->sh_down.qtype == t->slot[2].qtype) {
            a.seg[1] = sh;
            a.nseg = 2;
        } else {
            b.seg[0] = sh;
            b.nseg = 1;
        }
    }
    if (e == hipSuccess)
        e = run_ffn(a, t->slot[0].qtype, t->slot[2].qtype, s);
    if (e == hipSuccess && b.nseg)
        e = run_ffn(b, L->sh_gate.qtype, L->sh_down.qtype, s);
    return e;
}

/* Quantise + router + selection (the resident forward's kernels). */
hipError_t route_into(const coli_tier* t, const float* x, int32_t S, int8_t* xq, float* xd, float* logits,
                      int32_t* ids, float* w, hipStream_t s)
{
    const coli_moe_layer* L = &t->L;
    const int32_t H = L->hidden, E = L->n_experts, k = L->top_k;
    hipError_t e = launch_route_prep(x, S, H, E, L->router_w, logits, xq, xd, s);
    if (e == hipSuccess)
        e = launch_router_select(logits, router_parts(S, E, H), L->router_bias, S, E, k,
                                 L->routed_scaling_factor, route_opts(L), ids, w, s);
    return e;
}

/* Argument checks shared by the forward and the prefetch. */
int check_call(const coli_tier* t, const float* x, int32_t S, const float* out, bool need_out, void* ws,
               size_t ws_bytes)
{
    if (!t)
        return COLI_E_INVAL;
    int st = check_tokens(S, t->L.top_k);
    if (st || S == 0)
        return st;
    if (!x || (need_out && !out) || !ws)
        return COLI_E_INVAL;
    if (!aligned(x, 16) || (need_out && !aligned(out, 16)) || !aligned(ws, kAlign))
        return COLI_E_UNSUPPORTED;
    if ((st = check_current_device(t)))
        return st;
    if (ws_bytes < tier_layout(&t->L, S).total)
        return COLI_E_WORKSPACE;
    return COLI_OK;
}

/* First half of a look-ahead prefetch, on the tier's copy stream after the
 * work enqueued on s so far (earlier forwards of this tier included) and
 * after the previous prefetch (same stream): route x with this layer's
 * router into the tier's own scratch and plan the prefetch on the state.
 * ev_pfplan marks the end, after which x is no longer read. */
hipError_t prefetch_plan(coli_tier* t, const float* x, int32_t S, hipStream_t s)
{
    hipError_t e = hipEventRecord(t->ev_issue, s);
    if (e == hipSuccess)
        e = hipStreamWaitEvent(t->copy, t->ev_issue, 0);
    if (e == hipSuccess)
        e = route_into(t, x, S, t->pf_xq, t->pf_xd, t->pf_logits, t->pf_ids, t->pf_w, t->copy);
    if (e == hipSuccess)
        e = launch_tier_plan(t->pf_ids, S * t->L.top_k, t->st, nullptr, t->pf_loads, t->pf_info, nullptr, true,
                             t->copy);
    if (e == hipSuccess)
        e = hipEventRecord(t->ev_pfplan, t->copy);
    return e;
}

/* Second half: the planned loads, next on the copy stream; the tier's next
 * forward waits for them (for the plan only, when its misses fit two
 * passes: the loaded slots are then late hits, read after the loads). */
hipError_t prefetch_loads(coli_tier* t)
{
    hipError_t e = launch_tier_fetch(t->pf_loads, t->pf_info, 1, t->banks, t->copy);
    if (e == hipSuccess)
        e = hipEventRecord(t->ev_prefetch, t->copy);
    if (e == hipSuccess)
        t->prefetch_pending = true;
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
    if (!aligned(slot_mem, kAlign) || !aligned(L->gate.row_scale, 16) || !aligned(L->up.row_scale, 16) ||
        !aligned(L->down.row_scale, 16))
        return COLI_E_UNSUPPORTED;
    const SlotLayout sl = slot_layout(L, n_slots);
    if (slot_bytes < sl.total)
        return COLI_E_WORKSPACE;
    const void* slow[6] = {L->gate.data, L->gate.row_scale, L->up.data,
                           L->up.row_scale, L->down.data, L->down.row_scale};
    const void* view[6];
    for (int r = 0; r < 6; ++r)
        if (!(view[r] = device_view(slow[r])))
            return COLI_E_UNSUPPORTED;

    coli_tier* t = new (std::nothrow) coli_tier();
    if (!t)
        return COLI_E_INVAL;
    t->L = *L;
    t->n_slots = n_slots;
    t->pinned_e.assign(L->n_experts, 0);
    size_t rb[6];
    region_bytes(L, rb);
    const coli_qbank* src[3] = {&L->gate, &L->up, &L->down};
    for (int m = 0; m < 3; ++m) {
        t->slot[m] = *src[m];
        t->slot[m].n_mat = n_slots;
        t->slot[m].data = at<uint8_t>(slot_mem, sl.reg[2 * m]);
        t->slot[m].row_scale = at<float>(slot_mem, sl.reg[2 * m + 1]);
    }
    for (int r = 0; r < 6; ++r) {
        t->banks.src[r] = static_cast<const uint4*>(view[r]);
        t->banks.dst[r] = at<uint4>(slot_mem, sl.reg[r]);
        t->banks.len[r] = (int64_t)(rb[r] / 16);
        t->expert_bytes += rb[r];
    }
    t->st.hdr = at<TierHdr>(slot_mem, sl.hdr);
    t->st.slot_of = at<int32_t>(slot_mem, sl.slot_of);
    t->st.expert_in = at<int32_t>(slot_mem, sl.expert_in);
    t->st.last_use = at<uint32_t>(slot_mem, sl.last_use);
    t->st.pinned = at<int32_t>(slot_mem, sl.pinned);
    t->st.inflight = at<int32_t>(slot_mem, sl.inflight);
    t->st.usage = at<unsigned long long>(slot_mem, sl.usage);
    t->st.E = L->n_experts;
    t->st.n = n_slots;
    t->pin_experts = at<int32_t>(slot_mem, sl.pin_experts);
    t->pin_loads = at<int4>(slot_mem, sl.pin_loads);
    t->pin_info = at<int32_t>(slot_mem, sl.pin_info);
    t->pf_loads = at<int4>(slot_mem, sl.pf_loads);
    t->pf_info = at<int32_t>(slot_mem, sl.pf_info);
    t->pf_logits = at<float>(slot_mem, sl.pf_logits);
    t->pf_xq = at<int8_t>(slot_mem, sl.pf_xq);
    t->pf_xd = at<float>(slot_mem, sl.pf_xd);
    t->pf_ids = at<int32_t>(slot_mem, sl.pf_ids);
    t->pf_w = at<float>(slot_mem, sl.pf_w);

    hipError_t e = hipGetDevice(&t->device);
    if (e == hipSuccess)
        e = hipStreamCreateWithFlags(&t->copy, hipStreamNonBlocking);
    if (e == hipSuccess)
        e = hipEventCreateWithFlags(&t->ev_plan, hipEventDisableTiming);
    if (e == hipSuccess)
        e = hipEventCreateWithFlags(&t->ev_d2h, hipEventDisableTiming);
    if (e == hipSuccess)
        e = hipEventCreateWithFlags(&t->ev_prefetch, hipEventDisableTiming);
    if (e == hipSuccess)
        e = hipEventCreateWithFlags(&t->ev_issue, hipEventDisableTiming);
    if (e == hipSuccess)
        e = hipEventCreateWithFlags(&t->ev_pfplan, hipEventDisableTiming);
    if (e == hipSuccess)
        e = hipEventCreateWithFlags(&t->ev_copy_tail, hipEventDisableTiming);
    if (e == hipSuccess)
        e = t->events(2);
    if (e == hipSuccess)
        e = launch_tier_init(t->st, t->copy);
    if (e == hipSuccess)
        e = hipStreamSynchronize(t->copy);
    if (e != hipSuccess) {
        delete t;
        return COLI_E_HIP;
    }
    *out = t;
    return COLI_OK;
}

void colibri_tier_destroy(coli_tier* t)
{
    delete t;
}

int colibri_tier_pin(coli_tier* t, const int32_t* experts, int32_t n, coli_stream_t stream)
{
    if (!t || n < 0 || (n > 0 && !experts))
        return COLI_E_INVAL;
    int st = check_current_device(t);
    if (st || n == 0)
        return st;
    const int32_t E = t->L.n_experts;
    std::vector<uint8_t> seen(E, 0);
    int32_t fresh = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t e = experts[i];
        if (e < 0 || e >= E || seen[e])
            return COLI_E_INVAL; /* out of range or repeated */
        seen[e] = 1;
        fresh += t->pinned_e[e] ? 0 : 1;
    }
    const int32_t total = t->n_pinned + fresh;
    if (!(total <= t->n_slots - 1 || (total == E && t->n_slots == E)))
        return COLI_E_UNSUPPORTED; /* a slot has to stay free for misses */
    hipStream_t s = (hipStream_t)stream;
    /* a pending prefetch may still be filling slots the pins take */
    hipError_t e = t->prefetch_pending ? hipStreamWaitEvent(s, t->ev_prefetch, 0) : hipSuccess;
    if (e == hipSuccess)
        e = t->staging((size_t)n);
    if (e == hipSuccess) {
        for (int32_t i = 0; i < n; ++i)
            t->h_buf[i] = experts[i];
        e = hipMemcpyAsync(t->pin_experts, t->h_buf, (size_t)n * 4, hipMemcpyHostToDevice, s);
    }
    if (e == hipSuccess)
        e = launch_tier_pin(t->pin_experts, n, t->st, t->pin_loads, t->pin_info, s);
    if (e == hipSuccess)
        e = launch_tier_fetch(t->pin_loads, t->pin_info, 1, t->banks, s);
    if (e == hipSuccess)
        e = hipStreamSynchronize(s); /* the staging is free again */
    if (e != hipSuccess)
        return COLI_E_HIP;
    for (int32_t i = 0; i < n; ++i)
        t->pinned_e[experts[i]] = 1;
    t->n_pinned = total;
    return COLI_OK;
}

size_t colibri_tier_workspace_bytes(const coli_tier* t, int32_t S)
{
    if (!t || check_tokens(S, t->L.top_k))
        return 0;
    return tier_layout(&t->L, S).total;
}

int colibri_tier_prefetch(coli_tier* t, const float* x, int32_t S, coli_stream_t stream)
{
    if (!t || S < 0)
        return COLI_E_INVAL;
    if (S == 0)
        return COLI_OK;
    if (S > kSmallS)
        return COLI_E_UNSUPPORTED;
    if (!x)
        return COLI_E_INVAL;
    if (!aligned(x, 16))
        return COLI_E_UNSUPPORTED;
    int st = check_current_device(t);
    if (st)
        return st;
    hipError_t e = prefetch_plan(t, x, S, (hipStream_t)stream);
    if (e == hipSuccess)
        e = prefetch_loads(t);
    return hip_status(e);
}

int colibri_tier_forward(coli_tier* t, const float* x, int32_t S, float* out, void* ws, size_t ws_bytes,
                         coli_stream_t stream)
{
    int st = check_call(t, x, S, out, true, ws, ws_bytes);
    if (st || S == 0)
        return st;
    const coli_moe_layer* L = &t->L;
    const TierLayout Lo = tier_layout(L, S);
    hipStream_t s = (hipStream_t)stream;
    const int32_t H = L->hidden, E = L->n_experts, k = L->top_k;
    const int32_t P = S * k, m = P < E ? P : E;
    /* with every expert pinned nothing can miss: pass 0 is the whole plan;
     * otherwise every plan fits two passes when the unpinned slots can take
     * every expert of the batch */
    const bool all_pinned = t->n_pinned == E;
    const bool two_passes = all_pinned || t->n_slots - t->n_pinned >= m;
    int32_t* ids = at<int32_t>(ws, Lo.l.ids);
    float* w = at<float>(ws, Lo.l.w);
    int32_t* codes = at<int32_t>(ws, Lo.codes);
    int4* loads = at<int4>(ws, Lo.loads);
    int32_t* info = at<int32_t>(ws, Lo.info);
    int32_t* pass_pairs = at<int32_t>(ws, Lo.pass_pairs);
    const size_t n_back = kInfoN + (size_t)(m + 1) + 4 * (size_t)m; /* info, pass_pairs, loads */

    hipError_t e = two_passes ? hipSuccess : t->staging(n_back);
    if (e != hipSuccess)
        return COLI_E_HIP;

    /* Every expert pinned, one token: the resident one-token kernels, with
     * the routed experts read through the slot map (the same kernels on the
     * same weights, so the same bits).  The batch is all hits: the fused
     * down + combine keeps the cache's usage and counters as the plan kernel
     * would, which then runs only when that launch is not fused. */
    const bool shared = L->has_shared != 0;
    if (all_pinned && S == 1 &&
        (!shared || (L->sh_gate.qtype == t->slot[0].qtype && L->sh_down.qtype == t->slot[2].qtype))) {
        if (t->prefetch_pending) {
            e = hipStreamWaitEvent(s, t->ev_pfplan, 0);
            t->prefetch_pending = false;
        }
        const UnitLists ul = layer_unit_lists(ws, Lo.l, P, E, S);
        FfnArgs a;
        debug_attach(a);
        a.seg[0] = make_seg(&t->slot[0], &t->slot[1], &t->slot[2], at<int32_t>(ws, Lo.l.sorted), &ul, k, S, P, 0, ul.mfma_min);
        a.nseg = 1;
        if (shared) {
            a.seg[1] = make_seg(&L->sh_gate, &L->sh_up, &L->sh_down, nullptr, nullptr, 1, S, S, P, ul.mfma_min);
            a.nseg = 2;
        }
        a.unit_tokens = 1;
        a.H = H;
        a.I = L->inter;
        a.xq = at<int8_t>(ws, Lo.l.xq);
        a.xd = at<float>(ws, Lo.l.xd);
        a.hq = at<int8_t>(ws, Lo.l.hq);
        a.hd = at<float>(ws, Lo.l.hd);
        a.y = at<float>(ws, Lo.l.y);
        bool noted = false;
        if (e == hipSuccess)
            e = one_token_forward(L, a, x, at<int8_t>(ws, Lo.l.xq), at<float>(ws, Lo.l.xd), at<float>(ws, Lo.l.logits),
                                  ids, w, out, t->st.slot_of, nullptr, s, &t->st, &noted);
        if (e == hipSuccess && !noted)
            e = launch_tier_plan(ids, P, t->st, codes, loads, info, pass_pairs, false, s);
        if (e == hipSuccess)
            e = hipEventRecord(t->ev_plan, s);
        if (e == hipSuccess)
            e = hipStreamWaitEvent(t->copy, t->ev_plan, 0);
        return hip_status(e);
    }

    /* 1-2. route and plan, the plan after a pending prefetch's plan.  With
     * two passes the misses always fit the free slots, so the slots the
     * prefetch is still filling are late hits, read only in pass 1, which
     * follows the copy stream's loads; otherwise wait for the whole
     * prefetch */
    if (t->prefetch_pending) {
        e = hipStreamWaitEvent(s, two_passes ? t->ev_pfplan : t->ev_prefetch, 0);
        t->prefetch_pending = false;
    }
    if (e == hipSuccess)
        e = route_into(t, x, S, at<int8_t>(ws, Lo.l.xq), at<float>(ws, Lo.l.xd), at<float>(ws, Lo.l.logits),
                       ids, w, s);
    if (e == hipSuccess)
        e = launch_tier_plan(ids, P, t->st, codes, loads, info, pass_pairs, false, s);
    int32_t* h_info = t->h_buf;
    int32_t* h_pp = two_passes ? nullptr : h_info + kInfoN;
    int4* h_loads = two_passes ? nullptr : reinterpret_cast<int4*>(h_pp + (m + 1));
    if (!two_passes) {
        if (e == hipSuccess)
            e = hipMemcpyAsync(h_info, info, kInfoN * 4, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync(h_pp, pass_pairs, (size_t)(m + 1) * 4, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync(h_loads, loads, (size_t)m * 16, hipMemcpyDeviceToHost, s);
        if (e == hipSuccess)
            e = hipEventRecord(t->ev_d2h, s);
    }
    if (e == hipSuccess)
        e = hipEventRecord(t->ev_plan, s);
    if (e == hipSuccess)
        e = hipStreamWaitEvent(t->copy, t->ev_plan, 0);

    /* 3. pass 0 at once */
    if (e == hipSuccess)
        e = run_pass(t, Lo, ws, codes, 0, 0, S, shared, s);
    if (e == hipSuccess)
        e = hipEventRecord(t->ev_pass[0], s);

    /* 4. the miss passes */
    if (all_pinned) {
        /* the copy stream has waited for the plan; nothing to fetch */
    } else if (two_passes) {
        if (e == hipSuccess)
            e = launch_tier_fetch(loads, info, 1, t->banks, t->copy);
        if (e == hipSuccess)
            e = hipEventRecord(t->ev_fetch[1], t->copy);
        if (e == hipSuccess)
            e = hipStreamWaitEvent(s, t->ev_fetch[1], 0);
        if (e == hipSuccess)
            e = run_pass(t, Lo, ws, codes, 1, P, S, false, s);
    } else {
        if (e == hipSuccess)
            e = hipEventSynchronize(t->ev_d2h);
        const int32_t n_pass = e == hipSuccess ? h_info[kInfoPass] : 0;
        if (e == hipSuccess && (h_info[kInfoError] || n_pass < 1 || n_pass > m + 1))
            e = hipErrorUnknown; /* every slot pinned: excluded by the pin limit */
        if (e == hipSuccess)
            e = t->events((size_t)n_pass + 1);
        int32_t li = 0, waited = -1, base = e == hipSuccess ? h_pp[0] : 0;
        for (int32_t j = 1; j < n_pass && e == hipSuccess; ++j) {
            int32_t after = -1;
            for (; li < h_info[kInfoLoad] && h_loads[li].z == j; ++li)
                after = h_loads[li].w > after ? h_loads[li].w : after;
            if (after > waited) {
                e = hipStreamWaitEvent(t->copy, t->ev_pass[after], 0);
                waited = after;
            }
            if (e == hipSuccess)
                e = launch_tier_fetch(loads, info, j, t->banks, t->copy);
            if (e == hipSuccess)
                e = hipEventRecord(t->ev_fetch[j], t->copy);
            if (e == hipSuccess)
                e = hipStreamWaitEvent(s, t->ev_fetch[j], 0);
            if (e == hipSuccess)
                e = run_pass(t, Lo, ws, codes, j, base, S, false, s);
            if (e == hipSuccess)
                e = hipEventRecord(t->ev_pass[j], s);
            base += h_pp[j];
        }
    }

    /* 5. combine over every pass's rows */
    if (e == hipSuccess)
        e = launch_combine(at<float>(ws, Lo.l.y), at<int32_t>(ws, Lo.l.inv), ids, w, S, k, H,
                           shared ? 2 * P : -1, out, s);
    return hip_status(e);
}

int colibri_tier_verify_step(coli_tier* const* tiers, int32_t n_layers, const float* x, int32_t S, float* out,
                             int32_t lookahead, void* ws, size_t ws_bytes, uint32_t* union_mask, int32_t* stats,
                             coli_stream_t stream)
{
    if (!tiers || n_layers < 1 || S < 0)
        return COLI_E_INVAL;
    for (int32_t l = 0; l < n_layers; ++l) {
        const coli_tier* t = tiers[l];
        if (!t)
            return COLI_E_INVAL;
        const coli_moe_layer &A = tiers[0]->L, &B = t->L;
        if (B.hidden != A.hidden || B.inter != A.inter || B.n_experts != A.n_experts || B.top_k != A.top_k ||
            B.has_shared != A.has_shared)
            return COLI_E_INVAL;
        for (int32_t j = 0; j < l; ++j)
            if (tiers[j] == t)
                return COLI_E_INVAL; /* one tier per layer: a tier's prefetch and forward would interleave */
    }
    coli_tier* const t0 = tiers[0];
    int st = check_call(t0, x, S, out, true, ws, ws_bytes);
    if (st || S == 0)
        return st;
    if (!union_mask != !stats)
        return COLI_E_INVAL;
    if (lookahead && S > kSmallS)
        return COLI_E_UNSUPPORTED;
    for (int32_t l = 1; l < n_layers; ++l)
        if ((st = check_current_device(tiers[l])))
            return st;
    hipStream_t s = (hipStream_t)stream;
    const int32_t H = t0->L.hidden, E = t0->L.n_experts, k = t0->L.top_k;
    const size_t layer_elems = (size_t)S * H;
    const int32_t* ids = at<int32_t>(ws, tier_layout(&t0->L, S).l.ids);
    const int32_t nw = (E + 31) / 32;
    hipError_t e = hipSuccess;
    for (int32_t l = 0; l < n_layers && e == hipSuccess; ++l) {
        coli_tier* t = tiers[l];
        coli_tier* nxt = lookahead && l + 1 < n_layers ? tiers[l + 1] : nullptr;
        const float* xl = x + (size_t)l * layer_elems;
        /* the next layer's routing predicted from this layer's input */
        if (nxt)
            e = prefetch_plan(nxt, xl, S, s);
        if (e == hipSuccess) {
            st = colibri_tier_forward(t, xl, S, out + (size_t)l * layer_elems, ws, ws_bytes, stream);
            if (st)
                return st;
        }
        if (nxt) {
            /* the predicted loads go after this layer's own misses */
            if (e == hipSuccess)
                e = hipEventRecord(t->ev_copy_tail, t->copy);
            if (e == hipSuccess)
                e = hipStreamWaitEvent(nxt->copy, t->ev_copy_tail, 0);
            if (e == hipSuccess)
                e = prefetch_loads(nxt);
            /* work the caller enqueues later may overwrite x: it follows the
             * prediction's read */
            if (e == hipSuccess)
                e = hipStreamWaitEvent(s, nxt->ev_pfplan, 0);
        }
        if (e == hipSuccess && stats)
            e = launch_verify_union(ids, S * k, E, union_mask + (size_t)l * nw, stats + 2 * (size_t)l, s);
    }
    return hip_status(e);
}

int colibri_tier_stats(const coli_tier* t, coli_cache_stats* out, coli_stream_t stream)
{
    if (!t || !out)
        return COLI_E_INVAL;
    int st = check_current_device(t);
    if (st)
        return st;
    hipStream_t s = (hipStream_t)stream;
    TierHdr h;
    std::vector<int32_t> ein(t->n_slots);
    hipError_t e = hipMemcpyAsync(&h, t->st.hdr, sizeof h, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(ein.data(), t->st.expert_in, ein.size() * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipStreamSynchronize(s);
    if (e != hipSuccess)
        return COLI_E_HIP;
    out->plans = h.plans;
    out->pairs = h.pairs;
    out->hits = h.hits;
    out->misses = h.misses;
    out->pin_loads = h.pin_loads;
    out->passes = h.passes;
    out->prefetches = h.prefetches;
    out->prefetch_loads = h.prefetch_loads;
    out->resident = 0;
    for (const int32_t v : ein)
        out->resident += v >= 0 ? 1 : 0;
    out->pinned = t->n_pinned;
    return COLI_OK;
}

int colibri_tier_state(const coli_tier* t, int32_t* slot_of, uint64_t* usage, coli_stream_t stream)
{
    if (!t)
        return COLI_E_INVAL;
    int st = check_current_device(t);
    if (st)
        return st;
    hipStream_t s = (hipStream_t)stream;
    const size_t E = (size_t)t->L.n_experts;
    hipError_t e = hipSuccess;
    if (slot_of)
        e = hipMemcpyAsync(slot_of, t->st.slot_of, E * 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess && usage)
        e = hipMemcpyAsync(usage, t->st.usage, E * 8, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipStreamSynchronize(s);
    return hip_status(e);
}

} // extern "C"
