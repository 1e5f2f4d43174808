/*
 * tier_kernels.hip -- device side of the tiered expert store: the slot
 * cache's plan and pin steps as one-workgroup kernels over cache state kept
 * in device memory, and the fetch kernel that pulls missing experts from
 * pinned host memory over PCIe into their slots.
 *
 * The policy is the host planner's (expert_cache.cpp; per-layer LRU cache
 * with a pinned hot set, "Show HN: 如何在我的低配置电脑上运行 GLM-5.2",
 * section "思路"), restated in closed form so that one workgroup computes it
 * without a sequential pass over the misses:
 *   - distinct experts in order of first appearance (first pair index);
 *   - hits keep their slots and run in pass 0;
 *   - the ring: unpinned slots without a hit ordered by the key (empty
 *     first by index, then by last use, ties to the lower slot), followed
 *     by the unpinned hit slots by index; R slots;
 *   - miss of rank i (order of first appearance among misses) goes to ring
 *     slot i mod R in pass 1 + i / c, c = n_miss if n_miss <= R, else
 *     max(1, R / 2); it waits for the pass of miss i - R (same ring slot)
 *     when i >= R, for pass 0 when its slot held a hit, else for nothing;
 *   - each ring slot ends up holding its last miss; the occupant it held
 *     before the plan (a hit included) is evicted.
 * A look-ahead prefetch (the same page's router look-ahead paragraph: the
 * next layer's experts are predicted from the current state and read ahead)
 * plans the same way with two differences: the ring is the free slots only
 * (no slot of an expert the prediction also names is given up), and the
 * misses beyond it are not loaded; usage is not counted.  The slots a
 * prefetch loads are marked in flight.  When a plan's misses fit its free
 * slots, a hit on such a slot (a late hit) runs in pass 1, after every load,
 * and the slot stays out of the ring; every plan clears the marks.
 * A workgroup of 1024 threads holds one expert and one slot per thread
 * (both at most 1024).  Ranks are counts over LDS arrays, so every result
 * is independent of thread timing.
 */
#include "device_common.h"
#include "kernels.h"

#include <limits.h>

namespace coli {

constexpr int kPlanThreads = 1024;
static_assert(kPlanThreads == kTierMaxE, "one expert and one slot per thread");

__global__ __launch_bounds__(256) void tier_init_kernel(TierState st)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < st.E) {
        st.slot_of[i] = -1;
        st.usage[i] = 0;
    }
    if (i < st.n) {
        st.expert_in[i] = -1;
        st.last_use[i] = 0;
        st.pinned[i] = 0;
        st.inflight[i] = 0;
    }
    if (i == 0) {
        TierHdr h = {};
        *st.hdr = h;
    }
}

hipError_t launch_tier_init(const TierState& st, hipStream_t s)
{
    const int m = st.E > st.n ? st.E : st.n;
    hipLaunchKernelGGL(tier_init_kernel, dim3((m + 255) / 256), dim3(256), 0, s, st);
    return hipGetLastError();
}

/* Victim order of an unpinned slot: empty slots first (by index), then
 * occupied ones by last use, ties to the lower slot. */
__device__ __forceinline__ unsigned long long victim_key(int32_t occupant, uint32_t last_use, int32_t s)
{
    return occupant >= 0 ? (1ull << 62) | ((unsigned long long)last_use << 16) | (uint32_t)s
                         : (unsigned long long)(uint32_t)s;
}

__global__ __launch_bounds__(kPlanThreads) void tier_plan_kernel(const int32_t* __restrict__ ids, int32_t P,
                                                                 TierState st, int32_t* __restrict__ codes,
                                                                 int4* __restrict__ loads,
                                                                 int32_t* __restrict__ info,
                                                                 int32_t* __restrict__ pass_pairs,
                                                                 int32_t prefetch)
{
    __shared__ int32_t first[kTierMaxE];  /* first pair of each expert; INT_MAX: absent */
    __shared__ int32_t mfirst[kTierMaxE]; /* the same, misses only */
    __shared__ int32_t ucnt[kTierMaxE];   /* pairs per expert */
    __shared__ int32_t pass_of[kTierMaxE];
    __shared__ int32_t slot_at[kTierMaxE];
    __shared__ int32_t miss_e[kTierMaxE]; /* expert of each miss rank */
    __shared__ int32_t ring[kTierMaxE];
    __shared__ unsigned long long key[kTierMaxE];
    __shared__ uint8_t hs[kTierMaxE];     /* slot holding a hit: 1 unpinned, 3 pinned */
    __shared__ uint8_t lt[kTierMaxE];     /* slot filled by a prefetch (in flight) */
    __shared__ int32_t pcnt[kTierMaxE + 1];
    __shared__ int32_t kept;

    const int tid = threadIdx.x;
    const int32_t E = st.E, n = st.n;
    const uint32_t tick = st.hdr->tick + 1;
    first[tid] = INT_MAX;
    mfirst[tid] = INT_MAX;
    ucnt[tid] = 0;
    hs[tid] = 0;
    lt[tid] = 0;
    pcnt[tid] = 0;
    if (tid == 0) {
        pcnt[kTierMaxE] = 0;
        kept = 0;
    }
    __syncthreads();
    for (int32_t p = tid; p < P; p += kPlanThreads) {
        const int32_t e = ids[p];
        if (e >= 0 && e < E) {
            atomicMin(&first[e], p);
            atomicAdd(&ucnt[e], 1);
        }
    }
    __syncthreads();

    /* thread tid holds expert e = tid and slot s = tid */
    const int e = tid, s = tid;
    const bool present = e < E && first[e] != INT_MAX;
    const int32_t s_hit = present ? st.slot_of[e] : -1;
    const bool hit = s_hit >= 0;
    const bool miss = present && !hit;
    if (miss)
        mfirst[e] = first[e];
    if (hit) {
        hs[s_hit] = st.pinned[s_hit] ? 3 : 1;
        lt[s_hit] = (!prefetch && st.inflight[s_hit] != 0) ? 1 : 0;
    }
    __syncthreads();
    bool cand = false;
    unsigned long long k = ~0ull;
    if (s < n) {
        cand = hs[s] == 0 && !st.pinned[s];
        if (cand)
            k = victim_key(st.expert_in[s], st.last_use[s], s);
    }
    key[s] = k;
    const int32_t n_free = __syncthreads_count(cand);
    const int32_t n_hit = __syncthreads_count(hit);
    const int32_t n_miss_all = __syncthreads_count(miss);
    /* late hits only when the misses fit the free slots */
    const bool honor = !prefetch && n_miss_all <= n_free;
    const bool late = hit && honor && lt[s_hit] != 0;
    const bool is_uh = !prefetch && s < n && hs[s] == 1 && !(honor && lt[s] != 0);
    const int32_t n_uh = __syncthreads_count(is_uh);
    const int32_t n_late = __syncthreads_count(late);
    const int32_t R = n_free + n_uh;
    /* a prefetch loads only the misses that fit the free slots */
    const int32_t n_miss = prefetch ? min(n_miss_all, R) : n_miss_all;
    int32_t mrank = 0;
    if (cand) {
        int32_t r = 0;
        for (int t = 0; t < n; ++t)
            r += key[t] < k ? 1 : 0;
        ring[r] = s;
    }
    if (is_uh) {
        int32_t r = 0;
        for (int t = 0; t < s; ++t)
            r += (hs[t] == 1 && !(honor && lt[t] != 0)) ? 1 : 0;
        ring[n_free + r] = s;
    }
    if (miss) {
        const int32_t f = first[e];
        for (int t = 0; t < E; ++t)
            mrank += mfirst[t] < f ? 1 : 0;
        miss_e[mrank] = e;
    }
    __syncthreads();

    /* every slot pinned with misses pending: excluded by the host's pin limit */
    const bool error = n_miss > 0 && R == 0;
    const int32_t c = error ? 1 : (n_miss <= R ? (n_miss > 0 ? n_miss : 1) : max(1, R / 2));
    if (!error) {
        if (miss && mrank < n_miss) {
            const int32_t i = mrank, pass = 1 + i / c, r = i % R, slot = ring[r];
            const int32_t after = i < R ? (r < n_free ? -1 : 0) : 1 + (i - R) / c;
            loads[i] = make_int4(e, slot, pass, after);
            pass_of[e] = pass;
            slot_at[e] = slot;
        } else if (hit) {
            pass_of[e] = late ? 1 : 0;
            slot_at[e] = s_hit;
        }
    }
    __syncthreads();

    /* state: hits are used now; each ring slot that took misses keeps the
     * last one and evicts what it held before; a prefetch marks its loads in
     * flight, a plan consumes every mark */
    if (!error) {
        if (hit)
            st.last_use[s_hit] = tick;
        if (!prefetch && tid < n)
            st.inflight[tid] = 0;
        const int r = tid;
        if (r < R && r < n_miss) {
            const int32_t slot = ring[r];
            const int32_t old = st.expert_in[slot];
            if (old >= 0)
                st.slot_of[old] = -1;
            const int32_t en = miss_e[r + R * ((n_miss - 1 - r) / R)];
            st.slot_of[en] = slot;
            st.expert_in[slot] = en;
            st.last_use[slot] = tick;
            if (prefetch)
                st.inflight[slot] = 1;
        }
    }
    for (int32_t p = tid; p < P && !prefetch; p += kPlanThreads) {
        const int32_t ep = ids[p];
        int32_t code = -1;
        if (!error && ep >= 0 && ep < E) {
            code = (pass_of[ep] << kPassSlotBits) | slot_at[ep];
            atomicAdd(&pcnt[pass_of[ep]], 1);
        }
        codes[p] = code;
    }
    if (present && !error && !prefetch) {
        st.usage[e] += (unsigned long long)ucnt[e];
        atomicAdd(&kept, ucnt[e]);
    }
    __syncthreads();
    int32_t n_pass = (error || n_miss == 0) ? 1 : 1 + (n_miss + c - 1) / c;
    if (!error && n_late > 0 && n_pass < 2)
        n_pass = 2;
    for (int j = tid; j < n_pass && !prefetch; j += kPlanThreads)
        pass_pairs[j] = pcnt[j];
    if (tid == 0) {
        info[kInfoPass] = n_pass;
        info[kInfoLoad] = error ? 0 : n_miss;
        info[kInfoHit] = n_hit;
        info[kInfoMiss] = n_miss;
        info[kInfoChunk] = c;
        info[kInfoRing] = R;
        info[kInfoError] = error ? 1 : 0;
        if (!error) {
            TierHdr h = *st.hdr;
            h.tick = tick;
            if (prefetch) {
                h.prefetches += 1;
                h.prefetch_loads += (unsigned long long)n_miss;
            } else {
                h.plans += 1;
                h.pairs += (unsigned long long)kept;
                h.hits += (unsigned long long)n_hit;
                h.misses += (unsigned long long)n_miss;
                h.passes += (unsigned long long)n_pass;
            }
            *st.hdr = h;
        }
    }
}

hipError_t launch_tier_plan(const int32_t* ids, int32_t P, const TierState& st, int32_t* codes, int4* loads,
                            int32_t* info, int32_t* pass_pairs, bool prefetch, hipStream_t s)
{
    hipLaunchKernelGGL(tier_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, ids, P, st, codes, loads, info,
                       pass_pairs, prefetch ? 1 : 0);
    return hipGetLastError();
}

/* Pins experts one after another: a resident one keeps its slot; any other
 * takes the unpinned slot with the smallest victim key.  The host has
 * checked that the experts are distinct, in range and within the pin limit,
 * so a victim always exists.  The per-slot state is mirrored in LDS for the
 * whole kernel, and only thread 0 reads or writes slot_of, so every branch
 * that guards a barrier reads values the workgroup agrees on. */
__global__ __launch_bounds__(kPlanThreads) void tier_pin_kernel(const int32_t* __restrict__ experts,
                                                                int32_t n_pin, TierState st,
                                                                int4* __restrict__ loads,
                                                                int32_t* __restrict__ info)
{
    __shared__ unsigned long long kmin[kPlanThreads];
    __shared__ int32_t occ[kTierMaxE];
    __shared__ uint32_t lu[kTierMaxE];
    __shared__ int32_t pin[kTierMaxE];
    __shared__ int32_t nl, cur;
    const int tid = threadIdx.x;
    const int32_t n = st.n;
    const uint32_t tick = st.hdr->tick + 1;
    if (tid < n) {
        occ[tid] = st.expert_in[tid];
        lu[tid] = st.last_use[tid];
        pin[tid] = st.pinned[tid];
    }
    if (tid == 0)
        nl = 0;
    __syncthreads();
    for (int32_t i = 0; i < n_pin; ++i) {
        if (tid == 0)
            cur = st.slot_of[experts[i]];
        __syncthreads();
        int32_t slot = cur;
        if (slot < 0) {
            unsigned long long k = ~0ull;
            if (tid < n && !pin[tid])
                k = victim_key(occ[tid], lu[tid], tid);
            kmin[tid] = k;
            __syncthreads();
            for (int w = kPlanThreads / 2; w > 0; w >>= 1) {
                if (tid < w && kmin[tid + w] < kmin[tid])
                    kmin[tid] = kmin[tid + w];
                __syncthreads();
            }
            slot = (int32_t)(kmin[0] & 0xFFFF);
        }
        if (tid == 0) {
            const int32_t e = experts[i];
            if (cur < 0) {
                if (occ[slot] >= 0)
                    st.slot_of[occ[slot]] = -1;
                occ[slot] = e;
                st.slot_of[e] = slot;
                loads[nl] = make_int4(e, slot, 1, -1);
                nl = nl + 1;
            }
            pin[slot] = 1;
            lu[slot] = tick;
        }
        __syncthreads();
    }
    if (tid < n) {
        st.expert_in[tid] = occ[tid];
        st.last_use[tid] = lu[tid];
        st.pinned[tid] = pin[tid];
    }
    if (tid == 0) {
        info[kInfoPass] = 2;
        info[kInfoLoad] = nl;
        info[kInfoHit] = 0;
        info[kInfoMiss] = nl;
        info[kInfoChunk] = nl > 0 ? nl : 1;
        info[kInfoRing] = 0;
        info[kInfoError] = 0;
        TierHdr h = *st.hdr;
        h.tick = tick;
        h.pin_loads += (unsigned long long)nl;
        *st.hdr = h;
    }
}

hipError_t launch_tier_pin(const int32_t* experts, int32_t n, const TierState& st, int4* loads, int32_t* info,
                           hipStream_t s)
{
    hipLaunchKernelGGL(tier_pin_kernel, dim3(1), dim3(kPlanThreads), 0, s, experts, n, st, loads, info);
    return hipGetLastError();
}

/* Loads [(pass-1)*c, min(pass*c, n_load)) of the plan: each expert's six
 * regions, 16 bytes per thread and step.  Reads of pinned host memory cross
 * PCIe; a few hundred workgroups keep enough of them in flight. */
constexpr int kFetchThreads = 256;
constexpr int kFetchBlocks = 256;

__global__ __launch_bounds__(kFetchThreads) void tier_fetch_kernel(const int4* __restrict__ loads,
                                                                   const int32_t* __restrict__ info,
                                                                   int32_t pass, TierBanks b)
{
    const int32_t c = info[kInfoChunk], nl = info[kInfoLoad];
    const int32_t l0 = (pass - 1) * c, l1 = min(pass * c, nl);
    const int64_t gid = (int64_t)blockIdx.x * kFetchThreads + threadIdx.x;
    const int64_t gsz = (int64_t)gridDim.x * kFetchThreads;
    for (int32_t l = l0; l < l1; ++l) {
        const int4 L = loads[l];
        for (int r = 0; r < 6; ++r) {
            const int64_t len = b.len[r];
            const uint4* src = b.src[r] + (int64_t)L.x * len;
            uint4* dst = b.dst[r] + (int64_t)L.y * len;
            for (int64_t i = gid; i < len; i += gsz)
                dst[i] = src[i];
        }
    }
}

hipError_t launch_tier_fetch(const int4* loads, const int32_t* info, int32_t pass, const TierBanks& b,
                             hipStream_t s)
{
    hipLaunchKernelGGL(tier_fetch_kernel, dim3(kFetchBlocks), dim3(kFetchThreads), 0, s, loads, info, pass, b);
    return hipGetLastError();
}

/* Draft-union statistics of one layer of a verify step ("Show HN:
 * 如何在我的低配置电脑上运行 GLM-5.2", section 已实现的功能, the MTP item:
 * every verified draft may route to experts of its own, and the
 * batched-union item: each distinct expert of the batch is read once).  One
 * workgroup builds the bit set of the distinct experts among the P routed
 * ids, counts it and counts how many of them the previous step's set held;
 * the stored set then becomes this step's.  The counts are sums of
 * population counts of LDS words, independent of thread timing. */
constexpr int kUnionThreads = 256;

__global__ __launch_bounds__(kUnionThreads) void verify_union_kernel(const int32_t* __restrict__ ids, int32_t P,
                                                                     int32_t E, uint32_t* __restrict__ mask,
                                                                     int32_t* __restrict__ stats)
{
    __shared__ uint32_t cur[kTierMaxE / 32];
    __shared__ int32_t cnt[2];
    const int32_t nw = (E + 31) / 32;
    for (int32_t w = threadIdx.x; w < nw; w += kUnionThreads)
        cur[w] = 0;
    if (threadIdx.x < 2)
        cnt[threadIdx.x] = 0;
    __syncthreads();
    for (int32_t p = threadIdx.x; p < P; p += kUnionThreads) {
        const int32_t e = ids[p];
        if (e >= 0 && e < E)
            atomicOr(&cur[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
    int32_t u = 0, r = 0;
    for (int32_t w = threadIdx.x; w < nw; w += kUnionThreads) {
        const uint32_t c = cur[w];
        u += __popc(c);
        r += __popc(c & mask[w]);
        mask[w] = c;
    }
    if (u)
        atomicAdd(&cnt[0], u);
    if (r)
        atomicAdd(&cnt[1], r);
    __syncthreads();
    if (threadIdx.x == 0) {
        stats[0] = cnt[0];
        stats[1] = cnt[1];
    }
}

hipError_t launch_verify_union(const int32_t* ids, int32_t P, int32_t E, uint32_t* mask, int32_t* stats,
                               hipStream_t s)
{
    hipLaunchKernelGGL(verify_union_kernel, dim3(1), dim3(kUnionThreads), 0, s, ids, P, E, mask, stats);
    return hipGetLastError();
}

} // namespace coli
