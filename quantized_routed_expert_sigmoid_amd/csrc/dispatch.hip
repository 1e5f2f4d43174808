/*
 * dispatch.hip -- batched-union dispatch and the routing-weighted combine.
 *
 * Union dispatch ("Show HN: 如何在我的低配置电脑上运行 GLM-5.2", implemented
 * features, batched-union MoE item: every expert present in the batch is read
 * once and applied to all positions routed to it).  The (token, slot) pairs
 * p = t*k + j are grouped by expert with a histogram, an exclusive prefix sum
 * and a stable counting sort, all inside one 1024-thread workgroup, with no
 * atomics on positions: ranks come from wave ballots and per-wave counts, so
 * the result is the unique stable order.
 *
 * Combine ("colibrì 深度拆解", section 4.3: shared-expert output plus the
 * routing-weighted sum of the selected experts' outputs).
 */
#include "device_common.h"
#include "kernels.h"
#include "select.h"

namespace coli {

constexpr int kDispThreads = 1024;
constexpr int kDispWaves = kDispThreads / 64;
constexpr int kMaxE = 1024;

/* Workgroup exclusive scan of one value per thread (1024 threads).  Returns
 * the exclusive prefix; *total receives the sum.  `tmp` holds kDispWaves + 1
 * values. */
template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* tmp, T* total)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    T inc = v;
    for (int off = 1; off < 64; off <<= 1) {
        const T o = __shfl_up(inc, off, 64);
        if (lane >= off)
            inc += o;
    }
    if (lane == 63)
        tmp[wv] = inc;
    __syncthreads();
    if (wv == 0) {
        const T w = lane < kDispWaves ? tmp[lane] : T(0);
        T winc = w;
        for (int off = 1; off < kDispWaves; off <<= 1) {
            const T o = __shfl_up(winc, off, 64);
            if (lane >= off)
                winc += o;
        }
        if (lane < kDispWaves)
            tmp[lane] = winc - w; /* exclusive wave base */
        if (lane == kDispWaves - 1)
            tmp[kDispWaves] = winc;
    }
    __syncthreads();
    const T res = tmp[wv] + inc - v;
    *total = tmp[kDispWaves];
    __syncthreads();
    return res;
}

/* Writes the work units of expert e (count n, first sorted position off) in
 * chunks of `chunk` positions, never past max_units units in all. */
__device__ __forceinline__ void emit_units(Unit* units, int32_t ubase, int32_t e, int32_t off,
                                           int32_t n, int32_t chunk, int32_t max_units)
{
    for (int32_t u = 0; u * chunk < n && ubase + u < max_units; ++u) {
        Unit U;
        U.e = e;
        U.pos0 = off + u * chunk;
        U.ntok = (n - u * chunk) < chunk ? (n - u * chunk) : chunk;
        U.pad = 0;
        units[ubase + u] = U;
    }
}

/* Unit counts of an expert with c positions under matrix-core threshold
 * mmin: (GEMV units, MFMA units). */
__device__ __forceinline__ void unit_counts(int32_t c, int32_t mmin, int32_t& nu_g, int32_t& nu_m)
{
    const bool big = c >= mmin;
    nu_g = big ? 0 : (c + kUnitTokens - 1) / kUnitTokens;
    nu_m = big ? (c + kMfmaUnitTokens - 1) / kMfmaUnitTokens : 0;
}

/* Packed per-expert counts for one workgroup scan: positions (bits 0..20),
 * active flag (21..31), GEMV units (32..43), MFMA units (44..63).  With at
 * most 2^20 pairs and 1024 experts no field can carry into the next. */
__device__ __forceinline__ uint64_t pack_counts(int32_t c, int32_t nu_g, int32_t nu_m)
{
    return (uint64_t)c | ((uint64_t)(c > 0 ? 1 : 0) << 21) | ((uint64_t)nu_g << 32) |
           ((uint64_t)nu_m << 44);
}

struct DispatchShared {
    int32_t cnt[kMaxE];
    int32_t base[kMaxE];
    uint8_t wcnt[kDispWaves][kMaxE];
    uint64_t tmp[kDispWaves + 1];
};

/* Routed ids of the pairs, read from global memory or LDS. */
struct PlainIds {
    const int32_t* ids;
    __device__ __forceinline__ int32_t operator()(int32_t p) const { return ids[p]; }
};

/* The pairs of one pass of a tiered forward: codes hold pass << kPassSlotBits
 * | slot, or -1; pairs of other passes read as dropped. */
struct PassIds {
    const int32_t* codes;
    int32_t pass;
    __device__ __forceinline__ int32_t operator()(int32_t p) const
    {
        const int32_t v = codes[p];
        return (v >= 0 && (v >> kPassSlotBits) == pass) ? (v & ((1 << kPassSlotBits) - 1)) : -1;
    }
};

/* The dispatch, run by all 1024 threads of a workgroup.  Kept pairs get
 * inv = inv_base + sorted position; dropped pairs get inv = -1 when
 * mark_dropped is set and are left untouched otherwise. */
template <typename Ids>
__device__ __forceinline__ void dispatch_body(const Ids& ids, int32_t S, int32_t k, int32_t E,
                                              int32_t* offsets, int32_t* sorted, int32_t* inv,
                                              int32_t* active, int32_t* n_active, const UnitLists& ul,
                                              bool has_ul, DispatchShared& sh, int32_t inv_base = 0,
                                              bool mark_dropped = true)
{
    int32_t* cnt = sh.cnt;
    int32_t* base = sh.base;
    auto& wcnt = sh.wcnt;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int32_t P = S * k;

    for (int e = tid; e < kMaxE; e += kDispThreads) {
        cnt[e] = 0;
        for (int w = 0; w < kDispWaves; ++w)
            wcnt[w][e] = 0;
    }
    __syncthreads();
    /* a negative id is a dropped slot (no pair); ids past E - 1 violate the
     * documented precondition and are clamped so that no access leaves its
     * buffer */
    /* eight ids per thread in flight before their counts (clamped loads,
     * masked after), so the count pass costs one memory round trip per
     * 8 * kDispThreads pairs */
    for (int32_t p0 = 0; p0 < P; p0 += 8 * kDispThreads) {
        int32_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            v[q] = ids(min(p0 + q * kDispThreads + tid, P - 1));
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (p0 + q * kDispThreads + tid < P && v[q] >= 0)
                atomicAdd(&cnt[min(v[q], E - 1)], 1);
    }
    __syncthreads();

    /* offsets, active list and unit lists: one expert per thread, one scan of
     * the packed counts */
    const int32_t e = tid;
    const int32_t c = e < E ? cnt[e] : 0;
    int32_t nu_g, nu_m;
    unit_counts(c, has_ul ? ul.mfma_min : kMfmaMinTokens, nu_g, nu_m);
    uint64_t tot;
    const uint64_t pre = block_exclusive_scan<uint64_t>(pack_counts(c, nu_g, nu_m), sh.tmp, &tot);
    const int32_t off = (int32_t)(pre & 0x1FFFFF);
    const int32_t aidx = (int32_t)((pre >> 21) & 0x7FF);
    const int32_t gbase = (int32_t)((pre >> 32) & 0xFFF);
    const int32_t mbase = (int32_t)(pre >> 44);
    if (e < E) {
        base[e] = off;
        offsets[e] = off;
        if (c > 0)
            active[aidx] = e;
        if (has_ul) {
            emit_units(ul.units, gbase, e, off, nu_g ? c : 0, kUnitTokens, ul.max_units);
            emit_units(ul.munits, mbase, e, off, nu_m ? c : 0, kMfmaUnitTokens, ul.max_munits);
        }
    }
    if (tid == 0) {
        offsets[E] = (int32_t)(tot & 0x1FFFFF); /* pairs kept */
        *n_active = (int32_t)((tot >> 21) & 0x7FF);
        if (has_ul) {
            *ul.n_units = min((int32_t)((tot >> 32) & 0xFFF), ul.max_units);
            *ul.n_munits = min((int32_t)(tot >> 44), ul.max_munits);
        }
    }
    __syncthreads();

    /* stable placement, 1024 pairs per round */
    int nbits = 1;
    while ((1 << nbits) < E)
        ++nbits;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    /* each round's id is loaded during the previous round */
    int32_t id_next = P > 0 ? ids(min(tid, P - 1)) : -1;
    for (int32_t r0 = 0; r0 < P; r0 += kDispThreads) {
        const int32_t p = r0 + tid;
        const int32_t id = p < P ? id_next : -1;
        if (r0 + kDispThreads < P)
            id_next = ids(min(r0 + kDispThreads + tid, P - 1));
        const bool valid = id >= 0;
        const int32_t ex = valid ? min(id, E - 1) : 0;
        if (p < P && !valid && inv && mark_dropped)
            inv[p] = -1;
        uint64_t m = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            uint64_t bal = __ballot(valid && ((ex >> b) & 1));
            m &= ((ex >> b) & 1) ? bal : ~bal;
        }
        const int32_t rank = __popcll(m & lt_mask);
        if (valid && rank == 0)
            wcnt[wv][ex] = (uint8_t)__popcll(m);
        __syncthreads();
        if (valid) {
            int32_t pos = base[ex] + rank;
            for (int w = 0; w < wv; ++w)
                pos += wcnt[w][ex];
            sorted[pos] = p;
            if (inv)
                inv[p] = inv_base + pos;
        }
        __syncthreads();
        for (int ee = tid; ee < E; ee += kDispThreads) {
            int32_t add = 0;
            for (int w = 0; w < kDispWaves; ++w) {
                add += wcnt[w][ee];
                wcnt[w][ee] = 0;
            }
            base[ee] += add;
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kDispThreads) void dispatch_kernel(
    const int32_t* __restrict__ ids, int32_t S, int32_t k, int32_t E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted, int32_t* __restrict__ inv, int32_t* __restrict__ active,
    int32_t* __restrict__ n_active, UnitLists ul, int32_t has_units)
{
    __shared__ DispatchShared sh;
    dispatch_body(PlainIds{ids}, S, k, E, offsets, sorted, inv, active, n_active, ul, has_units != 0, sh);
}

hipError_t launch_dispatch(const int32_t* ids, int32_t S, int32_t k, int32_t E, int32_t* offsets,
                           int32_t* sorted, int32_t* inv, int32_t* active, int32_t* n_active,
                           const UnitLists* ul, hipStream_t st)
{
    UnitLists none = {};
    hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(kDispThreads), 0, st, ids, S, k, E, offsets,
                       sorted, inv, active, n_active, ul ? *ul : none, ul ? 1 : 0);
    return hipGetLastError();
}

__global__ __launch_bounds__(kDispThreads) void dispatch_pass_kernel(
    const int32_t* __restrict__ codes, int32_t pass, int32_t inv_base, int32_t S, int32_t k,
    int32_t n_slots, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted,
    int32_t* __restrict__ inv, int32_t* __restrict__ active, int32_t* __restrict__ n_active,
    UnitLists ul)
{
    __shared__ DispatchShared sh;
    dispatch_body(PassIds{codes, pass}, S, k, n_slots, offsets, sorted, inv, active, n_active, ul, true, sh,
                  inv_base, pass == 0);
}

hipError_t launch_dispatch_pass(const int32_t* codes, int32_t pass, int32_t inv_base, int32_t S,
                                int32_t k, int32_t n_slots, int32_t* offsets, int32_t* sorted,
                                int32_t* inv, int32_t* active, int32_t* n_active, const UnitLists& ul,
                                hipStream_t st)
{
    hipLaunchKernelGGL(dispatch_pass_kernel, dim3(1), dim3(kDispThreads), 0, st, codes, pass, inv_base,
                       S, k, n_slots, offsets, sorted, inv, active, n_active, ul);
    return hipGetLastError();
}

/* The dispatch of at most 64 pairs (ids in LDS, 16-byte aligned), with the
 * result of dispatch_body written out directly: a pair's sorted position is
 * the number of kept pairs of lower experts plus those of its own expert
 * before it.  Every thread e <= E writes offsets[e] from the ids read as
 * 16-byte vectors; wave 0 holds pair p in lane p and finds, with one ballot
 * per bit of the expert id, the pairs of its expert and those of lower
 * experts, then writes the positions, the active list and the unit lists
 * (in expert order, as the scan of dispatch_body places them).  No
 * histogram, scan or placement rounds, and no barrier. */
__device__ __forceinline__ void dispatch_few(const int32_t* sel_ids, int32_t P, int32_t E, int32_t* offsets,
                                             int32_t* sorted, int32_t* inv, int32_t* active, int32_t* n_active,
                                             const UnitLists& ul)
{
    const int tid = threadIdx.x, lane = tid & 63;
    int32_t key[64];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int4 v = reinterpret_cast<const int4*>(sel_ids)[i];
        key[4 * i] = v.x;
        key[4 * i + 1] = v.y;
        key[4 * i + 2] = v.z;
        key[4 * i + 3] = v.w;
    }
    /* a kept pair's key is its clamped expert id; past P and dropped: E */
#pragma unroll
    for (int q = 0; q < 64; ++q)
        key[q] = (q < P && key[q] >= 0) ? min(key[q], E - 1) : E;
    for (int32_t e = tid; e <= E; e += (int32_t)blockDim.x) {
        int32_t below = 0;
#pragma unroll
        for (int q = 0; q < 64; ++q)
            below += key[q] < e ? 1 : 0;
        offsets[e] = below;
    }
    if (tid >= 64)
        return;
    const int32_t raw = lane < P ? sel_ids[lane] : -1;
    const bool valid = raw >= 0;
    const int32_t ex = valid ? min(raw, E - 1) : 0;
    /* bit-sliced compare against every lane, most significant bit first */
    int nbits = 1;
    while ((1 << nbits) < E)
        ++nbits;
    uint64_t eqm = __ballot(valid), ltm = 0;
    for (int b = nbits - 1; b >= 0; --b) {
        const bool bit = (ex >> b) & 1;
        const uint64_t ones = __ballot(valid && bit);
        if (bit) {
            ltm |= eqm & ~ones;
            eqm &= ones;
        } else {
            eqm &= ~ones;
        }
    }
    const uint64_t lt_lane = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int32_t below = __popcll(ltm), cnt = __popcll(eqm), before = __popcll(eqm & lt_lane);
    const int32_t pos = below + before;
    if (valid) {
        sorted[pos] = lane;
        if (inv)
            inv[lane] = pos;
    } else if (lane < P && inv) {
        inv[lane] = -1;
    }
    /* the first pair of each expert speaks for it */
    const bool first = valid && before == 0;
    const uint64_t fm = __ballot(first);
    int32_t gq, mq;
    unit_counts(cnt, ul.mfma_min, gq, mq);
    /* sums over the first pairs (of lower experts), one ballot per bit of
     * the unit counts (at most 64 units per expert here) */
    const uint64_t lower = fm & ltm;
    const int32_t aidx = __popcll(lower);
    int32_t gbase = 0, mbase = 0, tot_g = 0, tot_m = 0;
#pragma unroll
    for (int b = 0; b < 7; ++b) {
        const uint64_t gb = fm & __ballot((gq >> b) & 1), mb = fm & __ballot((mq >> b) & 1);
        gbase += __popcll(gb & lower) << b;
        mbase += __popcll(mb & lower) << b;
        tot_g += __popcll(gb) << b;
        tot_m += __popcll(mb) << b;
    }
    if (first) {
        active[aidx] = ex;
        emit_units(ul.units, gbase, ex, below, gq ? cnt : 0, kUnitTokens, ul.max_units);
        emit_units(ul.munits, mbase, ex, below, mq ? cnt : 0, kMfmaUnitTokens, ul.max_munits);
    }
    if (lane == 0) {
        *n_active = __popcll(fm);
        *ul.n_units = min(tot_g, ul.max_units);
        *ul.n_munits = min(tot_m, ul.max_munits);
    }
}

/* Small batches (S <= kSmallS): wave t selects token t's experts (select.h),
 * then the whole workgroup dispatches the S*k pairs from LDS. */
__global__ __launch_bounds__(kDispThreads) void select_dispatch_small(
    const float* __restrict__ logits, const float* __restrict__ bias, int32_t S, int32_t E, int32_t k,
    float rsf, RouteOpts opt, int32_t* __restrict__ ids, float* __restrict__ weights,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted, int32_t* __restrict__ inv,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active, UnitLists ul)
{
    __shared__ DispatchShared sh;
    __shared__ __attribute__((aligned(16))) float sel_s[kSmallS][kSelScratch];
    __shared__ int32_t sel_ids[kSmallS * 64];
    const int wv = threadIdx.x >> 6;
    if (wv < S)
        select_token(logits + (int64_t)wv * E, bias, E, k, rsf, ids + (int64_t)wv * k,
                     weights + (int64_t)wv * k, sel_s[wv], sel_ids + wv * k, 1, 0, opt);
    __syncthreads();
    dispatch_body(PlainIds{sel_ids}, S, k, E, offsets, sorted, inv, active, n_active, ul, true, sh);
}

/* Small batches of at most 64 pairs: one wave per token (S waves), selection
 * as above, then dispatch_few. */
__global__ __launch_bounds__(kSmallS * 64) void select_dispatch_few(
    const float* __restrict__ logits, const float* __restrict__ bias, int32_t S, int32_t E, int32_t k,
    float rsf, RouteOpts opt, int32_t* __restrict__ ids, float* __restrict__ weights,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted, int32_t* __restrict__ inv,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active, UnitLists ul)
{
    __shared__ __attribute__((aligned(16))) float sel_s[kSmallS][kSelScratch];
    __shared__ __attribute__((aligned(16))) int32_t sel_ids[64];
    const int wv = threadIdx.x >> 6;
    select_token(logits + (int64_t)wv * E, bias, E, k, rsf, ids + (int64_t)wv * k, weights + (int64_t)wv * k,
                 sel_s[wv], sel_ids + wv * k, 1, 0, opt);
    __syncthreads();
    dispatch_few(sel_ids, S * k, E, offsets, sorted, inv, active, n_active, ul);
}

hipError_t launch_select_dispatch_small(const float* logits, const float* bias, int32_t S, int32_t E,
                                        int32_t k, float rsf, const RouteOpts& opt, int32_t* ids,
                                        float* weights, int32_t* offsets, int32_t* sorted, int32_t* inv,
                                        int32_t* active, int32_t* n_active, const UnitLists& ul,
                                        hipStream_t st)
{
    if (S > 0 && S * k <= 64)
        hipLaunchKernelGGL(select_dispatch_few, dim3(1), dim3(64 * S), 0, st, logits, bias, S, E, k, rsf, opt, ids,
                           weights, offsets, sorted, inv, active, n_active, ul);
    else
        hipLaunchKernelGGL(select_dispatch_small, dim3(1), dim3(kDispThreads), 0, st, logits, bias, S, E, k,
                           rsf, opt, ids, weights, offsets, sorted, inv, active, n_active, ul);
    return hipGetLastError();
}

/* Unit lists from offsets produced elsewhere.  Offsets that break the
 * documented contract (non-decreasing, last == S*k) cannot make it write past
 * the lists' bounds; the FFN kernels bound positions separately. */
__global__ __launch_bounds__(kDispThreads) void schedule_kernel(const int32_t* __restrict__ offsets,
                                                                int32_t n_mat, UnitLists ul)
{
    __shared__ uint64_t tmp[kDispWaves + 1];
    const int e = threadIdx.x;
    const int32_t off = e < n_mat ? offsets[e] : 0;
    const int32_t c = e < n_mat ? min(max(0, offsets[e + 1] - off), kPairLimit) : 0;
    int32_t nu_g, nu_m;
    unit_counts(c, ul.mfma_min, nu_g, nu_m);
    uint64_t tot;
    const uint64_t pre = block_exclusive_scan<uint64_t>(pack_counts(c, nu_g, nu_m), tmp, &tot);
    if (e < n_mat) {
        emit_units(ul.units, (int32_t)((pre >> 32) & 0xFFF), e, off, nu_g ? c : 0, kUnitTokens,
                   ul.max_units);
        emit_units(ul.munits, (int32_t)(pre >> 44), e, off, nu_m ? c : 0, kMfmaUnitTokens, ul.max_munits);
    }
    if (e == 0) {
        *ul.n_units = min((int32_t)((tot >> 32) & 0xFFF), ul.max_units);
        *ul.n_munits = min((int32_t)(tot >> 44), ul.max_munits);
    }
}

hipError_t launch_schedule(const int32_t* offsets, int32_t n_mat, const UnitLists& ul, hipStream_t st)
{
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kDispThreads), 0, st, offsets, n_mat, ul);
    return hipGetLastError();
}

/* ---- combine: out[t] = y_shared[t] + sum_j w[t][j] * y[inv[t*k+j]] --------
 * (dropped slots, inv < 0 or with inv null ids < 0, are skipped).  Slots go
 * in rounds of 8: the round's rows and weights, then its row loads, are all
 * issued before the first fma (a dropped or missing slot loads row 0 and
 * adds nothing), so a token costs one round trip per 8 slots; the fmas stay
 * in slot order. */

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ inv,
                                                      const int32_t* __restrict__ ids,
                                                      const float* __restrict__ w, int32_t S,
                                                      int32_t k, int32_t H, int32_t shared_row0,
                                                      float* __restrict__ out)
{
    constexpr int R = 8;
    const int64_t n4 = H / 4;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)S * n4)
        return;
    const int32_t t = (int32_t)(gid / n4);
    const int64_t c = gid - (int64_t)t * n4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (shared_row0 >= 0)
        acc = reinterpret_cast<const float4*>(y + (int64_t)(shared_row0 + t) * H)[c];
    for (int j0 = 0; j0 < k; j0 += R) {
        int32_t row[R];
        float wj[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int32_t p = t * k + min(j0 + i, k - 1);
            row[i] = inv ? inv[p] : (ids[p] >= 0 ? p : -1);
            wj[i] = w[p];
        }
        float4 v[R];
#pragma unroll
        for (int i = 0; i < R; ++i)
            v[i] = reinterpret_cast<const float4*>(y + (int64_t)max(row[i], 0) * H)[c];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            if (j0 + i < k && row[i] >= 0) {
                acc.x = __builtin_fmaf(wj[i], v[i].x, acc.x);
                acc.y = __builtin_fmaf(wj[i], v[i].y, acc.y);
                acc.z = __builtin_fmaf(wj[i], v[i].z, acc.z);
                acc.w = __builtin_fmaf(wj[i], v[i].w, acc.w);
            }
        }
    }
    reinterpret_cast<float4*>(out + (int64_t)t * H)[c] = acc;
}

hipError_t launch_combine(const float* y, const int32_t* inv, const int32_t* ids, const float* w,
                          int32_t S, int32_t k, int32_t H, int32_t shared_row0, float* out, hipStream_t st)
{
    if (S == 0)
        return hipSuccess;
    int64_t threads = (int64_t)S * (H / 4);
    hipLaunchKernelGGL(combine_kernel, dim3((uint32_t)((threads + 255) / 256)), dim3(256), 0, st, y,
                       inv, ids, w, S, k, H, shared_row0, out);
    return hipGetLastError();
}

} // namespace coli
