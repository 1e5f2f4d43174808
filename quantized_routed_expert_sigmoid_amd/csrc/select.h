/*
 * select.h -- top-k selection of the sigmoid router for one token, run by
 * one wavefront ("Show HN: 如何在我的低配置电脑上运行 GLM-5.2", implemented-
 * features section, sigmoid-router item: DeepSeek-V3 style sigmoid scores,
 * noaux_tc selection bias, routed_scaling_factor).
 *
 * Each lane holds the scores of experts lane, lane+64, ...; the top-k is taken
 * on the order-preserving bits of the biased score, equal scores resolving to
 * the lower id, in slots of descending score.  For k <= 8 the few candidates
 * above a lower bound of the k-th key are ranked in parallel; otherwise (or
 * with more than 64 candidates) k rounds of a wave-wide maximum pick them.
 * Weights: rsf * s_j / sum of the selected unbiased scores (slot order).
 */
#ifndef COLI_SELECT_H
#define COLI_SELECT_H

#include "device_common.h"
#include "kernels.h"

namespace coli {

constexpr int kMaxPerLane = 16; /* E <= 1024 */
constexpr int kSelScratch = 256; /* floats of LDS scratch per selecting wave, 16-byte aligned */

__device__ __forceinline__ uint32_t order_bits(float c)
{
    uint32_t u = __float_as_uint(c);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

/* The float an order_bits key came from. */
__device__ __forceinline__ float key_value(uint32_t key)
{
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

/* Wave maximum of key over the lane's PL experts e with group(e) == g (all
 * experts when g < 0), then the lowest such expert holding it; returns the
 * key and writes the expert to *e_out (-1 when the set is empty). */
template <int PL>
__device__ __forceinline__ uint32_t argmax_key(const uint32_t (&key)[PL], int E, int gsz, int g, int skip_e,
                                               int* e_out)
{
    const int lane = threadIdx.x & 63;
    uint32_t best = 0;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int e = lane + 64 * i;
        if (e < E && (g < 0 || e / gsz == g) && e != skip_e)
            best = key[i] > best ? key[i] : best;
    }
    best = wave_reduce_u32<true>(best);
    uint32_t mine = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int e = lane + 64 * i;
        if (e < E && (g < 0 || e / gsz == g) && e != skip_e && key[i] == best && mine == 0xFFFFFFFFu)
            mine = (uint32_t)e;
    }
    const uint32_t e = wave_reduce_u32<false>(mine);
    *e_out = best == 0 ? -1 : (int)e;
    return best;
}

/* lt: the token's E logits, or with n_parts > 1 the first of n_parts partial
 * sums part_stride floats apart (added in slice order).  Writes ids_out[0..k),
 * w_out[0..k) (skipped when w_out is null and top-p is off) and, when ids_lds
 * is not null, ids_lds[0..k).  sel_s: kSelScratch floats
 * of LDS owned by the calling wave.  Called by a whole wave.
 *
 * Group stage (opt.n_group > 1): per group the largest biased score, the
 * lowest expert holding it, then the largest score among the group's other
 * experts; their fp32 sum is the group score.  topk_group rounds of a wave
 * maximum pick the groups (ties to the lower group); experts of the other
 * groups become unavailable.
 *
 * Top-p (0 < opt.top_p < 1): each slot's rank by unbiased score (descending,
 * ties in slot order) is computed in parallel; lane 0 then accumulates the
 * fp32 shares s / sum s in rank order, in the order and precision of the
 * oracle, up to the first cumulative share >= top_p.  Slots past the cut get
 * id -1 and weight 0; the kept weights are renormalised over the kept slots
 * (denominator in slot order). */
template <int PL, bool SLICED>
__device__ __forceinline__ void select_token_pl(const float* lt, const float* bias, int32_t E, int32_t k,
                                                float rsf, int32_t* ids_out, float* w_out, float* sel_s,
                                                int32_t* ids_lds, int32_t n_parts, int64_t part_stride,
                                                RouteOpts opt)
{
    const int lane = threadIdx.x & 63;
    float s[PL];
    uint32_t key[PL]; /* order-preserving bits of the biased score; 0 = unavailable */
    /* K slices of the logits, added in slice order.  Each round issues the
     * loads of Q slices for all of the lane's experts before any add
     * (clamped to the last slice and expert, so every load is in bounds): the
     * slices cost one memory round trip per Q rather than one each. */
    float lg[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i)
        lg[i] = lt[min(lane + 64 * i, E - 1)];
    if constexpr (SLICED) {
        constexpr int Q = PL <= 2 ? 16 : 32 / PL;
        for (int p0 = 1; p0 < n_parts; p0 += Q) {
            float v[PL][Q];
#pragma unroll
            for (int q = 0; q < Q; ++q)
#pragma unroll
                for (int i = 0; i < PL; ++i)
                    v[i][q] = lt[(int64_t)min(p0 + q, n_parts - 1) * part_stride + min(lane + 64 * i, E - 1)];
#pragma unroll
            for (int q = 0; q < Q; ++q)
#pragma unroll
                for (int i = 0; i < PL; ++i)
                    if (p0 + q < n_parts)
                        lg[i] = lg[i] + v[i][q];
        }
    }
#pragma unroll
    for (int i = 0; i < PL; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
            const float l = lg[i];
            const float sg = 1.0f / (1.0f + expf(-l));
            s[i] = sg;
            key[i] = order_bits(sg + bias[e]);
        } else {
            s[i] = 0.0f;
            key[i] = 0;
        }
    }
    if (opt.n_group > 1) {
        const int G = min(opt.n_group, kMaxGroups), gsz = E / G;
        float gscore = 0.0f;
        for (int g = 0; g < G; ++g) {
            int e1, e2;
            const uint32_t k1 = argmax_key<PL>(key, E, gsz, g, -1, &e1);
            const uint32_t k2 = argmax_key<PL>(key, E, gsz, g, e1, &e2);
            if (lane == g)
                gscore = key_value(k1) + key_value(k2);
        }
        uint32_t gkey = lane < G ? order_bits(gscore) : 0;
        uint64_t kept = 0;
        for (int r = 0; r < opt.topk_group; ++r) {
            const uint32_t best = wave_reduce_u32<true>(gkey);
            const uint32_t gsel = wave_reduce_u32<false>(gkey == best && lane < G ? (uint32_t)lane : 0xFFFFFFFFu);
            kept |= 1ull << gsel;
            if (lane == (int)gsel)
                gkey = 0;
        }
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            const int e = lane + 64 * i;
            if (e < E && !((kept >> (e / gsz)) & 1))
                key[i] = 0;
        }
    }
    /* Candidates (k <= 8): the maxima of the eight 8-lane groups are eight
     * distinct keys, so their minimum L is at most the k-th largest key and
     * every expert of the top-k has a key >= L.  The candidates (few for
     * scores that are not massively tied) are packed into LDS in ascending id
     * order and each finds its slot as its rank by (key descending, id
     * ascending) among them -- no chain of wave-wide steps.  More than 64
     * candidates: k rounds of a wave-wide maximum instead. */
    bool done = false;
    if (k <= 8) {
        uint32_t g = key[0];
#pragma unroll
        for (int i = 1; i < PL; ++i)
            g = key[i] > g ? key[i] : g;
        /* row_shr 1, 2, 4: lane 8q + 7 ends with the maximum of lanes 8q .. 8q+7 */
        uint32_t t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)g, 0x111, 0xF, 0xF, false);
        g = t > g ? t : g;
        t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)g, 0x112, 0xF, 0xF, false);
        g = t > g ? t : g;
        t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)g, 0x114, 0xF, 0xF, false);
        g = t > g ? t : g;
        uint32_t L = 0xFFFFFFFFu;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)g, 8 * q + 7);
            L = m < L ? m : L;
        }
        uint64_t cm[PL];
        int n_c = 0;
#pragma unroll
        for (int i = 0; i < PL; ++i) {
            cm[i] = __ballot(key[i] >= L);
            n_c += __popcll(cm[i]);
        }
        if (n_c <= 64) {
            uint32_t* ck = reinterpret_cast<uint32_t*>(sel_s + 64);
            int32_t* ci = reinterpret_cast<int32_t*>(sel_s + 128);
            float* cs = sel_s + 192;
            int base = 0;
#pragma unroll
            for (int i = 0; i < PL; ++i) {
                if ((cm[i] >> lane) & 1) {
                    const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(cm[i] >> 32),
                                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)cm[i], 0u));
                    ck[pos] = key[i];
                    ci[pos] = lane + 64 * i;
                    cs[pos] = s[i];
                }
                base += __popcll(cm[i]);
            }
            /* padding to a multiple of 8 never outranks a candidate */
            const int n_c8 = (n_c + 7) & ~7;
            if (lane >= n_c && lane < n_c8) {
                ck[lane] = 0;
                ci[lane] = 0x7FFFFFFF;
            }
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            if (lane < n_c) {
                const uint32_t mk = ck[lane];
                const int mi = ci[lane];
                int rank = 0;
                for (int j = 0; j < n_c8; j += 8) {
                    /* eight candidates per round of (broadcast) reads */
                    const uint4 k0 = *reinterpret_cast<const uint4*>(ck + j);
                    const uint4 k1 = *reinterpret_cast<const uint4*>(ck + j + 4);
                    const int4 i0 = *reinterpret_cast<const int4*>(ci + j);
                    const int4 i1 = *reinterpret_cast<const int4*>(ci + j + 4);
                    const uint32_t kk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
                    const int ii[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        rank += (kk[q] > mk || (kk[q] == mk && ii[q] < mi)) ? 1 : 0;
                }
                if (rank < k) {
                    sel_s[rank] = cs[lane];
                    ids_out[rank] = mi;
                    if (ids_lds)
                        ids_lds[rank] = mi;
                }
            }
            done = true;
        }
    }
    if (!done) {
        for (int j = 0; j < k; ++j) {
            /* the lane's best key and the lowest of its indices holding it */
            uint32_t lbest = key[0];
            int li = 0;
#pragma unroll
            for (int i = 1; i < PL; ++i) {
                if (key[i] > lbest) {
                    lbest = key[i];
                    li = i;
                }
            }
            const uint32_t best = wave_reduce_u32<true>(lbest);
            const uint64_t holders = __ballot(lbest == best);
            int e;
            if (__popcll(holders) == 1) {
                /* one lane holds it: its lowest index is the lowest expert id */
                const int wl = __builtin_ctzll(holders);
                e = wl + 64 * __builtin_amdgcn_readlane(li, wl);
            } else {
                /* several lanes: the lowest expert id holding the best key */
                uint32_t mine = 0xFFFFFFFFu;
#pragma unroll
                for (int i = 0; i < PL; ++i)
                    if (key[i] == best && mine == 0xFFFFFFFFu)
                        mine = (uint32_t)(lane + 64 * i);
                e = (int)wave_reduce_u32<false>(mine);
            }
            const int ie = e >> 6; /* uniform */
            float cand = 0.0f;
#pragma unroll
            for (int i = 0; i < PL; ++i) {
                if (i == ie) {
                    cand = s[i];
                    if (lane == (e & 63))
                        key[i] = 0; /* taken */
                }
            }
            const float sj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cand), e & 63));
            if (lane == 0) {
                sel_s[j] = sj;
                ids_out[j] = e;
                if (ids_lds)
                    ids_lds[j] = e;
            }
        }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    if (opt.top_p > 0.0f && opt.top_p < 1.0f) {
        int32_t* slot_of_rank = reinterpret_cast<int32_t*>(sel_s + 64);
        if (lane < k) {
            const float mine = sel_s[lane];
            int rank = 0;
            for (int i = 0; i < k; ++i)
                rank += (sel_s[i] > mine || (sel_s[i] == mine && i < lane)) ? 1 : 0;
            slot_of_rank[rank] = lane;
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        int m = k;
        if (lane == 0) {
            float den = 0.0f;
            for (int j = 0; j < k; ++j)
                den = den + sel_s[j];
            float cum = 0.0f;
            for (int r = 0; r < k; ++r) {
                cum = cum + sel_s[slot_of_rank[r]] / den;
                if (cum >= opt.top_p) {
                    m = r + 1;
                    break;
                }
            }
        }
        m = __builtin_amdgcn_readfirstlane(m);
        /* slot j is kept iff its rank is below m */
        bool keep = false;
        if (lane < k) {
            const float mine = sel_s[lane];
            int rank = 0;
            for (int i = 0; i < k; ++i)
                rank += (sel_s[i] > mine || (sel_s[i] == mine && i < lane)) ? 1 : 0;
            keep = rank < m;
        }
        const uint64_t kept_slots = __ballot(keep);
        float denom = 0.0f;
        for (int j = 0; j < k; ++j)
            if ((kept_slots >> j) & 1)
                denom += sel_s[j];
        if (lane < k)
            w_out[lane] = keep ? rsf * (sel_s[lane] / denom) : 0.0f;
        if (lane == 0) /* the lane that stored the ids rewrites them, in order */
            for (int j = 0; j < k; ++j)
                if (!((kept_slots >> j) & 1)) {
                    ids_out[j] = -1;
                    if (ids_lds)
                        ids_lds[j] = -1;
                }
        return;
    }
    if (w_out == nullptr) /* ids only */
        return;
    float denom = 0.0f;
    for (int j = 0; j < k; ++j)
        denom += sel_s[j];
    if (lane < k)
        w_out[lane] = rsf * (sel_s[lane] / denom);
}

/* Dispatches on the experts per lane (a multiple of 64 up to E), so that the
 * per-lane loops run exactly as many times as there are experts.  SLICED:
 * the logits are n_parts K slices part_stride apart, added in slice order
 * (the many-token router); otherwise one slice (n_parts is 1). */
template <bool SLICED = false>
__device__ __forceinline__ void select_token(const float* lt, const float* bias, int32_t E, int32_t k,
                                             float rsf, int32_t* ids_out, float* w_out, float* sel_s,
                                             int32_t* ids_lds, int32_t n_parts = 1,
                                             int64_t part_stride = 0, RouteOpts opt = RouteOpts{1, 1, 1.0f})
{
    const int per_lane = (E + 63) / 64; /* uniform */
    if (per_lane <= 1)
        select_token_pl<1, SLICED>(lt, bias, E, k, rsf, ids_out, w_out, sel_s, ids_lds, n_parts, part_stride, opt);
    else if (per_lane <= 2)
        select_token_pl<2, SLICED>(lt, bias, E, k, rsf, ids_out, w_out, sel_s, ids_lds, n_parts, part_stride, opt);
    else if (per_lane <= 4)
        select_token_pl<4, SLICED>(lt, bias, E, k, rsf, ids_out, w_out, sel_s, ids_lds, n_parts, part_stride, opt);
    else if (per_lane <= 8)
        select_token_pl<8, SLICED>(lt, bias, E, k, rsf, ids_out, w_out, sel_s, ids_lds, n_parts, part_stride, opt);
    else
        select_token_pl<kMaxPerLane, SLICED>(lt, bias, E, k, rsf, ids_out, w_out, sel_s, ids_lds, n_parts,
                                             part_stride, opt);
}

} // namespace coli

#endif
