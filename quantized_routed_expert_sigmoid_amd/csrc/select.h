/*
 * select.h -- top-k selection of the sigmoid router for one token, run by
 * one wavefront ("Show HN: 如何在我的低配置电脑上运行 GLM-5.2", implemented-
 * features section, sigmoid-router item: DeepSeek-V3 style sigmoid scores,
 * noaux_tc selection bias, routed_scaling_factor).
 *
 * Each lane holds the scores of experts lane, lane+64, ...; the top-k is k
 * rounds of a wave-wide maximum of the order-preserving bits of the biased
 * score followed by a wave-wide minimum of the expert ids holding it (equal
 * scores resolve to the lower id).
 * Weights: rsf * s_j / sum of the selected unbiased scores (slot order).
 */
#ifndef COLI_SELECT_H
#define COLI_SELECT_H

#include "device_common.h"

namespace coli {

constexpr int kMaxPerLane = 16; /* E <= 1024 */

__device__ __forceinline__ uint32_t order_bits(float c)
{
    uint32_t u = __float_as_uint(c);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

/* lt: the token's E logits, or with n_parts > 1 the first of n_parts partial
 * sums part_stride floats apart (added in slice order); writes ids_out[0..k), w_out[0..k) and, when
 * ids_lds is not null, ids_lds[0..k).  sel_s: 64 floats of LDS owned by the
 * calling wave. */
__device__ __forceinline__ void select_token(const float* lt, const float* bias, int32_t E, int32_t k,
                                             float rsf, int32_t* ids_out, float* w_out, float* sel_s,
                                             int32_t* ids_lds, int32_t n_parts = 1,
                                             int64_t part_stride = 0)
{
    const int lane = threadIdx.x & 63;
    const int per_lane = (E + 63) / 64; /* uniform */
    float s[kMaxPerLane];
    uint32_t key[kMaxPerLane]; /* order-preserving bits of the biased score; 0 = unavailable */
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        if (i < per_lane && e < E) {
            float l = lt[e];
            for (int p = 1; p < n_parts; ++p) /* K slices, added in order */
                l = l + lt[p * part_stride + e];
            const float sg = 1.0f / (1.0f + expf(-l));
            s[i] = sg;
            key[i] = order_bits(sg + bias[e]);
        } else {
            s[i] = 0.0f;
            key[i] = 0;
        }
    }
    for (int j = 0; j < k; ++j) {
        /* best score, then the lowest expert id holding it */
        uint32_t best = 0;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i)
            if (i < per_lane)
                best = key[i] > best ? key[i] : best;
        best = wave_reduce_u32<true>(best);
        uint32_t mine = 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i)
            if (i < per_lane && key[i] == best && mine == 0xFFFFFFFFu)
                mine = (uint32_t)(lane + 64 * i);
        const int e = (int)wave_reduce_u32<false>(mine);
        const int ie = e >> 6; /* uniform */
        float cand = 0.0f;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) {
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
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    float denom = 0.0f;
    for (int j = 0; j < k; ++j)
        denom += sel_s[j];
    if (lane < k)
        w_out[lane] = rsf * (sel_s[lane] / denom);
}

} // namespace coli

#endif
