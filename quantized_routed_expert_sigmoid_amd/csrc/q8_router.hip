/*
 * q8_router.hip -- Q8_0-style activation quantisation and the sigmoid router.
 *
 * Q8_0 ("Show HN: 如何在我的低配置电脑上运行 GLM-5.2", implemented-features
 * section, integer dot-product item): per 32-element block one fp32 scale
 * d = amax / 127 and int8 codes round-half-away(v / d) in [-127, 127].
 *
 * Router (same section, sigmoid-router item: DeepSeek-V3 style, noaux_tc,
 * routed_scaling_factor): sigmoid scores, a selection bias, top-k with ties
 * to the lower expert id, weights renormalised over the unbiased scores of
 * the selected experts and multiplied by routed_scaling_factor.
 */
#include "device_common.h"
#include "kernels.h"

namespace coli {

/* ---- Q8_0: 8 lanes per block, 4 consecutive values per lane ------------- */

__global__ __launch_bounds__(256) void quantize_q8_0_kernel(const float* __restrict__ x,
                                                            int64_t n_blocks,
                                                            int8_t* __restrict__ q,
                                                            float* __restrict__ d)
{
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t blk = gid >> 3;
    bool live = blk < n_blocks;
    float4 v = live ? reinterpret_cast<const float4*>(x)[gid] : make_float4(0.f, 0.f, 0.f, 0.f);
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = fmaxf(a, shfl_xor(a, 1));
    a = fmaxf(a, shfl_xor(a, 2));
    a = fmaxf(a, shfl_xor(a, 4));
    if (!live)
        return;
    float scale = a / 127.0f;
    float inv = (a == 0.0f) ? 0.0f : 1.0f / scale;
    uint32_t packed = (uint32_t)(q8_code(v.x, inv) & 0xFF) | ((uint32_t)(q8_code(v.y, inv) & 0xFF) << 8) |
                      ((uint32_t)(q8_code(v.z, inv) & 0xFF) << 16) |
                      ((uint32_t)(q8_code(v.w, inv) & 0xFF) << 24);
    reinterpret_cast<uint32_t*>(q)[gid] = packed;
    if ((gid & 7) == 0)
        d[blk] = scale;
}

hipError_t launch_quantize_q8_0(const float* x, int64_t n_blocks, int8_t* q, float* d,
                                hipStream_t st)
{
    if (n_blocks == 0)
        return hipSuccess;
    int64_t threads = n_blocks * 8;
    int64_t grid = (threads + 255) / 256;
    hipLaunchKernelGGL(quantize_q8_0_kernel, dim3((uint32_t)grid), dim3(256), 0, st, x, n_blocks, q, d);
    return hipGetLastError();
}

/* ---- router logits --------------------------------------------------------
 * Few tokens: one wave per expert streams its router row once (float4,
 * coalesced) and keeps one partial sum per token; wave reduction at the end.
 * Many tokens: 32 x 32 output tiles through LDS. Both sum in fp32. */

constexpr int kSmallS = 8;

__global__ __launch_bounds__(256) void router_logits_small(const float* __restrict__ x, int32_t S,
                                                           int32_t H, int32_t E,
                                                           const float* __restrict__ w,
                                                           float* __restrict__ logits)
{
    int lane = threadIdx.x & 63;
    int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E)
        return;
    const float4* wr = reinterpret_cast<const float4*>(w + (int64_t)e * H);
    float acc[kSmallS];
#pragma unroll
    for (int t = 0; t < kSmallS; ++t)
        acc[t] = 0.0f;
    int n4 = H / 4;
    for (int i = lane; i < n4; i += 64) {
        float4 wv = wr[i];
#pragma unroll
        for (int t = 0; t < kSmallS; ++t) {
            if (t < S) {
                float4 xv = reinterpret_cast<const float4*>(x + (int64_t)t * H)[i];
                acc[t] = __builtin_fmaf(wv.x, xv.x, acc[t]);
                acc[t] = __builtin_fmaf(wv.y, xv.y, acc[t]);
                acc[t] = __builtin_fmaf(wv.z, xv.z, acc[t]);
                acc[t] = __builtin_fmaf(wv.w, xv.w, acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kSmallS; ++t) {
        if (t < S) {
            float s = wave_sum(acc[t]);
            if (lane == 0)
                logits[(int64_t)t * E + e] = s;
        }
    }
}

constexpr int kTile = 32;
constexpr int kTileK = 32;

__global__ __launch_bounds__(256) void router_logits_tiled(const float* __restrict__ x, int32_t S,
                                                           int32_t H, int32_t E,
                                                           const float* __restrict__ w,
                                                           float* __restrict__ logits)
{
    __shared__ float xs[kTileK][kTile + 1];
    __shared__ float ws[kTileK][kTile + 1];
    int t0 = blockIdx.x * kTile, e0 = blockIdx.y * kTile;
    int tid = threadIdx.x;
    int tr = (tid / 16) * 2, tc = (tid % 16) * 2; /* 2 x 2 outputs per thread */
    float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
    int lr = tid / 8, lk = (tid % 8) * 4; /* loader: row lr, 4 consecutive k */
    for (int k0 = 0; k0 < H; k0 += kTileK) {
        {
            int t = t0 + lr;
            float4 v = (t < S) ? *reinterpret_cast<const float4*>(x + (int64_t)t * H + k0 + lk)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
            xs[lk + 0][lr] = v.x;
            xs[lk + 1][lr] = v.y;
            xs[lk + 2][lr] = v.z;
            xs[lk + 3][lr] = v.w;
            int e = e0 + lr;
            float4 u = (e < E) ? *reinterpret_cast<const float4*>(w + (int64_t)e * H + k0 + lk)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
            ws[lk + 0][lr] = u.x;
            ws[lk + 1][lr] = u.y;
            ws[lk + 2][lr] = u.z;
            ws[lk + 3][lr] = u.w;
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < kTileK; ++kk) {
            float a0 = xs[kk][tr], a1 = xs[kk][tr + 1];
            float b0 = ws[kk][tc], b1 = ws[kk][tc + 1];
            acc[0][0] = __builtin_fmaf(a0, b0, acc[0][0]);
            acc[0][1] = __builtin_fmaf(a0, b1, acc[0][1]);
            acc[1][0] = __builtin_fmaf(a1, b0, acc[1][0]);
            acc[1][1] = __builtin_fmaf(a1, b1, acc[1][1]);
        }
        __syncthreads();
    }
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j) {
            int t = t0 + tr + i, e = e0 + tc + j;
            if (t < S && e < E)
                logits[(int64_t)t * E + e] = acc[i][j];
        }
}

hipError_t launch_router_logits(const float* x, int32_t S, int32_t H, int32_t E, const float* w,
                                float* logits, hipStream_t st)
{
    if (S == 0)
        return hipSuccess;
    if (S <= kSmallS) {
        hipLaunchKernelGGL(router_logits_small, dim3((E + 3) / 4), dim3(256), 0, st, x, S, H, E, w,
                           logits);
    } else {
        dim3 grid((S + kTile - 1) / kTile, (E + kTile - 1) / kTile);
        hipLaunchKernelGGL(router_logits_tiled, grid, dim3(256), 0, st, x, S, H, E, w, logits);
    }
    return hipGetLastError();
}

/* ---- router selection: one wave per token ---------------------------------
 * Each lane holds the scores of experts lane, lane+64, ...; the top-k is k
 * rounds of a wave-wide maximum over 64-bit keys (order-preserving score bits
 * above the complemented expert id, so equal scores resolve to the lower id). */

constexpr int kMaxPerLane = 16; /* E <= 1024 */

__device__ __forceinline__ uint32_t order_bits(float c)
{
    uint32_t u = __float_as_uint(c);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(256) void router_select_kernel(const float* __restrict__ logits,
                                                            const float* __restrict__ bias,
                                                            int32_t S, int32_t E, int32_t k,
                                                            float rsf, int32_t* __restrict__ ids,
                                                            float* __restrict__ weights)
{
    __shared__ float sel_s[4][64];
    int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int t = blockIdx.x * 4 + wv;
    if (t >= S)
        return;
    const float* lt = logits + (int64_t)t * E;
    float s[kMaxPerLane];
    uint64_t key[kMaxPerLane];
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        int e = lane + 64 * i;
        if (e < E) {
            float sg = 1.0f / (1.0f + expf(-lt[e]));
            s[i] = sg;
            key[i] = ((uint64_t)order_bits(sg + bias[e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
        } else {
            s[i] = 0.0f;
            key[i] = 0;
        }
    }
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i)
            best = key[i] > best ? key[i] : best;
        for (int m = 32; m >= 1; m >>= 1) {
            uint64_t o = __shfl_xor(best, m, 64);
            best = o > best ? o : best;
        }
        int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
        float cand = 0.0f;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) {
            if (key[i] == best) {
                cand = s[i];
                key[i] = 0; /* taken */
            }
        }
        float sj = __shfl(cand, e & 63, 64);
        if (lane == 0) {
            sel_s[wv][j] = sj;
            ids[(int64_t)t * k + j] = e;
        }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    float denom = 0.0f;
    for (int j = 0; j < k; ++j)
        denom += sel_s[wv][j];
    if (lane < k)
        weights[(int64_t)t * k + lane] = rsf * (sel_s[wv][lane] / denom);
}

hipError_t launch_router_select(const float* logits, const float* bias, int32_t S, int32_t E,
                                int32_t k, float rsf, int32_t* ids, float* weights, hipStream_t st)
{
    if (S == 0)
        return hipSuccess;
    hipLaunchKernelGGL(router_select_kernel, dim3((S + 3) / 4), dim3(256), 0, st, logits, bias, S, E,
                       k, rsf, ids, weights);
    return hipGetLastError();
}

} // namespace coli
