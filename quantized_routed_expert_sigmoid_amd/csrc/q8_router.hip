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
#include "select.h"

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
 * Few tokens: one 256-thread workgroup per expert streams its router row once
 * (float4, coalesced, each wave a quarter of the row), keeps one partial sum
 * per token and reduces across lanes and waves.  Many tokens: 32 x 32 output
 * tiles through LDS.  Both sum in fp32 (the order is free: only the
 * selection decision depends on it, and inputs keep a score gap).
 *
 * With xq != nullptr the small-batch kernel also quantises x: workgroups
 * past the E router rows each quantise 32 blocks. */

__device__ __forceinline__ void quantize_blocks(const float* x, int64_t n_blocks, int8_t* q, float* d,
                                                int64_t gid)
{
    const int64_t blk = gid >> 3;
    const bool live = blk < n_blocks;
    const float4 v = live ? reinterpret_cast<const float4*>(x)[gid] : make_float4(0.f, 0.f, 0.f, 0.f);
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = fmaxf(a, shfl_xor(a, 1));
    a = fmaxf(a, shfl_xor(a, 2));
    a = fmaxf(a, shfl_xor(a, 4));
    if (!live)
        return;
    const float scale = a / 127.0f;
    const float inv = (a == 0.0f) ? 0.0f : 1.0f / scale;
    const uint32_t packed = (uint32_t)(q8_code(v.x, inv) & 0xFF) |
                            ((uint32_t)(q8_code(v.y, inv) & 0xFF) << 8) |
                            ((uint32_t)(q8_code(v.z, inv) & 0xFF) << 16) |
                            ((uint32_t)(q8_code(v.w, inv) & 0xFF) << 24);
    reinterpret_cast<uint32_t*>(q)[gid] = packed;
    if ((gid & 7) == 0)
        d[blk] = scale;
}

__global__ __launch_bounds__(256) void router_logits_small(const float* __restrict__ x, int32_t S,
                                                           int32_t H, int32_t E,
                                                           const float* __restrict__ w,
                                                           float* __restrict__ logits,
                                                           int8_t* __restrict__ xq,
                                                           float* __restrict__ xd)
{
    __shared__ float part[4][kSmallS];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int e = blockIdx.x;
    if (e >= E) {
        /* quantiser workgroups */
        const int64_t n_blocks = (int64_t)S * (H / 32);
        quantize_blocks(x, n_blocks, xq, xd, (int64_t)(e - E) * 256 + threadIdx.x);
        return;
    }
    const float4* wr = reinterpret_cast<const float4*>(w + (int64_t)e * H);
    float acc[kSmallS];
#pragma unroll
    for (int t = 0; t < kSmallS; ++t)
        acc[t] = 0.0f;
    const int n4 = H / 4;
    const int q0 = (wv * n4) / 4, q1 = ((wv + 1) * n4) / 4;
    for (int i = q0 + lane; i < q1; i += 64) {
        const float4 wv4 = wr[i];
#pragma unroll
        for (int t = 0; t < kSmallS; ++t) {
            if (t < S) {
                const float4 xv = reinterpret_cast<const float4*>(x + (int64_t)t * H)[i];
                acc[t] = __builtin_fmaf(wv4.x, xv.x, acc[t]);
                acc[t] = __builtin_fmaf(wv4.y, xv.y, acc[t]);
                acc[t] = __builtin_fmaf(wv4.z, xv.z, acc[t]);
                acc[t] = __builtin_fmaf(wv4.w, xv.w, acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kSmallS; ++t) {
        const float s = wave_sum(acc[t]);
        if (lane == 0)
            part[wv][t] = s;
    }
    __syncthreads();
    if (threadIdx.x < S)
        logits[(int64_t)threadIdx.x * E + e] =
            ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) + part[3][threadIdx.x];
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
        hipLaunchKernelGGL(router_logits_small, dim3(E), dim3(256), 0, st, x, S, H, E, w, logits,
                           (int8_t*)nullptr, (float*)nullptr);
    } else {
        dim3 grid((S + kTile - 1) / kTile, (E + kTile - 1) / kTile);
        hipLaunchKernelGGL(router_logits_tiled, grid, dim3(256), 0, st, x, S, H, E, w, logits);
    }
    return hipGetLastError();
}

hipError_t launch_route_prep_small(const float* x, int32_t S, int32_t H, int32_t E, const float* w,
                                   float* logits, int8_t* xq, float* xd, hipStream_t st)
{
    if (S == 0)
        return hipSuccess;
    const int64_t qthreads = (int64_t)S * (H / 32) * 8;
    const int64_t qgroups = (qthreads + 255) / 256;
    hipLaunchKernelGGL(router_logits_small, dim3((uint32_t)(E + qgroups)), dim3(256), 0, st, x, S, H, E,
                       w, logits, xq, xd);
    return hipGetLastError();
}

/* ---- router selection: one wave per token (select.h) ------------------- */

__global__ __launch_bounds__(256) void router_select_kernel(const float* __restrict__ logits,
                                                            const float* __restrict__ bias,
                                                            int32_t S, int32_t E, int32_t k,
                                                            float rsf, int32_t* __restrict__ ids,
                                                            float* __restrict__ weights)
{
    __shared__ float sel_s[4][64];
    const int wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    if (t >= S)
        return;
    select_token(logits + (int64_t)t * E, bias, E, k, rsf, ids + (int64_t)t * k,
                 weights + (int64_t)t * k, sel_s[wv], nullptr);
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
