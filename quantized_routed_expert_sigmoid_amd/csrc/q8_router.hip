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
 * (float4, coalesced, thread t taking float4 t, t + 256, ...), keeps one
 * partial sum per token and reduces across lanes and waves.  Many tokens: fp32 matrix
 * cores over 64 x 64 output tiles and K slices.  Both sum in fp32 (the order is free: only the
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

/* ST: tokens the instantiation carries (S <= ST; tokens past S recompute the
 * last one and are not stored, so no load sits under a branch); CH: float4
 * per thread per round. */
template <int ST, int CH>
__global__ __launch_bounds__(256) void router_logits_small(const float* __restrict__ x, int32_t S,
                                                           int32_t H, int32_t E,
                                                           const float* __restrict__ w,
                                                           float* __restrict__ logits,
                                                           int8_t* __restrict__ xq,
                                                           float* __restrict__ xd)
{
    __shared__ float part[4][ST];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int e = blockIdx.x;
    if (e >= E) {
        /* quantiser workgroups */
        const int64_t n_blocks = (int64_t)S * (H / 32);
        quantize_blocks(x, n_blocks, xq, xd, (int64_t)(e - E) * 256 + threadIdx.x);
        return;
    }
    const float4* wr = reinterpret_cast<const float4*>(w + (int64_t)e * H);
    float acc[ST];
#pragma unroll
    for (int t = 0; t < ST; ++t)
        acc[t] = 0.0f;
    const int n4 = H / 4;
    /* a round: each thread issues its CH row loads and every token's
     * matching x loads before any fma -- one memory round trip per round */
    for (int i0 = threadIdx.x; i0 < n4; i0 += 256 * CH) {
        float4 wv4[CH];
        float m[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            /* past the row the last float4 is loaded (in bounds) and its
             * products are multiplied by 0 (no branch, no early wait) */
            const int i = i0 + 256 * u;
            wv4[u] = wr[min(i, n4 - 1)];
            m[u] = i < n4 ? 1.0f : 0.0f;
        }
        float4 xv[ST][CH];
#pragma unroll
        for (int t = 0; t < ST; ++t) {
            const float4* xt = reinterpret_cast<const float4*>(x + (int64_t)min(t, S - 1) * H);
#pragma unroll
            for (int u = 0; u < CH; ++u)
                xv[t][u] = xt[min(i0 + 256 * u, n4 - 1)];
        }
#pragma unroll
        for (int t = 0; t < ST; ++t) {
#pragma unroll
            for (int u = 0; u < CH; ++u) {
                acc[t] = __builtin_fmaf(wv4[u].x * m[u], xv[t][u].x, acc[t]);
                acc[t] = __builtin_fmaf(wv4[u].y * m[u], xv[t][u].y, acc[t]);
                acc[t] = __builtin_fmaf(wv4[u].z * m[u], xv[t][u].z, acc[t]);
                acc[t] = __builtin_fmaf(wv4[u].w * m[u], xv[t][u].w, acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < ST; ++t) {
        const float s = wave_sum(acc[t]);
        if (lane == 0)
            part[wv][t] = s;
    }
    __syncthreads();
    if (threadIdx.x < S)
        logits[(int64_t)threadIdx.x * E + e] =
            ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) + part[3][threadIdx.x];
}

static void launch_logits_small(dim3 grid, int32_t S, hipStream_t st, const float* x, int32_t H, int32_t E,
                                const float* w, float* logits, int8_t* xq, float* xd)
{
    const dim3 block(256);
    if (S <= 1)
        hipLaunchKernelGGL((router_logits_small<1, 8>), grid, block, 0, st, x, S, H, E, w, logits, xq, xd);
    else if (S <= 2)
        hipLaunchKernelGGL((router_logits_small<2, 8>), grid, block, 0, st, x, S, H, E, w, logits, xq, xd);
    else if (S <= 4)
        hipLaunchKernelGGL((router_logits_small<4, 4>), grid, block, 0, st, x, S, H, E, w, logits, xq, xd);
    else
        hipLaunchKernelGGL((router_logits_small<kSmallS, 2>), grid, block, 0, st, x, S, H, E, w, logits, xq, xd);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

/* 16-wide k chunks of operands in flight per lane (ring slots) */
constexpr int kRouterDepth = 4;

/* Many tokens: fp32 matrix cores (v_mfma_f32_16x16x4f32).  A workgroup
 * computes a T-token x T-expert tile of one K slice (T = 32 WT); the launch
 * splits K into n_parts slices so that it fills the chip, and the selection
 * kernel adds the slices in order.  Wave (wm, wn) owns 16 WT tokens x 16 WT
 * experts, WT x WT MFMA tiles.  Operands come straight from global memory:
 * lane (r, kg) loads four consecutive k of each of its token rows and expert
 * rows, and MFMA i of a 16-k chunk takes element i -- any assignment of k to
 * MFMA slots is exact as long as both operands use the same one.  Rows past
 * S or E load the last row; their results are not stored.  Larger wave tiles
 * read each operand for more MFMAs (WT = 4: half the L1 traffic of WT = 2).
 * D chunks of 16 k are in flight per lane (4: the loads of one chunk ahead
 * left the many-token launches waiting on memory). */
template <int WT, int D>
__global__ __launch_bounds__(256) void router_logits_mfma(const float* __restrict__ x, int32_t S,
                                                          int32_t H, int32_t E,
                                                          const float* __restrict__ w,
                                                          float* __restrict__ part, int32_t n_parts,
                                                          int8_t* __restrict__ xq, float* __restrict__ xd)
{
    constexpr int T = 32 * WT, WH = 16 * WT;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int r = lane & 15, kg = lane >> 4;
    const int tiles_e = (E + T - 1) / T;
    const int n_logit_groups = ((S + T - 1) / T) * tiles_e * n_parts;
    if ((int)blockIdx.x >= n_logit_groups) {
        /* quantiser workgroups (launched only with xq != nullptr) */
        quantize_blocks(x, (int64_t)S * (H / 32), xq, xd, (int64_t)(blockIdx.x - n_logit_groups) * 256 + threadIdx.x);
        return;
    }
    const int p = blockIdx.x % n_parts;
    const int tile = blockIdx.x / n_parts;
    const int t0 = (tile / tiles_e) * T + (wv >> 1) * WH;
    const int e0 = (tile % tiles_e) * T + (wv & 1) * WH;
    const float* xr[WT];
    const float* wr[WT];
#pragma unroll
    for (int m = 0; m < WT; ++m) {
        xr[m] = x + (int64_t)min(t0 + 16 * m + r, S - 1) * H + 4 * kg;
        wr[m] = w + (int64_t)min(e0 + 16 * m + r, E - 1) * H + 4 * kg;
    }
    const int nchunk = H / 16;
    const int c0 = (int)((int64_t)p * nchunk / n_parts);
    const int c1 = (int)((int64_t)(p + 1) * nchunk / n_parts);
    f32x4 acc[WT][WT];
#pragma unroll
    for (int m = 0; m < WT; ++m)
#pragma unroll
        for (int n = 0; n < WT; ++n)
            acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    /* a ring of D chunks in flight: slot i holds chunk c + i; a chunk past
     * the slice reloads the slice's last one (in bounds) and enters with
     * its token operand zeroed, adding +0 products, so that the loop needs
     * no branch around its loads */
    float4 a[D][WT], b[D][WT];
#pragma unroll
    for (int i = 0; i < D; ++i)
#pragma unroll
        for (int m = 0; m < WT; ++m) {
            const int64_t ci = min(c0 + i, c1 - 1);
            a[i][m] = *reinterpret_cast<const float4*>(xr[m] + ci * 16);
            b[i][m] = *reinterpret_cast<const float4*>(wr[m] + ci * 16);
        }
    for (int c = c0; c < c1; c += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const float live = c + i < c1 ? 1.0f : 0.0f;
            float4 am[WT];
#pragma unroll
            for (int m = 0; m < WT; ++m)
                am[m] = make_float4(a[i][m].x * live, a[i][m].y * live, a[i][m].z * live, a[i][m].w * live);
#pragma unroll
            for (int m = 0; m < WT; ++m)
#pragma unroll
                for (int n = 0; n < WT; ++n) {
                    acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(am[m].x, b[i][n].x, acc[m][n], 0, 0, 0);
                    acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(am[m].y, b[i][n].y, acc[m][n], 0, 0, 0);
                    acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(am[m].z, b[i][n].z, acc[m][n], 0, 0, 0);
                    acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(am[m].w, b[i][n].w, acc[m][n], 0, 0, 0);
                }
            const int64_t cn = min(c + i + D, c1 - 1);
#pragma unroll
            for (int m = 0; m < WT; ++m) {
                a[i][m] = *reinterpret_cast<const float4*>(xr[m] + cn * 16);
                b[i][m] = *reinterpret_cast<const float4*>(wr[m] + cn * 16);
            }
        }
    }
    /* lane holds D[4 kg + v][r]: token t0 + 16m + 4kg + v, expert e0 + 16n + r */
    float* out = part + (int64_t)p * S * E;
#pragma unroll
    for (int m = 0; m < WT; ++m)
#pragma unroll
        for (int n = 0; n < WT; ++n)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = t0 + 16 * m + 4 * kg + v, e = e0 + 16 * n + r;
                if (t < S && e < E)
                    out[(int64_t)t * E + e] = acc[m][n][v];
            }
}

/* The many-token router launch; with xq != nullptr the grid carries the
 * quantiser workgroups of x's Q8_0 after the logit tiles. */
static hipError_t launch_logits_mfma(const float* x, int32_t S, int32_t H, int32_t E, const float* w,
                                     float* logits, int8_t* xq, float* xd, hipStream_t st)
{
    const int32_t parts = router_parts(S, E, H);
    const int32_t T = router_tile(S, E);
    const int64_t tiles = (int64_t)((S + T - 1) / T) * ((E + T - 1) / T);
    const int64_t qgroups = xq ? ((int64_t)S * (H / 32) * 8 + 255) / 256 : 0;
    const dim3 grid((uint32_t)(tiles * parts + qgroups)), block(256);
    if (T == 128)
        hipLaunchKernelGGL((router_logits_mfma<4, kRouterDepth>), grid, block, 0, st, x, S, H, E, w, logits, parts,
                           xq, xd);
    else
        hipLaunchKernelGGL((router_logits_mfma<2, kRouterDepth>), grid, block, 0, st, x, S, H, E, w, logits, parts,
                           xq, xd);
    return hipGetLastError();
}

hipError_t launch_router_logits(const float* x, int32_t S, int32_t H, int32_t E, const float* w,
                                float* logits, hipStream_t st)
{
    if (S == 0)
        return hipSuccess;
    if (S <= kSmallS) {
        launch_logits_small(dim3(E), S, st, x, H, E, w, logits, (int8_t*)nullptr, (float*)nullptr);
        return hipGetLastError();
    }
    return launch_logits_mfma(x, S, H, E, w, logits, nullptr, nullptr, st);
}

hipError_t launch_route_prep(const float* x, int32_t S, int32_t H, int32_t E, const float* w, float* logits,
                             int8_t* xq, float* xd, hipStream_t st)
{
    if (S <= kSmallS)
        return launch_route_prep_small(x, S, H, E, w, logits, xq, xd, st);
    return launch_logits_mfma(x, S, H, E, w, logits, xq, xd, st);
}

hipError_t launch_route_prep_small(const float* x, int32_t S, int32_t H, int32_t E, const float* w,
                                   float* logits, int8_t* xq, float* xd, hipStream_t st)
{
    if (S == 0)
        return hipSuccess;
    const int64_t qthreads = (int64_t)S * (H / 32) * 8;
    const int64_t qgroups = (qthreads + 255) / 256;
    launch_logits_small(dim3((uint32_t)(E + qgroups)), S, st, x, H, E, w, logits, xq, xd);
    return hipGetLastError();
}

/* ---- router selection: one wave per token (select.h) ------------------- */

__global__ __launch_bounds__(256) void router_select_kernel(const float* __restrict__ logits,
                                                            int32_t n_parts,
                                                            const float* __restrict__ bias,
                                                            int32_t S, int32_t E, int32_t k,
                                                            float rsf, RouteOpts opt,
                                                            int32_t* __restrict__ ids,
                                                            float* __restrict__ weights)
{
    __shared__ __attribute__((aligned(16))) float sel_s[4][kSelScratch];
    const int wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    if (t >= S)
        return;
    select_token<true>(logits + (int64_t)t * E, bias, E, k, rsf, ids + (int64_t)t * k,
                       weights + (int64_t)t * k, sel_s[wv], nullptr, n_parts, (int64_t)S * E, opt);
}

hipError_t launch_router_select(const float* logits, int32_t n_parts, const float* bias, int32_t S,
                                int32_t E, int32_t k, float rsf, const RouteOpts& opt, int32_t* ids,
                                float* weights, hipStream_t st)
{
    if (S == 0)
        return hipSuccess;
    hipLaunchKernelGGL(router_select_kernel, dim3((S + 3) / 4), dim3(256), 0, st, logits, n_parts, bias,
                       S, E, k, rsf, opt, ids, weights);
    return hipGetLastError();
}

} // namespace coli
