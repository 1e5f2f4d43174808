/*
 * device_common.h -- gfx950 device helpers shared by libcolibri's kernels:
 * the canonical rounding, exp and SiLU of the layer, and wavefront-64
 * cross-lane helpers.
 */
#ifndef COLI_DEVICE_COMMON_H
#define COLI_DEVICE_COMMON_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#define COLI_QDOT_FN __device__ __forceinline__
#define COLI_PERM(a, b, s) __builtin_amdgcn_perm((a), (b), (s))
#define COLI_SDOT4(a, b, c) __builtin_amdgcn_sdot4((int)(a), (int)(b), (c), false)
#define COLI_SDOT8(a, b, c) __builtin_amdgcn_sdot8((int)(a), (int)(b), (c), false)
#include "qdot.h"

namespace coli {

constexpr int kWave = 64;

/* Round half away from zero (the rounding of the Q8_0 codes). */
__device__ __forceinline__ float round_half_away(float v)
{
    float t = __builtin_truncf(v);
    if (__builtin_fabsf(v - t) >= 0.5f)
        t += (v > 0.0f) ? 1.0f : -1.0f;
    return t;
}

/* Q8_0 code of v given the block's reciprocal scale. */
__device__ __forceinline__ int32_t q8_code(float v, float inv)
{
    float r = round_half_away(v * inv);
    r = r > 127.0f ? 127.0f : r;
    r = r < -127.0f ? -127.0f : r;
    return (int32_t)r;
}

/* exp for the SiLU: exp(z) = 2^n exp(r) with n the nearest integer to z/ln2
 * and r = z - n ln2 taken in two fused steps (Cody & Waite, 1980), ln2 split
 * into a head of 16 significant bits (n * head exact for |n| <= 128) and a
 * fp32 tail; exp(r) by the degree-7 Taylor polynomial with coefficients 1/j!
 * rounded to fp32, Horner with fma.  +inf above 88, +0 below -87. */
struct ExpConsts {
    static constexpr double ln2 = 0.69314718055994530942;
    static constexpr float log2e = (float)(1.0 / ln2);
    static constexpr double ln2_hi_d = (double)(long long)(ln2 * 65536.0 + 0.5) / 65536.0;
    static constexpr float ln2_hi = (float)ln2_hi_d;
    static constexpr float ln2_lo = (float)(ln2 - ln2_hi_d);
    static constexpr float c0 = (float)(1.0 / 1.0);
    static constexpr float c1 = (float)(1.0 / 1.0);
    static constexpr float c2 = (float)(1.0 / 2.0);
    static constexpr float c3 = (float)(1.0 / 6.0);
    static constexpr float c4 = (float)(1.0 / 24.0);
    static constexpr float c5 = (float)(1.0 / 120.0);
    static constexpr float c6 = (float)(1.0 / 720.0);
    static constexpr float c7 = (float)(1.0 / 5040.0);
};

__device__ __forceinline__ float canon_exp(float z)
{
    if (z > 88.0f)
        return __builtin_inff();
    if (z < -87.0f)
        return 0.0f;
    using C = ExpConsts;
    float n = __builtin_rintf(z * C::log2e);
    float r = __builtin_fmaf(-n, C::ln2_hi, z);
    r = __builtin_fmaf(-n, C::ln2_lo, r);
    float p = C::c7;
    p = __builtin_fmaf(p, r, C::c6);
    p = __builtin_fmaf(p, r, C::c5);
    p = __builtin_fmaf(p, r, C::c4);
    p = __builtin_fmaf(p, r, C::c3);
    p = __builtin_fmaf(p, r, C::c2);
    p = __builtin_fmaf(p, r, C::c1);
    p = __builtin_fmaf(p, r, C::c0);
    return __builtin_ldexpf(p, (int)n);
}

__device__ __forceinline__ float canon_silu(float g)
{
    return g / (1.0f + canon_exp(-g));
}

/* Cross-lane helpers (wavefront of 64). */
__device__ __forceinline__ float shfl_xor(float v, int m)
{
    return __shfl_xor(v, m, kWave);
}

__device__ __forceinline__ int32_t shfl_xor_i(int32_t v, int m)
{
    return __shfl_xor(v, m, kWave);
}

__device__ __forceinline__ float wave_sum(float v)
{
    for (int m = 32; m >= 1; m >>= 1)
        v += shfl_xor(v, m);
    return v;
}

/* Wave-wide max / min of unsigned values with DPP lane moves (no LDS
 * crossbar): row shifts 1, 2, 4, 8 scan each 16-lane row, row broadcasts 15
 * and 31 carry the row results into the last row; lane 63 holds the result,
 * which is read back as a uniform value.  Lanes a move does not reach keep
 * the operation's identity. */
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v)
{
    const int id = MAX ? 0 : (int)0xFFFFFFFFu;
    auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x111, 0xF, 0xF, false)); /* row_shr:1 */
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x112, 0xF, 0xF, false)); /* row_shr:2 */
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x114, 0xF, 0xF, false)); /* row_shr:4 */
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x118, 0xF, 0xF, false)); /* row_shr:8 */
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xA, 0xF, false)); /* row_bcast:15 */
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xC, 0xF, false)); /* row_bcast:31 */
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

} // namespace coli

#endif
