/*
 * ffn_mfma.hip -- gated expert FFN on the integer dot path, grouped-GEMM form
 * on the int8 matrix cores, for experts that hold many tokens of the batch
 * (prefill / verify batches: "Show HN: 如何在我的低配置电脑上运行 GLM-5.2",
 * implemented features, batched-union MoE item; integer dot-product and
 * quantised-kernel items; Metal section: SwiGLU; resource-policy section:
 * gate and up in one dispatch).
 *
 * Work unit: one expert and up to kMfmaUnitTokens of its sorted positions
 * (up to four N-tiles of 16 tokens).  A 256-thread workgroup covers 64 row
 * dots (gate/up kernel: 32 gate rows and the same 32 up rows, one 32-block of
 * h; down kernel: 64 output rows); wave w owns the 16-row M-tile w.
 *
 * One v_mfma_i32_16x16x32_i8 covers exactly one Q8_0 block (K = 32), so its
 * int32 result is the exact block partial of 16 rows x 16 tokens.  Weights
 * enter as their packed fields shifted to the top of each byte (2^(8-b) * v,
 * see qdot.h) and activations in the matching operand order; the 2^(8-b)
 * factor is taken out of the block scale (exact whenever d * 2^-(8-b) is a
 * normal number; otherwise the wave shifts the partials back instead).  The
 * fp32 fold is the canonical one: four consecutive block groups, each from +0
 * in ascending block order, group sums added in order, then the row scale.
 *
 * Per K step of four blocks the workgroup stages the weight tile (64 rows x 4
 * blocks) and the activation tile (64 tokens x 4 blocks, operand order, with
 * scales) in LDS, double-buffered: the next step's global loads are in flight
 * while the current step's MFMAs and folds run.
 */
#include "device_common.h"
#include "kernels.h"

namespace coli {

namespace {

constexpr int kStep = 4;   /* K blocks per step */
constexpr int kTokPad = 9; /* operand words per (token, block) in LDS (8 + 1 pad) */

template <int BITS>
struct MfmaLds {
    uint32_t a[2][64][kStep][BITS + 1];  /* weight tile, natural packed words (+1 pad) */
    uint32_t b[2][64][kStep][kTokPad];   /* activation operands */
    float d[2][64][kStep];               /* activation block scales */
};

struct EpiLds {
    float v[64][65];                     /* [row dot][token] */
};

template <int BITS>
union MfmaShared {
    MfmaLds<BITS> k;
    EpiLds e;
};

struct MLoc {
    int seg, unit, rb;
};

__device__ __forceinline__ FfnSeg pick_m(const FfnArgs& a, int s)
{
    const bool one = s != 0;
    FfnSeg r = one ? a.seg[1] : a.seg[0];
    return r;
}

__device__ __forceinline__ bool locate_m(const FfnArgs& a, int64_t job, int RB, MLoc& L)
{
    const int64_t n0 = (int64_t)a.seg[0].max_munits * RB;
    if (job < n0) {
        L.seg = 0;
    } else {
        job -= n0;
        if (a.nseg < 2 || job >= (int64_t)a.seg[1].max_munits * RB)
            return false;
        L.seg = 1;
    }
    L.unit = (int)(job / RB);
    L.rb = (int)(job - (int64_t)L.unit * RB);
    return true;
}

__device__ __forceinline__ bool munit_info(const FfnSeg& sg, int u, int& e, int& pos0, int& ntok)
{
    if (sg.munits) {
        if (u >= *sg.n_munits || u >= sg.max_munits)
            return false;
        const Unit U = sg.munits[u];
        e = U.e;
        pos0 = U.pos0;
        ntok = U.ntok;
    } else {
        e = 0;
        pos0 = u * kMfmaUnitTokens;
        ntok = kMfmaUnitTokens;
    }
    if (e < 0 || e >= sg.n_mat || pos0 < 0 || pos0 >= sg.rows || ntok <= 0)
        return false;
    ntok = min(min(ntok, kMfmaUnitTokens), sg.rows - pos0);
    return true;
}

__device__ __forceinline__ int token_of_m(const FfnSeg& sg, int pos)
{
    const int tok = sg.sorted ? sg.sorted[pos] / sg.k : pos;
    return min(max(tok, 0), sg.S - 1);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

/* Registers holding one thread's share of the next step's global loads. */
template <int BITS>
struct Prefetch {
    uint32_t w[BITS];
    uint32_t x[8];
    float d;
};

/* Thread l of the workgroup loads block (b0 + (l & 3)) of row dot (l >> 2)
 * and of token (l >> 2). */
template <int BITS>
__device__ __forceinline__ void fetch(Prefetch<BITS>& P, const uint8_t* wrow, int64_t rowbytes,
                                      bool row_ok, const int8_t* xrow, const float* xdrow, bool tok_ok,
                                      int b, int nb)
{
    (void)rowbytes;
    const bool blk_ok = b < nb;
    if (row_ok && blk_ok) {
        const uint8_t* p = wrow + (int64_t)b * (4 * BITS);
        if constexpr (BITS == 8) {
            const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
            const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + 1);
            P.w[0] = u.x; P.w[1] = u.y; P.w[2] = u.z; P.w[3] = u.w;
            P.w[4] = v.x; P.w[5] = v.y; P.w[6] = v.z; P.w[7] = v.w;
        } else if constexpr (BITS == 4) {
            const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
            P.w[0] = u.x; P.w[1] = u.y; P.w[2] = u.z; P.w[3] = u.w;
        } else {
            const u32x2 u = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
            P.w[0] = u.x; P.w[1] = u.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < BITS; ++i)
            P.w[i] = 0;
    }
    if (tok_ok && blk_ok) {
        const uint4* q = reinterpret_cast<const uint4*>(xrow + (int64_t)b * 32);
        const uint4 u = q[0], v = q[1];
        P.x[0] = u.x; P.x[1] = u.y; P.x[2] = u.z; P.x[3] = u.w;
        P.x[4] = v.x; P.x[5] = v.y; P.x[6] = v.z; P.x[7] = v.w;
        P.d = xdrow[b];
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            P.x[i] = 0;
        P.d = 0.0f;
    }
}

template <int BITS>
__device__ __forceinline__ void commit(const Prefetch<BITS>& P, MfmaLds<BITS>& S, int buf)
{
    const int l = threadIdx.x, r = l >> 2, j = l & 3;
#pragma unroll
    for (int i = 0; i < BITS; ++i)
        S.a[buf][r][j][i] = P.w[i];
    uint32_t xa[8];
    prep_activation<BITS>(P.x, xa);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        S.b[buf][r][j][i] = xa[i];
    S.d[buf][r][j] = P.d;
}

/* A operand of lane group g (elements 8g .. 8g+7 of the block, in the order
 * prep_activation gives the activation codes) from the row's packed words. */
template <int BITS>
__device__ __forceinline__ long a_operand(const uint32_t* w, int g)
{
    uint32_t lo, hi;
    if constexpr (BITS == 8) {
        lo = w[2 * g];
        hi = w[2 * g + 1];
    } else if constexpr (BITS == 4) {
        lo = w[g] & 0xF0F0F0F0u;
        hi = (w[g] << 4) & 0xF0F0F0F0u;
    } else {
        const uint32_t ww = w[g >> 1];
        const int r0 = 2 * (g & 1);
        lo = (ww << (2 * r0)) & 0xC0C0C0C0u;
        hi = (ww << (2 * r0 + 2)) & 0xC0C0C0C0u;
    }
    return (long)(((uint64_t)hi << 32) | lo);
}

/* B operand of lane group g: activation operand words 2g, 2g+1. */
__device__ __forceinline__ long b_operand(const uint32_t* xa, int g)
{
    return (long)(((uint64_t)xa[2 * g + 1] << 32) | xa[2 * g]);
}

/* The K loop shared by both kernels.  Returns tot[n][v]: the folded sums of
 * rows 16w + 4(lane/16) + v for token 16n + lane%16. */
template <int BITS>
__device__ __forceinline__ void mfma_k_loop(MfmaLds<BITS>& S, const uint8_t* wrow, int64_t rowbytes,
                                            bool row_ok, const int8_t* xrow, const float* xdrow,
                                            bool tok_ok, int nb, int ntiles, float (&tot)[4][4])
{
    constexpr int SHIFT = 8 - BITS;
    const float unscale = 1.0f / (float)(1 << SHIFT);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int j_ld = threadIdx.x & 3;
    const int bnd1 = nb / 4, bnd2 = (2 * nb) / 4, bnd3 = (3 * nb) / 4;
    float acc[4][4];
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            acc[n][v] = 0.0f;
            tot[n][v] = 0.0f;
        }
    const int nsteps = (nb + kStep - 1) / kStep;
    Prefetch<BITS> P;
    fetch<BITS>(P, wrow, rowbytes, row_ok, xrow, xdrow, tok_ok, j_ld, nb);
    commit<BITS>(P, S, 0);
    __syncthreads();
    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        if (st + 1 < nsteps)
            fetch<BITS>(P, wrow, rowbytes, row_ok, xrow, xdrow, tok_ok, (st + 1) * kStep + j_ld, nb);
#pragma unroll
        for (int j = 0; j < kStep; ++j) {
            const int b = st * kStep + j;
            if (b >= nb)
                break;
            /* canonical group boundaries (a repeated boundary adds +0) */
            const int flushes = (b == bnd1) + (b == bnd2) + (b == bnd3);
            if (flushes) {
#pragma unroll
                for (int n = 0; n < 4; ++n)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        tot[n][v] = tot[n][v] + acc[n][v];
                        acc[n][v] = 0.0f;
                    }
            }
            const long A = a_operand<BITS>(S.a[buf][16 * wv + r][j], g);
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                if (n < ntiles) {
                    const int t = 16 * n + r;
                    const long B = b_operand(S.b[buf][t][j], g);
                    i32x4 c = {0, 0, 0, 0};
                    c = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, c, 0, 0, 0);
                    const float d = S.d[buf][t][j];
                    const float ds = d * unscale;
                    const bool exact = (d == 0.0f) || (ds >= 1.17549435e-38f);
                    if (SHIFT == 0 || __ballot(!exact) == 0) {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[n][v] = __builtin_fmaf(SHIFT ? ds : d, (float)c[v], acc[n][v]);
                    } else {
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[n][v] = __builtin_fmaf(d, (float)(c[v] >> SHIFT), acc[n][v]);
                    }
                }
            }
        }
        __syncthreads();
        if (st + 1 < nsteps)
            commit<BITS>(P, S, buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            tot[n][v] = tot[n][v] + acc[n][v];
}

} // namespace

template <int BITS>
__global__ __launch_bounds__(256) void ffn_gate_up_mfma(FfnArgs a)
{
    __shared__ MfmaShared<BITS> sm;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int RB = a.I / 32;
    MLoc L;
    if (!locate_m(a, blockIdx.x, RB, L))
        return;
    const FfnSeg sg = pick_m(a, L.seg);
    int e, pos0, ntok;
    if (!munit_info(sg, L.unit, e, pos0, ntok))
        return;
    const int nb = a.H / 32;
    const int64_t rowbytes = (int64_t)a.H * BITS / 8;
    /* this thread's load lane: row dot l>>2 (gate rows 0..31, then up) and token l>>2 */
    const int rd = threadIdx.x >> 2;
    const uint8_t* wrow = (rd < 32 ? sg.gate_w : sg.up_w) +
                          ((int64_t)e * a.I + L.rb * 32 + (rd & 31)) * rowbytes;
    const bool tok_ok = rd < ntok;
    const int tok = token_of_m(sg, pos0 + (tok_ok ? rd : 0));
    const int8_t* xrow = a.xq + (int64_t)tok * a.H;
    const float* xdrow = a.xd + (int64_t)tok * nb;
    const int ntiles = (ntok + 15) / 16;
    float tot[4][4];
    mfma_k_loop<BITS>(sm.k, wrow, rowbytes, true, xrow, xdrow, tok_ok, nb, ntiles, tot);

    /* epilogue: scaled g (row dots 0..31) and u (32..63) through LDS, then
     * h = silu(g) * u and one Q8_0 block of h per token */
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int rdot = 16 * wv + 4 * g + v;
        const float sc = (rdot < 32 ? sg.gate_s : sg.up_s)[(int64_t)e * a.I + L.rb * 32 + (rdot & 31)];
#pragma unroll
        for (int n = 0; n < 4; ++n)
            if (n < ntiles)
                sm.e.v[rdot][16 * n + r] = sc * tot[n][v];
    }
    __syncthreads();
    const int t = threadIdx.x >> 2, q = threadIdx.x & 3;
    float h[8];
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float gv = sm.e.v[8 * q + i][t];
        const float uv = sm.e.v[32 + 8 * q + i][t];
        h[i] = canon_silu(gv) * uv;
        am = fmaxf(am, __builtin_fabsf(h[i]));
    }
    am = fmaxf(am, shfl_xor(am, 1));
    am = fmaxf(am, shfl_xor(am, 2));
    if (t < ntok) {
        const float dsc = am / 127.0f;
        const float inv = (am == 0.0f) ? 0.0f : 1.0f / dsc;
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo |= (uint32_t)(q8_code(h[i], inv) & 0xFF) << (8 * i);
            hi |= (uint32_t)(q8_code(h[4 + i], inv) & 0xFF) << (8 * i);
        }
        const int64_t row_out = sg.out_base + pos0 + t;
        *reinterpret_cast<uint2*>(a.hq + row_out * a.I + L.rb * 32 + 8 * q) = make_uint2(lo, hi);
        if (q == 0)
            a.hd[row_out * (a.I / 32) + L.rb] = dsc;
    }
}

template <int BITS>
__global__ __launch_bounds__(256) void ffn_down_mfma(FfnArgs a)
{
    __shared__ MfmaShared<BITS> sm;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int RB = (a.H + 63) / 64;
    MLoc L;
    if (!locate_m(a, blockIdx.x, RB, L))
        return;
    const FfnSeg sg = pick_m(a, L.seg);
    int e, pos0, ntok;
    if (!munit_info(sg, L.unit, e, pos0, ntok))
        return;
    const int nb = a.I / 32;
    const int64_t rowbytes = (int64_t)a.I * BITS / 8;
    const int rd = threadIdx.x >> 2;
    const int row = L.rb * 64 + rd;
    const bool row_ok = row < a.H;
    const uint8_t* wrow = sg.down_w + ((int64_t)e * a.H + (row_ok ? row : 0)) * rowbytes;
    const bool tok_ok = rd < ntok;
    const int64_t row_in = sg.out_base + pos0 + (tok_ok ? rd : 0);
    const int8_t* xrow = a.hq + row_in * a.I;
    const float* xdrow = a.hd + row_in * nb;
    const int ntiles = (ntok + 15) / 16;
    float tot[4][4];
    mfma_k_loop<BITS>(sm.k, wrow, rowbytes, row_ok, xrow, xdrow, tok_ok, nb, ntiles, tot);

    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int rr = 16 * wv + 4 * g + v;
        const int n_out = L.rb * 64 + rr;
        const float sc = n_out < a.H ? sg.down_s[(int64_t)e * a.H + n_out] : 0.0f;
#pragma unroll
        for (int n = 0; n < 4; ++n)
            if (n < ntiles)
                sm.e.v[rr][16 * n + r] = sc * tot[n][v];
    }
    __syncthreads();
    /* thread: token t, rows 16q .. 16q+15 of the block */
    const int t = threadIdx.x >> 2, q = threadIdx.x & 3;
    if (t < ntok) {
        float* yr = a.y + (int64_t)(sg.out_base + pos0 + t) * a.H + L.rb * 64 + 16 * q;
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
            if (L.rb * 64 + 16 * q + i < a.H) {
                const float4 o = make_float4(sm.e.v[16 * q + i][t], sm.e.v[16 * q + i + 1][t],
                                             sm.e.v[16 * q + i + 2][t], sm.e.v[16 * q + i + 3][t]);
                *reinterpret_cast<float4*>(yr + i) = o;
            }
        }
    }
}

static int64_t total_mjobs(const FfnArgs& a, int RB)
{
    int64_t n = (int64_t)a.seg[0].max_munits * RB;
    if (a.nseg > 1)
        n += (int64_t)a.seg[1].max_munits * RB;
    return n;
}

hipError_t launch_ffn_gate_up_mfma(const FfnArgs& a, int32_t bits, hipStream_t st)
{
    const int64_t jobs = total_mjobs(a, a.I / 32);
    if (jobs == 0)
        return hipSuccess;
    const dim3 grid((uint32_t)jobs), block(256);
    switch (bits) {
    case 8: hipLaunchKernelGGL(ffn_gate_up_mfma<8>, grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL(ffn_gate_up_mfma<4>, grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL(ffn_gate_up_mfma<2>, grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_ffn_down_mfma(const FfnArgs& a, int32_t bits, hipStream_t st)
{
    const int64_t jobs = total_mjobs(a, (a.H + 63) / 64);
    if (jobs == 0)
        return hipSuccess;
    const dim3 grid((uint32_t)jobs), block(256);
    switch (bits) {
    case 8: hipLaunchKernelGGL(ffn_down_mfma<8>, grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL(ffn_down_mfma<4>, grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL(ffn_down_mfma<2>, grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}

} // namespace coli
