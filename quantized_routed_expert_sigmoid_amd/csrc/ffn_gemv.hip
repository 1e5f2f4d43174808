/*
 * ffn_gemv.hip -- gated expert FFN on the integer dot path, GEMV form.
 *
 * ("Show HN: 如何在我的低配置电脑上运行 GLM-5.2": implemented-features section,
 * integer dot-product item -- Q8_0-style int8 activations -- and quantised-
 * kernel item -- int8 / packed int4 / packed int2 weights, per-row scales,
 * dequantised on use; Metal section: the routed-expert work is a SwiGLU;
 * resource-policy section: gate and up share one dispatch.)
 *
 * One wavefront is one job: an expert, up to kUnitTokens of its tokens, and
 * 64 weight rows (gate/up kernel: 32 gate rows and the same 32 up rows, i.e.
 * exactly one 32-block of the intermediate h; down kernel: 64 output rows).
 *
 * Lane mapping.  The wave is eight octets of eight lanes; octet o owns rows
 * 8o .. 8o+7 of the job.  For a K step of eight blocks, lane j of an octet
 * loads block (step*8 + j) of each of its octet's eight rows, so each load
 * instruction reads one contiguous run of eight blocks per row (128 bytes at
 * int4).  The exact int32 block partials go through LDS with a skewed 8x8
 * transpose per octet (conflict-free on 64 banks for both the writes and the
 * reads) so that lane j then owns row 8o + j and folds that row's eight
 * partials in ascending block order: acc = fma(d_b, (float)S_b, acc).
 *
 * Epilogue of the gate/up kernel: g = row scale * acc on lanes 0..31, u on
 * lanes 32..63, h = silu(g) * u, one Q8_0 block of h per token (amax over 32
 * lanes), codes and scale stored for the down kernel.
 */
#include "device_common.h"
#include "kernels.h"

namespace coli {

namespace {

constexpr int kRowsPerJob = 64;

struct JobLoc {
    int seg, unit, rb;
};

/* Field-wise select keeps the segment in scalar registers. */
__device__ __forceinline__ FfnSeg pick(const FfnArgs& a, int s)
{
    FfnSeg r;
    const bool one = s != 0;
    r.gate_w = one ? a.seg[1].gate_w : a.seg[0].gate_w;
    r.gate_s = one ? a.seg[1].gate_s : a.seg[0].gate_s;
    r.up_w = one ? a.seg[1].up_w : a.seg[0].up_w;
    r.up_s = one ? a.seg[1].up_s : a.seg[0].up_s;
    r.down_w = one ? a.seg[1].down_w : a.seg[0].down_w;
    r.down_s = one ? a.seg[1].down_s : a.seg[0].down_s;
    r.sorted = one ? a.seg[1].sorted : a.seg[0].sorted;
    r.units = one ? a.seg[1].units : a.seg[0].units;
    r.n_units = one ? a.seg[1].n_units : a.seg[0].n_units;
    r.k = one ? a.seg[1].k : a.seg[0].k;
    r.out_base = one ? a.seg[1].out_base : a.seg[0].out_base;
    r.max_units = one ? a.seg[1].max_units : a.seg[0].max_units;
    r.S = one ? a.seg[1].S : a.seg[0].S;
    r.rows = one ? a.seg[1].rows : a.seg[0].rows;
    r.n_mat = one ? a.seg[1].n_mat : a.seg[0].n_mat;
    return r;
}

__device__ __forceinline__ bool locate(const FfnArgs& a, int64_t job, int RB, JobLoc& L)
{
    const int64_t n0 = (int64_t)a.seg[0].max_units * RB;
    if (job < n0) {
        L.seg = 0;
    } else {
        job -= n0;
        if (a.nseg < 2 || job >= (int64_t)a.seg[1].max_units * RB)
            return false;
        L.seg = 1;
    }
    L.unit = (int)(job / RB);
    L.rb = (int)(job - (int64_t)L.unit * RB);
    return true;
}

/* Unit of a segment; false when the unit does not exist for this batch.
 * Units are clamped to the segment's positions and matrices, so a unit list
 * built from inconsistent offsets cannot move an access out of its buffer. */
__device__ __forceinline__ bool unit_info(const FfnSeg& sg, int u, int& e, int& pos0, int& ntok)
{
    if (sg.units) {
        if (u >= *sg.n_units || u >= sg.max_units)
            return false;
        const Unit U = sg.units[u];
        e = U.e;
        pos0 = U.pos0;
        ntok = U.ntok;
    } else {
        e = 0;
        pos0 = u * kUnitTokens;
        ntok = kUnitTokens;
    }
    if (e < 0 || e >= sg.n_mat || pos0 < 0 || pos0 >= sg.rows || ntok <= 0)
        return false;
    ntok = min(min(ntok, kUnitTokens), sg.rows - pos0);
    return true;
}

/* Token of sorted position pos, clamped to the batch. */
__device__ __forceinline__ int token_of(const FfnSeg& sg, int pos)
{
    const int tok = sg.sorted ? sg.sorted[pos] / sg.k : pos;
    return min(max(tok, 0), sg.S - 1);
}

template <int BITS>
__device__ __forceinline__ void load_block(const uint8_t* p, uint32_t (&w)[BITS])
{
    if constexpr (BITS == 8) {
        const uint4 a = reinterpret_cast<const uint4*>(p)[0];
        const uint4 b = reinterpret_cast<const uint4*>(p)[1];
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else if constexpr (BITS == 4) {
        const uint4 a = *reinterpret_cast<const uint4*>(p);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    } else {
        const uint2 a = *reinterpret_cast<const uint2*>(p);
        w[0] = a.x; w[1] = a.y;
    }
}

__device__ __forceinline__ void load_codes(const int8_t* p, uint32_t (&x)[8])
{
    const uint4 a = reinterpret_cast<const uint4*>(p)[0];
    const uint4 b = reinterpret_cast<const uint4*>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

/* LDS word of the partial written by lane `writer` of octet o for row rho of
 * the octet, token t: rows and writers are skewed by the octet index. */
__device__ __forceinline__ int part_index(int t, int o, int rho, int writer)
{
    return t * 512 + o * 64 + 8 * ((rho + o) & 7) + ((writer + o) & 7);
}

/* The K loop shared by both kernels: rows of this lane's octet start at
 * row0 (8 consecutive rows, rowbytes apart); act(t) gives token t's codes,
 * scl(t) its block scales; `rows_ok` masks rows past the matrix end.
 * Returns the folded accumulators of row (8o + lane-in-octet). */
template <int BITS>
__device__ __forceinline__ void k_loop(const uint8_t* row0, int64_t rowbytes, int nb, int ntok,
                                       const int8_t* const (&act)[kUnitTokens],
                                       const float* const (&scl)[kUnitTokens], int rows_ok,
                                       int32_t* part, float (&acc)[kUnitTokens])
{
    const int lane = threadIdx.x & 63;
    const int o = lane >> 3, j8 = lane & 7;
    for (int s = 0; s < nb; s += 8) {
        const int b = s + j8;
        const bool valid = b < nb;
        uint32_t w[8][BITS];
#pragma unroll
        for (int rho = 0; rho < 8; ++rho) {
            if (valid && rho < rows_ok) {
                load_block<BITS>(row0 + rho * rowbytes + (int64_t)b * (4 * BITS), w[rho]);
            } else {
#pragma unroll
                for (int i = 0; i < BITS; ++i)
                    w[rho][i] = 0;
            }
        }
#pragma unroll
        for (int t = 0; t < kUnitTokens; ++t) {
            if (t < ntok) {
                uint32_t x[8], xa[8];
                if (valid) {
                    load_codes(act[t] + (int64_t)b * 32, x);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        x[i] = 0;
                }
                prep_activation<BITS>(x, xa);
#pragma unroll
                for (int rho = 0; rho < 8; ++rho)
                    part[part_index(t, o, rho, j8)] = block_partial<BITS>(w[rho], xa);
            }
        }
        __syncthreads();
        const int nbs = min(8, nb - s);
#pragma unroll
        for (int t = 0; t < kUnitTokens; ++t) {
            if (t < ntok) {
                const float* d = scl[t] + s;
                for (int jj = 0; jj < nbs; ++jj)
                    acc[t] = __builtin_fmaf(d[jj], (float)part[part_index(t, o, j8, jj)], acc[t]);
            }
        }
        __syncthreads();
    }
}

} // namespace

template <int BITS>
__global__ __launch_bounds__(64) void ffn_gate_up_gemv(FfnArgs a)
{
    __shared__ int32_t part[kUnitTokens * 512];
    const int lane = threadIdx.x;
    const int o = lane >> 3;
    const int RB = a.I / 32;
    JobLoc L;
    if (!locate(a, blockIdx.x, RB, L))
        return;
    const FfnSeg sg = pick(a, L.seg);
    int e, pos0, ntok;
    if (!unit_info(sg, L.unit, e, pos0, ntok))
        return;
    const int nb = a.H / 32;
    const int64_t rowbytes = (int64_t)a.H * BITS / 8;
    const int8_t* act[kUnitTokens];
    const float* scl[kUnitTokens];
#pragma unroll
    for (int t = 0; t < kUnitTokens; ++t) {
        const int tok = token_of(sg, pos0 + (t < ntok ? t : 0));
        act[t] = a.xq + (int64_t)tok * a.H;
        scl[t] = a.xd + (int64_t)tok * nb;
    }
    /* octets 0..3: gate rows rb*32 + 8o ..; octets 4..7: the same up rows */
    const uint8_t* row0 = (o < 4 ? sg.gate_w : sg.up_w) +
                          ((int64_t)e * a.I + L.rb * 32 + 8 * (o & 3)) * rowbytes;
    float acc[kUnitTokens];
#pragma unroll
    for (int t = 0; t < kUnitTokens; ++t)
        acc[t] = 0.0f;
    k_loop<BITS>(row0, rowbytes, nb, ntok, act, scl, 8, part, acc);

    const int r = L.rb * 32 + (lane & 31);
    const float sc = (lane < 32 ? sg.gate_s : sg.up_s)[(int64_t)e * a.I + r];
    const int nbi = a.I / 32;
#pragma unroll
    for (int t = 0; t < kUnitTokens; ++t) {
        if (t < ntok) {
            const float v = sc * acc[t];
            const float u = shfl_xor(v, 32);
            const float h = canon_silu(v) * u;
            float am = lane < 32 ? __builtin_fabsf(h) : 0.0f;
            for (int m = 16; m >= 1; m >>= 1)
                am = fmaxf(am, shfl_xor(am, m));
            const float dsc = am / 127.0f;
            const float inv = (am == 0.0f) ? 0.0f : 1.0f / dsc;
            const int64_t row_out = sg.out_base + pos0 + t;
            if (lane < 32)
                a.hq[row_out * a.I + r] = (int8_t)q8_code(h, inv);
            if (lane == 0)
                a.hd[row_out * nbi + L.rb] = dsc;
        }
    }
}

template <int BITS>
__global__ __launch_bounds__(64) void ffn_down_gemv(FfnArgs a)
{
    __shared__ int32_t part[kUnitTokens * 512];
    const int lane = threadIdx.x;
    const int o = lane >> 3;
    const int RB = (a.H + kRowsPerJob - 1) / kRowsPerJob;
    JobLoc L;
    if (!locate(a, blockIdx.x, RB, L))
        return;
    const FfnSeg sg = pick(a, L.seg);
    int e, pos0, ntok;
    if (!unit_info(sg, L.unit, e, pos0, ntok))
        return;
    const int nb = a.I / 32;
    const int64_t rowbytes = (int64_t)a.I * BITS / 8;
    const int8_t* act[kUnitTokens];
    const float* scl[kUnitTokens];
#pragma unroll
    for (int t = 0; t < kUnitTokens; ++t) {
        const int64_t row_in = sg.out_base + pos0 + (t < ntok ? t : 0);
        act[t] = a.hq + row_in * a.I;
        scl[t] = a.hd + row_in * nb;
    }
    const int first = L.rb * kRowsPerJob + 8 * o;
    const int rows_ok = min(8, max(0, a.H - first));
    const uint8_t* row0 = sg.down_w + ((int64_t)e * a.H + first) * rowbytes;
    float acc[kUnitTokens];
#pragma unroll
    for (int t = 0; t < kUnitTokens; ++t)
        acc[t] = 0.0f;
    k_loop<BITS>(row0, rowbytes, nb, ntok, act, scl, rows_ok, part, acc);

    const int n = L.rb * kRowsPerJob + lane;
    if (n < a.H) {
        const float sc = sg.down_s[(int64_t)e * a.H + n];
#pragma unroll
        for (int t = 0; t < kUnitTokens; ++t)
            if (t < ntok)
                a.y[(int64_t)(sg.out_base + pos0 + t) * a.H + n] = sc * acc[t];
    }
}

static int64_t total_jobs(const FfnArgs& a, int RB)
{
    int64_t n = (int64_t)a.seg[0].max_units * RB;
    if (a.nseg > 1)
        n += (int64_t)a.seg[1].max_units * RB;
    return n;
}

hipError_t launch_ffn_gate_up(const FfnArgs& a, int32_t bits, hipStream_t st)
{
    const int64_t jobs = total_jobs(a, a.I / 32);
    if (jobs == 0)
        return hipSuccess;
    const dim3 grid((uint32_t)jobs), block(64);
    switch (bits) {
    case 8: hipLaunchKernelGGL(ffn_gate_up_gemv<8>, grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL(ffn_gate_up_gemv<4>, grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL(ffn_gate_up_gemv<2>, grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_ffn_down(const FfnArgs& a, int32_t bits, hipStream_t st)
{
    const int64_t jobs = total_jobs(a, (a.H + kRowsPerJob - 1) / kRowsPerJob);
    if (jobs == 0)
        return hipSuccess;
    const dim3 grid((uint32_t)jobs), block(64);
    switch (bits) {
    case 8: hipLaunchKernelGGL(ffn_down_gemv<8>, grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL(ffn_down_gemv<4>, grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL(ffn_down_gemv<2>, grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}

} // namespace coli
