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
#include "select.h"

namespace coli {

namespace {

constexpr int kRowsPerJob = 64;

struct JobLoc {
    int seg, unit, rb;
};

/* Field-wise select keeps the segment in scalar registers (every field of
 * FfnSeg is selected; the zero initialisation only guards additions). */
__device__ __forceinline__ FfnSeg pick(const FfnArgs& a, int s)
{
    FfnSeg r = {};
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
    r.munits = one ? a.seg[1].munits : a.seg[0].munits;
    r.n_munits = one ? a.seg[1].n_munits : a.seg[0].n_munits;
    r.max_munits = one ? a.seg[1].max_munits : a.seg[0].max_munits;
    r.k = one ? a.seg[1].k : a.seg[0].k;
    r.out_base = one ? a.seg[1].out_base : a.seg[0].out_base;
    r.max_units = one ? a.seg[1].max_units : a.seg[0].max_units;
    r.S = one ? a.seg[1].S : a.seg[0].S;
    r.rows = one ? a.seg[1].rows : a.seg[0].rows;
    r.n_mat = one ? a.seg[1].n_mat : a.seg[0].n_mat;
    r.gu_gb = one ? a.seg[1].gu_gb : a.seg[0].gu_gb;
    r.d_gb = one ? a.seg[1].d_gb : a.seg[0].d_gb;
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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

/* Weight loads are streamed once per call: nontemporal loads keep them from
 * displacing reused data in the caches (measured +5-10% read bandwidth). */
template <int BITS>
__device__ __forceinline__ void load_block(const uint8_t* p, uint32_t (&w)[BITS])
{
    if constexpr (BITS == 8) {
        const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + 1);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else if constexpr (BITS == 4) {
        const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    } else {
        const u32x2 a = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        w[0] = a.x; w[1] = a.y;
    }
}

/* Orders one wave's LDS writes before its following LDS reads by other lanes
 * of the same wave.  A wave's LDS instructions execute in issue order, so only
 * the compiler has to be kept from moving accesses across this point. */
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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

/* Waves per job: wave g computes fold group g (see block_group). */
constexpr int kGroups = 4;

/* First block of fold group g out of nb blocks: the canonical fold adds four
 * consecutive groups of blocks, each folded from +0 in ascending order. */
__device__ __forceinline__ int block_group(int g, int nb)
{
    return (g * nb) / kGroups;
}

/* Blocks of one fold group that a wave stages in LDS (K <= 8192). */
constexpr int kMaxGroupBlocks = 64;

template <int BITS>
struct StepWeights {
    uint32_t w[8][BITS];
};

/* LDS owned by one wave of a job: the partial transpose area, and the wave's
 * fold group of activation codes (already in block_dot operand order) and
 * block scales for each token of the unit. */
template <int TMAX>
struct WaveLds {
    int32_t part[TMAX * 512];
    uint32_t xa[TMAX][kMaxGroupBlocks][8];
    float d[TMAX][kMaxGroupBlocks];
};

/* Loads this lane's block of each of its octet's 8 rows for one K step.
 * The loads are unconditional: rows past rows_ok read the octet's first row
 * and a block past the group reads b_last (both in bounds; their partials
 * are never folded or stored), so no load sits under a branch and each use
 * waits only for its own step. */
template <int BITS>
__device__ __forceinline__ void load_step(StepWeights<BITS>& W, const uint8_t* row0, int64_t rowbytes,
                                          int b, int b_last, int rows_ok)
{
    const int bb = min(b, b_last);
#pragma unroll
    for (int rho = 0; rho < 8; ++rho)
        load_block<BITS>(row0 + (rho < rows_ok ? rho : 0) * rowbytes + (int64_t)bb * (4 * BITS), W.w[rho]);
}

/* Stages the codes and scales of blocks [b_begin, b_end) of every token into
 * the wave's LDS (one block per lane), once per job. */
template <int BITS, int TMAX>
__device__ __forceinline__ void stage_activations(WaveLds<TMAX>& L, int b_begin, int b_end, int ntok,
                                                  const int8_t* const (&act)[TMAX],
                                                  const float* const (&scl)[TMAX])
{
    const int lane = threadIdx.x & 63;
    const int b = b_begin + lane;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (t < ntok && b < b_end) {
            uint32_t x[8], xa[8];
            load_codes(act[t] + (int64_t)b * 32, x);
            prep_dot<BITS>(x, xa);
            uint4* dst = reinterpret_cast<uint4*>(L.xa[t][lane]);
            dst[0] = make_uint4(xa[0], xa[1], xa[2], xa[3]);
            dst[1] = make_uint4(xa[4], xa[5], xa[6], xa[7]);
            L.d[t][lane] = scl[t][b];
        }
    }
    wave_lds_sync();
}

/* One token's block of the wave's group, held in registers between its load
 * and its LDS commit (so other loads can be issued in between). */
struct TokenBlock {
    uint32_t x[8];
    float d;
};

__device__ __forceinline__ void load_token_block(TokenBlock& T, const int8_t* act, const float* scl,
                                                 int b_begin, int b_end)
{
    const int b = min(b_begin + (int)(threadIdx.x & 63), b_end - 1);
    load_codes(act + (int64_t)b * 32, T.x);
    T.d = scl[b];
}

template <int BITS>
__device__ __forceinline__ void commit_token_block(const TokenBlock& T, WaveLds<1>& L, int b_begin,
                                                   int b_end)
{
    const int lane = threadIdx.x & 63;
    if (b_begin + lane < b_end) {
        uint32_t xa[8];
        prep_dot<BITS>(T.x, xa);
        uint4* dst = reinterpret_cast<uint4*>(L.xa[0][lane]);
        dst[0] = make_uint4(xa[0], xa[1], xa[2], xa[3]);
        dst[1] = make_uint4(xa[4], xa[5], xa[6], xa[7]);
        L.d[0][lane] = T.d;
    }
    wave_lds_sync();
}

/* Block partials of K step st of the wave's group (nblk blocks from
 * b_begin), transposed through the wave's LDS, folded into acc (lane = row
 * 8o + j of the octet).  ws: the lane's row's group-wise scales (gb blocks
 * each), or null for per-row scales. */
template <int BITS, int TMAX>
__device__ __forceinline__ void fold_step(const StepWeights<BITS>& W, int st, int nblk, int ntok,
                                          WaveLds<TMAX>& L, float (&acc)[TMAX], const float* ws, int gb,
                                          int b_begin)
{
    const int lane = threadIdx.x & 63;
    const int o = lane >> 3, j8 = lane & 7;
    const int lb = 8 * st + j8;
    const bool valid = lb < nblk;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (t < ntok) {
            uint32_t xa[8];
            if (valid) {
                const uint4* src = reinterpret_cast<const uint4*>(L.xa[t][lb]);
                const uint4 u0 = src[0], u1 = src[1];
                xa[0] = u0.x; xa[1] = u0.y; xa[2] = u0.z; xa[3] = u0.w;
                xa[4] = u1.x; xa[5] = u1.y; xa[6] = u1.z; xa[7] = u1.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    xa[i] = 0;
            }
#pragma unroll
            for (int rho = 0; rho < 8; ++rho)
                L.part[part_index(t, o, rho, j8)] = block_dot<BITS>(W.w[rho], xa);
        }
    }
    wave_lds_sync();
    const int nbs = max(0, min(8, nblk - 8 * st));
    if (ws) {
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t < ntok) {
                for (int jj = 0; jj < nbs; ++jj)
                    acc[t] = __builtin_fmaf(group_coef(ws, gb, b_begin + 8 * st + jj, L.d[t][8 * st + jj]),
                                            (float)L.part[part_index(t, o, j8, jj)], acc[t]);
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t < ntok) {
                for (int jj = 0; jj < nbs; ++jj)
                    acc[t] = __builtin_fmaf(L.d[t][8 * st + jj], (float)L.part[part_index(t, o, j8, jj)], acc[t]);
            }
        }
    }
    wave_lds_sync();
}

/* Issues the weight loads of the first K step of a wave's fold group. */
template <int BITS>
__device__ __forceinline__ void first_step(StepWeights<BITS>& A, const uint8_t* row0, int64_t rowbytes,
                                           int b_begin, int b_end, int rows_ok)
{
    const int j8 = threadIdx.x & 7;
    load_step<BITS>(A, row0, rowbytes, b_begin + j8, max(b_end, b_begin + 1) - 1, rows_ok);
}

/* The K loop of one wave over its fold group, blocks [b_begin, b_end), in
 * steps of 8 blocks, the next step's weight loads issued before the current
 * step is computed; A holds the first step (first_step).  Waves of a
 * workgroup run their loops independently. */
template <int BITS, int TMAX>
__device__ __forceinline__ void k_loop(StepWeights<BITS>& A, const uint8_t* row0, int64_t rowbytes,
                                       int b_begin, int b_end, int ntok, int rows_ok, WaveLds<TMAX>& L,
                                       float (&acc)[TMAX], const float* ws, int gb)
{
    const int j8 = threadIdx.x & 7;
    const int nblk = b_end - b_begin;
    const int nsteps = (nblk + 7) / 8;
    const int b_last = max(b_end, b_begin + 1) - 1;
    StepWeights<BITS> B;
    /* loads and steps are unconditional (a step past the group folds
     * nothing), so A and B keep their registers across iterations */
    for (int st = 0; st < nsteps; st += 2) {
        load_step<BITS>(B, row0, rowbytes, b_begin + 8 * (st + 1) + j8, b_last, rows_ok);
        fold_step<BITS, TMAX>(A, st, nblk, ntok, L, acc, ws, gb, b_begin);
        load_step<BITS>(A, row0, rowbytes, b_begin + 8 * (st + 2) + j8, b_last, rows_ok);
        fold_step<BITS, TMAX>(B, st + 1, nblk, ntok, L, acc, ws, gb, b_begin);
    }
}

/* Adds the four group sums of each row in order; valid on wave 0 only. */
template <int TMAX>
__device__ __forceinline__ void sum_groups(float (*gsum)[TMAX][64], float (&acc)[TMAX])
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
        gsum[wv][t][lane] = acc[t];
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        float v = gsum[0][t][lane];
        v = v + gsum[1][t][lane];
        v = v + gsum[2][t][lane];
        v = v + gsum[3][t][lane];
        acc[t] = v;
    }
}

} // namespace

template <int BITS, int TMAX>
__global__ __launch_bounds__(256) void ffn_gate_up_gemv(FfnArgs a)
{
    __shared__ WaveLds<TMAX> lds[kGroups];
    __shared__ float gsum[kGroups][TMAX][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int o = lane >> 3;
    const int RB = a.I / 32;
    JobLoc L;
    if (!locate(a, blockIdx.x, RB, L))
        return;
    const FfnSeg sg = pick(a, L.seg);
    int e, pos0, ntok;
    if (!unit_info(sg, L.unit, e, pos0, ntok))
        return;
    ntok = min(ntok, TMAX);
    const int nb = a.H / 32;
    const int64_t rowbytes = (int64_t)a.H * BITS / 8;
    const int8_t* act[TMAX];
    const float* scl[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        const int tok = token_of(sg, pos0 + (t < ntok ? t : 0));
        act[t] = a.xq + (int64_t)tok * a.H;
        scl[t] = a.xd + (int64_t)tok * nb;
    }
    const int b0 = block_group(wv, nb), b1 = block_group(wv + 1, nb);
    /* octets 0..3: gate rows rb*32 + 8o ..; octets 4..7: the same up rows */
    const uint8_t* row0 = (o < 4 ? sg.gate_w : sg.up_w) +
                          ((int64_t)e * a.I + L.rb * 32 + 8 * (o & 3)) * rowbytes;
    /* group-wise scales of this lane's fold row (row 8(o & 3) + j of the job) */
    const int ng = sg.gu_gb ? nb / sg.gu_gb : 0;
    const float* ws = sg.gu_gb ? (o < 4 ? sg.gate_s : sg.up_s) +
                                     ((int64_t)e * a.I + L.rb * 32 + 8 * (o & 3) + (lane & 7)) * ng
                               : nullptr;
    StepWeights<BITS> A;
    first_step<BITS>(A, row0, rowbytes, b0, b1, 8);
    stage_activations<BITS, TMAX>(lds[wv], b0, b1, ntok, act, scl);
    float acc[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
        acc[t] = 0.0f;
    k_loop<BITS, TMAX>(A, row0, rowbytes, b0, b1, ntok, 8, lds[wv], acc, ws, sg.gu_gb);
    sum_groups<TMAX>(gsum, acc);
    if (wv != 0)
        return;

    const int r = L.rb * 32 + (lane & 31);
    const float sc = sg.gu_gb ? 1.0f : (lane < 32 ? sg.gate_s : sg.up_s)[(int64_t)e * a.I + r];
    const int nbi = a.I / 32;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
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

template <int BITS, int TMAX>
__global__ __launch_bounds__(256) void ffn_down_gemv(FfnArgs a)
{
    __shared__ WaveLds<TMAX> lds[kGroups];
    __shared__ float gsum[kGroups][TMAX][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int o = lane >> 3;
    const int RB = (a.H + kRowsPerJob - 1) / kRowsPerJob;
    JobLoc L;
    if (!locate(a, blockIdx.x, RB, L))
        return;
    const FfnSeg sg = pick(a, L.seg);
    int e, pos0, ntok;
    if (!unit_info(sg, L.unit, e, pos0, ntok))
        return;
    ntok = min(ntok, TMAX);
    const int nb = a.I / 32;
    const int64_t rowbytes = (int64_t)a.I * BITS / 8;
    const int8_t* act[TMAX];
    const float* scl[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        const int64_t row_in = sg.out_base + pos0 + (t < ntok ? t : 0);
        act[t] = a.hq + row_in * a.I;
        scl[t] = a.hd + row_in * nb;
    }
    const int b0 = block_group(wv, nb), b1 = block_group(wv + 1, nb);
    const int first = L.rb * kRowsPerJob + 8 * o;
    const int rows_ok = min(8, max(0, a.H - first));
    const uint8_t* row0 = sg.down_w + ((int64_t)e * a.H + min(first, a.H - 1)) * rowbytes;
    const int ng = sg.d_gb ? nb / sg.d_gb : 0;
    const float* ws = sg.d_gb ? sg.down_s + ((int64_t)e * a.H + min(first + (lane & 7), a.H - 1)) * ng : nullptr;
    StepWeights<BITS> A;
    first_step<BITS>(A, row0, rowbytes, b0, b1, rows_ok);
    stage_activations<BITS, TMAX>(lds[wv], b0, b1, ntok, act, scl);
    float acc[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
        acc[t] = 0.0f;
    k_loop<BITS, TMAX>(A, row0, rowbytes, b0, b1, ntok, rows_ok, lds[wv], acc, ws, sg.d_gb);
    sum_groups<TMAX>(gsum, acc);
    if (wv != 0)
        return;

    const int n = L.rb * kRowsPerJob + lane;
    if (n < a.H) {
        const float sc = sg.d_gb ? 1.0f : sg.down_s[(int64_t)e * a.H + n];
#pragma unroll
        for (int t = 0; t < TMAX; ++t)
            if (t < ntok)
                a.y[(int64_t)(sg.out_base + pos0 + t) * a.H + n] = sc * acc[t];
    }
}

/* ---- one-token batches ---------------------------------------------------
 * Unit u < k is the expert of selection slot u, unit k the shared expert;
 * hq / hd / y row u belongs to unit u, so the combine reads y in slot order.
 * The gate/up kernel selects the experts itself: wave 0 of every routed job
 * runs the top-k over the token's logits (the same selection as
 * router_select_kernel), so no workgroup waits for another, and the first
 * routed job stores ids and weights.
 *
 * Whole-row loads.  A job is 64 rows; wave w owns rows 16w .. 16w+15 and
 * reads them whole, two rows per load instruction: lane l takes row
 * 2p + (l >> 5) of pair p and blocks (l & 31) + 32 i, i < NI, so each half
 * wave reads 32 consecutive blocks of one row (512 bytes at int4).  Reading
 * each row in one sweep streams markedly faster than splitting K across the
 * waves (measured 6.5 vs 5.5 TB/s on 113 MB).  A lane's activation blocks are
 * the same for every row, so they stay in registers.  The exact partials of
 * the 16 rows go to LDS; lane (r, g) then folds row r's group g in ascending
 * block order and the four group sums are added in order.
 *
 * (A combine inside the down kernel -- the last unit to finish a row block
 * adding the others' rows -- needs a device-scope release per workgroup,
 * which on this chip writes back the XCD's L2; measured 3x slower than the
 * separate combine launch.) */

constexpr int kDecRows = 16; /* rows of a job per wave */

/* Load instructions per row pair for nb blocks, rounded up to an
 * instantiated count. */
inline int dec_ni(int nb)
{
    const int n = (nb + 31) / 32;
    return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : n <= 6 ? 6 : 8;
}

/* Dynamic LDS, in words: per wave the partials [16][nb | 1] (before the K
 * loop wave 0's selection scratch), then the token's block scales [nb], the
 * job's row sums [64] and the selected ids [64]. */
__host__ __device__ inline int dec_region(int nb)
{
    const int p = kDecRows * (nb | 1);
    return p > kSelScratch ? p : kSelScratch;
}

__host__ __device__ inline size_t dec_lds_bytes(int nb)
{
    return (size_t)(kGroups * dec_region(nb) + nb + 64 + 64) * 4;
}

template <int BITS, int NI>
struct PairLoad {
    uint32_t w[NI][BITS];
};

/* Loads are unconditional: a lane past the job's rows or the row's blocks
 * reads the last row / block instead (in bounds; its partial is never used),
 * so no load sits under a branch and each use waits only for its own loads. */
template <int BITS, int NI>
__device__ __forceinline__ void pair_load(PairLoad<BITS, NI>& L, const uint8_t* rows0, int64_t rowbytes,
                                          int p, int rows_ok, int nb, const uint8_t* rows8 = nullptr)
{
    const int lane = threadIdx.x & 63;
    const int row = min(2 * p + (lane >> 5), max(rows_ok, 1) - 1), c = lane & 31;
    /* rows8: where rows 8.. start, when not right after row 7 */
    const uint8_t* rp = (rows8 && row >= 8) ? rows8 + (int64_t)(row - 8) * rowbytes : rows0 + (int64_t)row * rowbytes;
#pragma unroll
    for (int i = 0; i < NI; ++i)
        load_block<BITS>(rp + (int64_t)min(c + 32 * i, nb - 1) * (4 * BITS), L.w[i]);
}

template <int BITS, int NI>
__device__ __forceinline__ void pair_partials(const PairLoad<BITS, NI>& L, const uint32_t (&xa)[NI][8], int p,
                                              int nb, int32_t* P, int sp)
{
    const int lane = threadIdx.x & 63;
    const int row = 2 * p + (lane >> 5), c = lane & 31;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int b = c + 32 * i;
        if (row < kDecRows && b < nb)
            P[row * sp + b] = block_dot<BITS>(L.w[i], xa[i]);
    }
}

/* The wave's 16 rows (rows0: its first row; rows_ok of them exist): returns
 * on every lane the folded sum of row (lane & 15) before the row scale.
 * The caller has issued pair 0 into A (so the weight stream starts before
 * the activations are prepared); two pairs are in flight while one is
 * multiplied. */
template <int BITS, int NI>
__device__ __forceinline__ float dec_k_loop(PairLoad<BITS, NI>& A, const uint8_t* rows0, int64_t rowbytes,
                                            int rows_ok, int nb, const uint32_t (&xa)[NI][8], int32_t* P,
                                            int sp, const float* dl, const float* ws0, int gb,
                                            const uint8_t* rows8 = nullptr)
{
    PairLoad<BITS, NI> B;
#pragma unroll
    for (int p = 0; p < kDecRows / 2; p += 2) {
        pair_load<BITS, NI>(B, rows0, rowbytes, p + 1, rows_ok, nb, rows8);
        pair_partials<BITS, NI>(A, xa, p, nb, P, sp);
        if (p + 2 < kDecRows / 2) /* resolved at compile time */
            pair_load<BITS, NI>(A, rows0, rowbytes, p + 2, rows_ok, nb, rows8);
        pair_partials<BITS, NI>(B, xa, p + 1, nb, P, sp);
    }
    wave_lds_sync();
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int b0 = block_group(g, nb), b1 = block_group(g + 1, nb);
    const int32_t* pr = P + r * sp;
    float acc = 0.0f;
    int b = b0;
    if (ws0) {
        /* group-wise scales of row r (rows past rows_ok read the last row's) */
        const float* ws = ws0 + (int64_t)min(r, max(rows_ok, 1) - 1) * (nb / gb);
        for (; b < b1; ++b)
            acc = __builtin_fmaf(group_coef(ws, gb, b, dl[b]), (float)pr[b], acc);
    } else {
        /* eight partials and scales read ahead of their (in-order) fmas */
        for (; b + 8 <= b1; b += 8) {
            int32_t q[8];
            float dd[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                q[i] = pr[b + i];
                dd[i] = dl[b + i];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc = __builtin_fmaf(dd[i], (float)q[i], acc);
        }
        for (; b < b1; ++b)
            acc = __builtin_fmaf(dl[b], (float)pr[b], acc);
    }
    float v = __shfl(acc, r, kWave);
    v = v + __shfl(acc, 16 + r, kWave);
    v = v + __shfl(acc, 32 + r, kWave);
    v = v + __shfl(acc, 48 + r, kWave);
    return v;
}

/* The token's activation blocks (l & 31) + 32 i, loaded raw ... */
template <int NI>
__device__ __forceinline__ void dec_act_load(const int8_t* act, int nb, uint32_t (&x)[NI][8])
{
    const int c = threadIdx.x & 31;
#pragma unroll
    for (int i = 0; i < NI; ++i)
        load_codes(act + (int64_t)min(c + 32 * i, nb - 1) * 32, x[i]);
}

/* The block scales b = lane + 64 i, i < kDlPre, loaded with the codes (so
 * that their latency is spent before the weight stream starts) ... */
constexpr int kDlPre = 4;

__device__ __forceinline__ void dec_scale_load(const float* scl, int nb, float (&pre)[kDlPre])
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kDlPre; ++i)
        pre[i] = scl[min(lane + 64 * i, nb - 1)];
}

/* ... then the codes put in operand order; every wave also writes the block
 * scales (the same values) so that its own reads follow its own writes. */
template <int BITS, int NI>
__device__ __forceinline__ void dec_act_prep(uint32_t (&x)[NI][8], const float (&pre)[kDlPre], const float* scl,
                                             int nb, float* dl)
{
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        uint32_t xa[8];
        prep_dot<BITS>(x[i], xa);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            x[i][q] = xa[q];
    }
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < kDlPre; ++i)
        if (lane + 64 * i < nb)
            dl[lane + 64 * i] = pre[i];
    for (int b = lane + 64 * kDlPre; b < nb; b += 64)
        dl[b] = scl[b];
    wave_lds_sync();
}

template <int BITS, int NI>
__global__ __launch_bounds__(256) void ffn_gate_up_decode(DecodeArgs d)
{
    extern __shared__ __attribute__((aligned(16))) int32_t dec_lds[];
    const FfnArgs& a = d.f;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int RB = a.I / 32;
    const int nb = a.H / 32, sp = nb | 1, region = dec_region(nb);
    int32_t* P = dec_lds + wv * region;
    float* dl = reinterpret_cast<float*>(dec_lds + kGroups * region);
    float* rsum = dl + nb;
    int32_t* sel_ids = reinterpret_cast<int32_t*>(rsum + 64); /* read by every wave after the barrier */
    const int64_t rowbytes = (int64_t)a.H * BITS / 8;
    const int n_mini = d.hs ? a.I / 8 : 0;
    if ((int)blockIdx.x < n_mini) {
        /* one-wave job of the shared expert (first, so that every CU gets
         * one before any routed job, and it streams during the selection):
         * gate rows 8m .. 8m+7 as rows 0..7 and the same up rows as rows
         * 8..15; h of its 8 rows in fp32 */
        if (wv != 0)
            return;
        const FfnSeg sh = pick(a, 1);
        const int m = blockIdx.x;
        const uint8_t* g0 = sh.gate_w + (int64_t)8 * m * rowbytes;
        const uint8_t* u0 = sh.up_w + (int64_t)8 * m * rowbytes;
        PairLoad<BITS, NI> A;
        pair_load<BITS, NI>(A, g0, rowbytes, 0, kDecRows, nb, u0);
        uint32_t xa[NI][8];
        dec_act_load<NI>(a.xq, nb, xa);
        float dpre[kDlPre];
        dec_scale_load(a.xd, nb, dpre);
        const int r = lane & 15;
        const float sc = (r < 8 ? sh.gate_s : sh.up_s)[8 * m + (r & 7)];
        dec_act_prep<BITS, NI>(xa, dpre, a.xd, nb, dl);
        const float v16 = dec_k_loop<BITS, NI>(A, g0, rowbytes, kDecRows, nb, xa, P, sp, dl, nullptr, 0, u0);
        const float v = sc * v16;
        const float up = __shfl(v, (lane & 7) + 8, kWave);
        if (lane < 8)
            d.hs[8 * m + lane] = canon_silu(v) * up;
        return;
    }
    const int nunits = d.k + (a.nseg > 1 && !d.hs ? 1 : 0);
    /* the shared expert's jobs come first: they need no selection, so they
     * stream while the routed jobs select, and they land first on the CUs
     * that also receive a third job */
    const int jb = blockIdx.x - n_mini;
    const int j = jb / RB, rb = jb - (jb / RB) * RB;
    if (j >= nunits)
        return;
    const int u = nunits > d.k ? (j == 0 ? d.k : j - 1) : j;
    const bool routed = u < d.k;
    const FfnSeg sg = pick(a, routed ? 0 : 1);
    uint32_t xa[NI][8];
    dec_act_load<NI>(a.xq, nb, xa);
    float dpre[kDlPre];
    dec_scale_load(a.xd, nb, dpre);
    int e = 0;
    bool prepped = false;
    if (routed) {
        /* wave 0 alone selects (a chain of wave-wide steps, so it runs best
         * without the other waves issuing the same work) while waves 1..3
         * prepare their activations; the scratch is wave 0's (not yet used)
         * partial buffer */
        float* sel_s = reinterpret_cast<float*>(dec_lds);
        if (wv == 0) {
            const bool store = u == 0 && rb == 0; /* the others need the ids only */
            select_token(d.logits, d.bias, d.E, d.k, d.rsf, store ? d.ids : sel_ids, store ? d.w : nullptr, sel_s,
                         sel_ids, 1, 0, d.opt);
        } else {
            dec_act_prep<BITS, NI>(xa, dpre, a.xd, nb, dl);
            prepped = true;
        }
        __syncthreads();
        const int sel = sel_ids[u];
        if (sel < 0) /* slot dropped by top-p: the whole workgroup leaves */
            return;
        e = min(sel, sg.n_mat - 1);
    }
    /* waves 0, 1: gate rows rb*32 + 16w ..; waves 2, 3: the same up rows */
    const uint8_t* rows0 = (wv < 2 ? sg.gate_w : sg.up_w) +
                           ((int64_t)e * a.I + rb * 32 + 16 * (wv & 1)) * rowbytes;
    PairLoad<BITS, NI> A;
    pair_load<BITS, NI>(A, rows0, rowbytes, 0, kDecRows, nb);
    /* the epilogue's row scale (lane: row rb*32 + lane%32 of gate, then up),
     * loaded now so that it is in hand after the K loop */
    const int r = rb * 32 + (lane & 31);
    const float sc = sg.gu_gb ? 1.0f : (lane < 32 ? sg.gate_s : sg.up_s)[(int64_t)e * a.I + r];
    if (!prepped)
        dec_act_prep<BITS, NI>(xa, dpre, a.xd, nb, dl);
    const float* ws0 = sg.gu_gb ? (wv < 2 ? sg.gate_s : sg.up_s) +
                                      ((int64_t)e * a.I + rb * 32 + 16 * (wv & 1)) * (nb / sg.gu_gb)
                                : nullptr;
    const float v16 = dec_k_loop<BITS, NI>(A, rows0, rowbytes, kDecRows, nb, xa, P, sp, dl, ws0, sg.gu_gb);
    if (lane < 16)
        rsum[16 * wv + lane] = v16;
    __syncthreads();
    if (wv != 0)
        return;
    const float acc = rsum[lane];
    const float v = sc * acc;
    const float up = shfl_xor(v, 32);
    const float h = canon_silu(v) * up;
    float am = lane < 32 ? __builtin_fabsf(h) : 0.0f;
    for (int m = 16; m >= 1; m >>= 1)
        am = fmaxf(am, shfl_xor(am, m));
    const float dsc = am / 127.0f;
    const float inv = (am == 0.0f) ? 0.0f : 1.0f / dsc;
    if (lane < 32)
        a.hq[(int64_t)u * a.I + r] = (int8_t)q8_code(h, inv);
    if (lane == 0)
        a.hd[(int64_t)u * (a.I / 32) + rb] = dsc;
}

template <int BITS, int NI>
__global__ __launch_bounds__(256) void ffn_down_decode(DecodeArgs d)
{
    extern __shared__ __attribute__((aligned(16))) int32_t dec_lds[];
    const FfnArgs& a = d.f;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int RB = (a.H + kRowsPerJob - 1) / kRowsPerJob;
    const int nunits = d.k + (a.nseg > 1 ? 1 : 0);
    const int u = blockIdx.x / RB, rb = blockIdx.x - (blockIdx.x / RB) * RB;
    if (u >= nunits)
        return;
    const bool routed = u < d.k;
    if (routed && d.ids[u] < 0) /* slot dropped by top-p */
        return;
    const FfnSeg sg = pick(a, routed ? 0 : 1);
    const int e = routed ? min(d.ids[u], sg.n_mat - 1) : 0;
    const int nb = a.I / 32, sp = nb | 1, region = dec_region(nb);
    int32_t* P = dec_lds + wv * region;
    float* dl = reinterpret_cast<float*>(dec_lds + kGroups * region);
    uint32_t xa[NI][8];
    dec_act_load<NI>(a.hq + (int64_t)u * a.I, nb, xa);
    float dpre[kDlPre];
    dec_scale_load(a.hd + (int64_t)u * nb, nb, dpre);
    const int row0 = rb * kRowsPerJob + kDecRows * wv;
    const int rows_ok = min(kDecRows, max(0, a.H - row0));
    const int64_t rowbytes = (int64_t)a.I * BITS / 8;
    const uint8_t* rows0 = sg.down_w + ((int64_t)e * a.H + min(row0, a.H - 1)) * rowbytes;
    PairLoad<BITS, NI> A;
    pair_load<BITS, NI>(A, rows0, rowbytes, 0, rows_ok, nb);
    dec_act_prep<BITS, NI>(xa, dpre, a.hd + (int64_t)u * nb, nb, dl);
    const float* ws0 = sg.d_gb ? sg.down_s + ((int64_t)e * a.H + min(row0, a.H - 1)) * (nb / sg.d_gb) : nullptr;
    const float v = dec_k_loop<BITS, NI>(A, rows0, rowbytes, rows_ok, nb, xa, P, sp, dl, ws0, sg.d_gb);
    const int n = row0 + lane;
    if (lane < rows_ok)
        a.y[(int64_t)u * a.H + n] = (sg.d_gb ? 1.0f : sg.down_s[(int64_t)e * a.H + n]) * v;
}

/* Items a thread stages per round (loads of all issued before any is converted). */
constexpr int kDcStage = 4;

/* ---- whole rows for units of up to kUnitTokens tokens --------------------
 *
 * The job of ffn_gate_up_gemv / ffn_down_gemv (one unit, 64 row dots), with
 * the whole-row streaming of the one-token kernels: wave w owns 16 whole rows
 * and reads two rows per load group (lane l: row 2p + l/32, blocks
 * l mod 32 + 32 i), two pairs in flight.  The unit's activation blocks of
 * every token are staged once per job in LDS in operand order; after each
 * pair the wave writes the exact partials of its 2 rows x the unit's tokens
 * and folds them -- lane (row, token, group) runs the canonical chain of its
 * group, the four group sums added in order -- while the next two pairs
 * load.
 *
 * Dynamic LDS, in words: codes [TMAX][nb][8], block scales [TMAX][nb | 1],
 * per wave the partials [2][TMAX][nb | 1], and the job's row values
 * [64][TMAX]; used while it fits 64 KB. */
__host__ __device__ inline size_t rows_lds_words(int nb, int tmax)
{
    const size_t sp = (size_t)(nb | 1);
    return (size_t)tmax * nb * 8 + (size_t)tmax * sp + (size_t)kGroups * 2 * tmax * sp + 64 * (size_t)tmax;
}

inline bool rows_fit(int nb, int tmax)
{
    return nb <= 32 * 8 && rows_lds_words(nb, tmax) * 4 <= 64 * 1024;
}

/* Exact partials of one loaded pair (rows 0, 1) for every token of the
 * unit, to P[(row * TMAX + t) * sp + b]. */
template <int BITS, int NI, int TMAX>
__device__ __forceinline__ void rows_partials(const PairLoad<BITS, NI>& L, const uint32_t* xal, int nb, int ntok,
                                              int32_t* P, int sp)
{
    const int lane = threadIdx.x & 63, c = lane & 31, row = lane >> 5;
    /* tokens one at a time (a rolled loop keeps one token's operands live) */
#pragma unroll 1
    for (int t = 0; t < ntok; ++t) {
        {
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int b = c + 32 * i;
                if (b < nb) {
                    const uint4* src = reinterpret_cast<const uint4*>(xal + ((int64_t)t * nb + b) * 8);
                    const uint4 u0 = src[0], u1 = src[1];
                    const uint32_t xa[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
                    P[(row * TMAX + t) * sp + b] = block_dot<BITS>(L.w[i], xa);
                }
            }
        }
    }
}

/* The canonical fold of the pair's 2 rows (rows rbase, rbase + 1 of the
 * job): lane (r2, t, g) folds group g of row r2 for token t, then the group
 * sums of (r2, t) are added in order into vs[row][t].  ws0: group-wise scales
 * of the pair's first row (gb blocks per scale, rows ng apart), or null;
 * a row past rows_left (not stored) reads the last existing row's. */
template <int TMAX>
__device__ __forceinline__ void rows_fold(const int32_t* P, int sp, int nb, int ntok, const float* dls,
                                          const float* ws0, int gb, int ng, int rows_left, float* vs, int rbase)
{
    const int lane = threadIdx.x & 63;
    const int g = lane & 3, t = (lane >> 2) % TMAX, r4 = (lane >> 2) / TMAX;
    const int rr = min(r4, 1);
    const int b0 = block_group(g, nb), b1 = block_group(g + 1, nb);
    const int32_t* pr = P + (rr * TMAX + t) * sp;
    const float* dj = dls + t * sp;
    float acc = 0.0f;
    int b = b0;
    if (ws0) {
        const float* ws = ws0 + (int64_t)min(rr, max(rows_left, 1) - 1) * ng;
        for (; b < b1; ++b)
            acc = __builtin_fmaf(group_coef(ws, gb, b, dj[b]), (float)pr[b], acc);
    } else {
        for (; b + 8 <= b1; b += 8) {
            int32_t q[8];
            float dd[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                q[i] = pr[b + i];
                dd[i] = dj[b + i];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc = __builtin_fmaf(dd[i], (float)q[i], acc);
        }
        for (; b < b1; ++b)
            acc = __builtin_fmaf(dj[b], (float)pr[b], acc);
    }
    const int base = lane & ~3;
    float v = __shfl(acc, base, kWave);
    v = v + __shfl(acc, base + 1, kWave);
    v = v + __shfl(acc, base + 2, kWave);
    v = v + __shfl(acc, base + 3, kWave);
    if (g == 0 && r4 < 2 && t < ntok)
        vs[(rbase + r4) * TMAX + t] = v;
}

/* Stages the codes (operand order) and block scales of the unit's tokens;
 * every thread issues up to kDcStage items' loads before converting any. */
template <int BITS, int TMAX>
__device__ __forceinline__ void rows_stage(uint32_t* xal, float* dls, int nb, int sp, int ntok,
                                           const int8_t* const (&act)[TMAX], const float* const (&scl)[TMAX])
{
    const int n_items = ntok * nb;
    for (int i0 = threadIdx.x; i0 < n_items; i0 += 64 * kGroups * kDcStage) {
        uint32_t x[kDcStage][8];
        float dv[kDcStage];
#pragma unroll
        for (int r = 0; r < kDcStage; ++r) {
            const int i = i0 + r * 64 * kGroups;
            if (i < n_items) {
                const int t = i / nb, b = i - t * nb;
                const int8_t* ap = act[0];
                const float* sp0 = scl[0];
#pragma unroll
                for (int tt = 1; tt < TMAX; ++tt)
                    if (t == tt) {
                        ap = act[tt];
                        sp0 = scl[tt];
                    }
                load_codes(ap + (int64_t)b * 32, x[r]);
                dv[r] = sp0[b];
            }
        }
#pragma unroll
        for (int r = 0; r < kDcStage; ++r) {
            const int i = i0 + r * 64 * kGroups;
            if (i < n_items) {
                const int t = i / nb, b = i - t * nb;
                uint32_t xa[8];
                prep_dot<BITS>(x[r], xa);
                uint4* dst = reinterpret_cast<uint4*>(xal + (int64_t)i * 8);
                dst[0] = make_uint4(xa[0], xa[1], xa[2], xa[3]);
                dst[1] = make_uint4(xa[4], xa[5], xa[6], xa[7]);
                dls[t * sp + b] = dv[r];
            }
        }
    }
    __syncthreads();
}

/* Partials and fold of pair p (in L) into vs[rbase0 + 2p ..]. */
template <int BITS, int NI, int TMAX>
__device__ __forceinline__ void rows_pair(const PairLoad<BITS, NI>& L, int p, int rows_ok, int nb, int sp,
                                          int ntok, const uint32_t* xal, const float* dls, int32_t* P,
                                          const float* ws0, int gb, int ng, float* vs, int rbase0)
{
    rows_partials<BITS, NI, TMAX>(L, xal, nb, ntok, P, sp);
    wave_lds_sync();
    const int r_first = min(2 * p, max(rows_ok, 1) - 1);
    rows_fold<TMAX>(P, sp, nb, ntok, dls, ws0 ? ws0 + (int64_t)r_first * ng : nullptr, gb, ng, rows_ok - 2 * p,
                    vs, rbase0 + 2 * p);
    wave_lds_sync(); /* the pair's partials are read before the next overwrites them */
}

/* The wave's 16 rows (rows0: its first row, rows_ok of them exist), pair 0
 * already in A; two pairs in flight while one is multiplied and folded. */
template <int BITS, int NI, int TMAX>
__device__ __forceinline__ void rows_k_loop(PairLoad<BITS, NI>& A, const uint8_t* rows0, int64_t rowbytes,
                                            int rows_ok, int nb, int sp, int ntok, const uint32_t* xal,
                                            const float* dls, int32_t* P, const float* ws0, int gb, int ng,
                                            float* vs, int rbase0)
{
    PairLoad<BITS, NI> B;
    pair_load<BITS, NI>(B, rows0, rowbytes, 1, rows_ok, nb);
#pragma unroll
    for (int p = 0; p < kDecRows / 2; p += 2) {
        if (p + 2 < kDecRows / 2) { /* resolved at compile time */
            rows_pair<BITS, NI, TMAX>(A, p, rows_ok, nb, sp, ntok, xal, dls, P, ws0, gb, ng, vs, rbase0);
            pair_load<BITS, NI>(A, rows0, rowbytes, p + 2, rows_ok, nb);
            rows_pair<BITS, NI, TMAX>(B, p + 1, rows_ok, nb, sp, ntok, xal, dls, P, ws0, gb, ng, vs, rbase0);
            pair_load<BITS, NI>(B, rows0, rowbytes, p + 3, rows_ok, nb);
        } else {
            rows_pair<BITS, NI, TMAX>(A, p, rows_ok, nb, sp, ntok, xal, dls, P, ws0, gb, ng, vs, rbase0);
            rows_pair<BITS, NI, TMAX>(B, p + 1, rows_ok, nb, sp, ntok, xal, dls, P, ws0, gb, ng, vs, rbase0);
        }
    }
}

template <int BITS, int NI, int TMAX>
__global__ __launch_bounds__(256) void ffn_gate_up_rows(FfnArgs a)
{
    extern __shared__ __attribute__((aligned(16))) int32_t rw_lds[];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int RB = a.I / 32;
    JobLoc L;
    if (!locate(a, blockIdx.x, RB, L))
        return;
    const FfnSeg sg = pick(a, L.seg);
    int e, pos0, ntok;
    if (!unit_info(sg, L.unit, e, pos0, ntok))
        return;
    ntok = min(ntok, TMAX);
    const int nb = a.H / 32, sp = nb | 1;
    const int64_t rowbytes = (int64_t)a.H * BITS / 8;
    uint32_t* xal = reinterpret_cast<uint32_t*>(rw_lds);
    float* dls = reinterpret_cast<float*>(xal + (int64_t)TMAX * nb * 8);
    int32_t* P = reinterpret_cast<int32_t*>(dls + TMAX * sp) + wv * (2 * TMAX * sp);
    float* vs = reinterpret_cast<float*>(reinterpret_cast<int32_t*>(dls + TMAX * sp) + kGroups * 2 * TMAX * sp);
    /* waves 0, 1: gate rows rb*32 + 16w ..; waves 2, 3: the same up rows */
    const int rloc = 16 * (wv & 1);
    const uint8_t* rows0 = (wv < 2 ? sg.gate_w : sg.up_w) + ((int64_t)e * a.I + L.rb * 32 + rloc) * rowbytes;
    PairLoad<BITS, NI> A;
    pair_load<BITS, NI>(A, rows0, rowbytes, 0, kDecRows, nb);
    const int r = L.rb * 32 + (lane & 31);
    const float sc = sg.gu_gb ? 1.0f : (lane < 32 ? sg.gate_s : sg.up_s)[(int64_t)e * a.I + r];
    const int8_t* act[TMAX];
    const float* scl[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        const int tok = token_of(sg, pos0 + (t < ntok ? t : 0));
        act[t] = a.xq + (int64_t)tok * a.H;
        scl[t] = a.xd + (int64_t)tok * nb;
    }
    rows_stage<BITS, TMAX>(xal, dls, nb, sp, ntok, act, scl);
    const int ng = sg.gu_gb ? nb / sg.gu_gb : 0;
    const float* ws0 = sg.gu_gb ? (wv < 2 ? sg.gate_s : sg.up_s) + ((int64_t)e * a.I + L.rb * 32 + rloc) * ng
                                : nullptr;
    /* job row of the wave's first row: gate rows 0..31, up rows 32..63 */
    rows_k_loop<BITS, NI, TMAX>(A, rows0, rowbytes, kDecRows, nb, sp, ntok, xal, dls, P, ws0, sg.gu_gb, ng, vs,
                                16 * wv);
    __syncthreads();
    if (wv != 0)
        return;
    const int nbi = a.I / 32;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (t < ntok) {
            const float v = sc * vs[lane * TMAX + t];
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

template <int BITS, int NI, int TMAX>
__global__ __launch_bounds__(256) void ffn_down_rows(FfnArgs a)
{
    extern __shared__ __attribute__((aligned(16))) int32_t rw_lds[];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int RB = (a.H + kRowsPerJob - 1) / kRowsPerJob;
    JobLoc L;
    if (!locate(a, blockIdx.x, RB, L))
        return;
    const FfnSeg sg = pick(a, L.seg);
    int e, pos0, ntok;
    if (!unit_info(sg, L.unit, e, pos0, ntok))
        return;
    ntok = min(ntok, TMAX);
    const int nb = a.I / 32, sp = nb | 1;
    const int64_t rowbytes = (int64_t)a.I * BITS / 8;
    uint32_t* xal = reinterpret_cast<uint32_t*>(rw_lds);
    float* dls = reinterpret_cast<float*>(xal + (int64_t)TMAX * nb * 8);
    int32_t* P = reinterpret_cast<int32_t*>(dls + TMAX * sp) + wv * (2 * TMAX * sp);
    float* vs = reinterpret_cast<float*>(reinterpret_cast<int32_t*>(dls + TMAX * sp) + kGroups * 2 * TMAX * sp);
    const int first = L.rb * kRowsPerJob + kDecRows * wv;
    const int rows_ok = min(kDecRows, max(0, a.H - first));
    const uint8_t* rows0 = sg.down_w + ((int64_t)e * a.H + min(first, a.H - 1)) * rowbytes;
    PairLoad<BITS, NI> A;
    pair_load<BITS, NI>(A, rows0, rowbytes, 0, rows_ok, nb);
    const int n = first + (lane & 15);
    const float sc = sg.d_gb ? 1.0f : sg.down_s[(int64_t)e * a.H + min(n, a.H - 1)];
    const int8_t* act[TMAX];
    const float* scl[TMAX];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        const int64_t row_in = sg.out_base + pos0 + (t < ntok ? t : 0);
        act[t] = a.hq + row_in * a.I;
        scl[t] = a.hd + row_in * nb;
    }
    rows_stage<BITS, TMAX>(xal, dls, nb, sp, ntok, act, scl);
    const int ng = sg.d_gb ? nb / sg.d_gb : 0;
    const float* ws0 = sg.d_gb ? sg.down_s + ((int64_t)e * a.H + min(first, a.H - 1)) * ng : nullptr;
    rows_k_loop<BITS, NI, TMAX>(A, rows0, rowbytes, rows_ok, nb, sp, ntok, xal, dls, P, ws0, sg.d_gb, ng, vs,
                                16 * wv);
    wave_lds_sync();
    /* lane (row l % 16): its row's value of every token */
    if (lane < 16 && n < a.H) {
#pragma unroll
        for (int t = 0; t < TMAX; ++t)
            if (t < ntok)
                a.y[(int64_t)(sg.out_base + pos0 + t) * a.H + n] = sc * vs[(16 * wv + lane) * TMAX + t];
    }
}

/* ---- one token: down projection with the combine --------------------------
 * A workgroup owns 8 output rows for all U = k (+1 shared) units; wave w
 * streams rows 2w, 2w+1 of every unit's down matrix as whole-row pairs
 * (pair j = unit j), two units in flight.  All units' h codes are staged in
 * LDS in operand order once per workgroup (measured faster than each lane
 * loading its own h blocks per unit, and than four units in flight).  After
 * the canonical fold of each (unit, row), the wave forms
 * out = y_shared + sum_j w_j * y_j for its rows with the same fma order as
 * combine_kernel, so the result is bit-identical to down + combine without
 * the y round trip or the extra launch.  (8 rows per workgroup give H / 8 =
 * 768 workgroups at H = 6144: three per CU.) */

/* A workgroup of DW waves owns 2 DW output rows (wave w: rows 2w, 2w+1).
 * kDcWide waves (one workgroup per CU at H = 6144) stage every unit's h once
 * per CU; the vector L1, whose lines bound this kernel, then spends a
 * twelfth as many lines on h as with three 4-wave workgroups per CU. */
constexpr int kDcWide = 12;

/* LDS words: h codes [U][nb][8], h scales [U][nb | 1], per wave the partials
 * [2U][nb | 1] and the row values [2U]. */
__host__ __device__ inline size_t dc_lds_words(int U, int nb, int DW)
{
    return (size_t)U * nb * 8 + (size_t)U * (nb | 1) + (size_t)DW * 2 * U * ((nb | 1) + 1);
}

constexpr size_t kDcLdsMax = 160 * 1024; /* LDS of one CU (gfx950) */

/* First of this wave's two rows of the down matrix of unit u (u = slot, or
 * k for the shared expert) whose matrix index is e. */
__device__ __forceinline__ const uint8_t* dc_rows(const DecodeArgs& d, int u, int e, int row0, int64_t rowbytes)
{
    const FfnArgs& a = d.f;
    const uint8_t* w = u < d.k ? a.seg[0].down_w : a.seg[1].down_w;
    return w + ((int64_t)e * a.H + row0) * rowbytes;
}

template <int NI>
__device__ __forceinline__ void dc_act(const uint32_t* xal, int j, int nb, uint32_t (&xa)[NI][8])
{
    const int c = threadIdx.x & 31;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const uint4* src = reinterpret_cast<const uint4*>(xal + ((int64_t)j * nb + min(c + 32 * i, nb - 1)) * 8);
        const uint4 u0 = src[0], u1 = src[1];
        xa[i][0] = u0.x; xa[i][1] = u0.y; xa[i][2] = u0.z; xa[i][3] = u0.w;
        xa[i][4] = u1.x; xa[i][5] = u1.y; xa[i][6] = u1.z; xa[i][7] = u1.w;
    }
}

/* Unit of compacted index n: the n-th kept routed slot (bit set in `kept`),
 * then the shared expert (index k).  Without top-p every slot is kept and
 * the index is the slot. */
__device__ __forceinline__ int dc_unit(uint64_t kept, int n_kept, int k, int n, bool all_kept)
{
    if (n >= n_kept)
        return k;
    if (all_kept)
        return n;
    for (int i = 0; i < n; ++i)
        kept &= kept - 1;
    return __builtin_ctzll(kept);
}

template <int BITS, int NI, int DW>
__global__ __launch_bounds__(64 * DW) void ffn_down_combine_decode(DecodeArgs d)
{
    extern __shared__ int32_t dc_lds[];
    const FfnArgs& a = d.f;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const bool shared = a.nseg > 1;
    /* slots dropped by top-p are neither streamed nor combined: the units are
     * the kept routed slots in slot order, then the shared expert */
    const bool all_kept = !(d.opt.top_p > 0.0f && d.opt.top_p < 1.0f);
    const uint64_t kept = all_kept ? 0 : __ballot(lane < d.k && d.ids[lane] >= 0);
    const int n_kept = all_kept ? d.k : __popcll(kept);
    const int U = n_kept + (shared ? 1 : 0);
    const int nb = a.I / 32, sp = nb | 1;
    uint32_t* xal = reinterpret_cast<uint32_t*>(dc_lds);        /* [U][nb][8] */
    /* the block scales' rows have the odd stride sp, like the partials', so
     * that the fold's reads (32 distinct addresses) spread over the banks */
    float* dls = reinterpret_cast<float*>(xal + U * nb * 8);    /* [U][sp] */
    int32_t* P0 = reinterpret_cast<int32_t*>(dls + U * sp);      /* [DW][2U][sp] */
    int32_t* P = P0 + wv * (2 * U * sp);
    float* ys = reinterpret_cast<float*>(P0 + DW * 2 * U * sp) + wv * 2 * U;
    const int row0 = blockIdx.x * (2 * DW) + 2 * wv;
    const int64_t rowbytes = (int64_t)a.I * BITS / 8;

    if (U == 0)
        return;
    /* stream order: the shared expert first (its rows need no id, so its
     * first pair is issued before the ids arrive), then the kept routed
     * slots; partials and the combine stay indexed by compacted unit */
    auto unit_at = [&](int q) { return shared ? (q == 0 ? U - 1 : q - 1) : q; };
    PairLoad<BITS, NI> A, B;
    if (shared)
        pair_load<BITS, NI>(A, dc_rows(d, d.k, 0, row0, rowbytes), rowbytes, 0, 2, nb);
    /* per-unit values in lane registers, loaded once (U <= 32): lane j holds
     * compacted unit j's unit id, matrix index and routing weight (lane
     * 2j + r gets the row scale of this wave's row r of unit j once h is
     * staged: its address needs the id, and h's loads need nothing) */
    const int u_l = dc_unit(kept, n_kept, d.k, min(lane, U - 1), all_kept);
    const bool rt_l = u_l < d.k;
    const int e_l = rt_l ? min(max(d.ids[u_l], 0), a.seg[0].n_mat - 1) : 0;
    const float w_l = rt_l ? d.w[u_l] : 0.0f;
    /* without a shared expert, compacted unit 0's pair is issued before h is staged */
    if (!shared)
        pair_load<BITS, NI>(A, dc_rows(d, __builtin_amdgcn_readlane(u_l, 0), __builtin_amdgcn_readlane(e_l, 0), row0,
                                       rowbytes),
                            rowbytes, 0, 2, nb);
    /* the shared expert's h in fp32 (one-wave gate/up jobs; 4 nb <= 256):
     * thread 4b + q loads elements 8q .. 8q+7 of block b now, and forms the
     * Q8_0 blocks after the routed items' loads are issued */
    const bool sh_fp32 = shared && d.hs;
    const int sb = threadIdx.x >> 2, sq = threadIdx.x & 3;
    float4 hv0 = make_float4(0.0f, 0.0f, 0.0f, 0.0f), hv1 = hv0;
    if (sh_fp32) {
        const float4* src = reinterpret_cast<const float4*>(d.hs + (int64_t)min(sb, nb - 1) * 32 + 8 * sq);
        hv0 = src[0];
        hv1 = src[1];
    }
    const int n_items = (sh_fp32 ? U - 1 : U) * nb;
    /* each thread issues the loads of up to kDcStage (unit, block) items
     * before it converts and stores any: one memory round trip, not one per
     * item */
    for (int i0 = threadIdx.x; i0 < n_items; i0 += 64 * DW * kDcStage) {
        uint32_t x[kDcStage][8];
        float dv[kDcStage];
#pragma unroll
        for (int r = 0; r < kDcStage; ++r) {
            const int i = i0 + r * 64 * DW;
            if (i < n_items) {
                const int j = i / nb, b = i - j * nb;
                const int u = dc_unit(kept, n_kept, d.k, j, all_kept);
                load_codes(a.hq + (int64_t)u * a.I + (int64_t)b * 32, x[r]);
                dv[r] = a.hd[(int64_t)u * nb + b];
            }
        }
#pragma unroll
        for (int r = 0; r < kDcStage; ++r) {
            const int i = i0 + r * 64 * DW;
            if (i < n_items) {
                uint32_t xa[8];
                prep_dot<BITS>(x[r], xa);
                uint4* dst = reinterpret_cast<uint4*>(xal + (int64_t)i * 8);
                dst[0] = make_uint4(xa[0], xa[1], xa[2], xa[3]);
                dst[1] = make_uint4(xa[4], xa[5], xa[6], xa[7]);
                dls[(i / nb) * sp + i % nb] = dv[r];
            }
        }
    }
    if (sh_fp32) {
        /* the arithmetic of the gate/up epilogue: amax over the block, d =
         * amax / 127, codes q8_code(h, 1 / d) */
        const float h[8] = {hv0.x, hv0.y, hv0.z, hv0.w, hv1.x, hv1.y, hv1.z, hv1.w};
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            am = fmaxf(am, __builtin_fabsf(h[i]));
        am = fmaxf(am, shfl_xor(am, 1));
        am = fmaxf(am, shfl_xor(am, 2));
        const float dsc = am / 127.0f;
        const float inv = (am == 0.0f) ? 0.0f : 1.0f / dsc;
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            w0 |= (uint32_t)(q8_code(h[k], inv) & 0xFF) << (8 * k);
            w1 |= (uint32_t)(q8_code(h[4 + k], inv) & 0xFF) << (8 * k);
        }
        /* the block's 8 code words, from its 4 threads */
        uint32_t x[8];
        const int base = lane & ~3;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            x[2 * q] = (uint32_t)__shfl((int)w0, base + q, kWave);
            x[2 * q + 1] = (uint32_t)__shfl((int)w1, base + q, kWave);
        }
        if (sq == 0 && sb < nb) {
            uint32_t xa[8];
            prep_dot<BITS>(x, xa);
            uint4* dst = reinterpret_cast<uint4*>(xal + ((int64_t)(U - 1) * nb + sb) * 8);
            dst[0] = make_uint4(xa[0], xa[1], xa[2], xa[3]);
            dst[1] = make_uint4(xa[4], xa[5], xa[6], xa[7]);
            dls[(U - 1) * sp + sb] = dsc;
        }
    }
    const int u_r = __shfl(u_l, min(lane >> 1, U - 1), kWave);
    const int e_r = __shfl(e_l, min(lane >> 1, U - 1), kWave);
    const bool rt_r = u_r < d.k;
    const float* ds_r = rt_r ? a.seg[0].down_s : a.seg[1].down_s;
    const float rs_l = (rt_r ? a.seg[0].d_gb : a.seg[1].d_gb) ? 1.0f : ds_r[(int64_t)e_r * a.H + row0 + (lane & 1)];
    __syncthreads();

    /* fold of chains [c_begin, c_end): chain (rd, g) = (compacted unit rd / 2,
     * row rd % 2; group g), lane ci - c0 of round c0 */
    auto fold_chains = [&](int c_begin, int c_end) {
        for (int c0 = c_begin; c0 < c_end; c0 += 64) {
            const int ci = c0 + lane;
            const int rd = min(ci >> 2, 2 * U - 1), g = ci & 3;
            const int b0 = block_group(g, nb), b1 = block_group(g + 1, nb);
            const int32_t* pr = P + rd * sp;
            const float* dj = dls + (rd >> 1) * sp;
            float acc = 0.0f;
            int b = b0;
            /* lane values are read before any branch: every lane is active */
            const int uf = __shfl(u_l, rd >> 1, kWave), ef = __shfl(e_l, rd >> 1, kWave);
            const float rsv = __shfl(rs_l, rd, kWave);
            const int gbf = uf < d.k ? a.seg[0].d_gb : a.seg[1].d_gb;
            if (gbf) {
                /* group-wise scales of (unit, row) */
                const float* ws = (uf < d.k ? a.seg[0].down_s : a.seg[1].down_s) +
                                  ((int64_t)ef * a.H + row0 + (rd & 1)) * (nb / gbf);
                for (; b < b1; ++b)
                    acc = __builtin_fmaf(group_coef(ws, gbf, b, dj[b]), (float)pr[b], acc);
            } else {
                for (; b + 8 <= b1; b += 8) {
                    int32_t q[8];
                    float dd[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        q[i] = pr[b + i];
                        dd[i] = dj[b + i];
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        acc = __builtin_fmaf(dd[i], (float)q[i], acc);
                }
                for (; b < b1; ++b)
                    acc = __builtin_fmaf(dj[b], (float)pr[b], acc);
            }
            const int base = lane & ~3;
            float v = __shfl(acc, base, kWave);
            v = v + __shfl(acc, base + 1, kWave);
            v = v + __shfl(acc, base + 2, kWave);
            v = v + __shfl(acc, base + 3, kWave);
            if (g == 0 && ci < c_end)
                ys[rd] = rsv * v; /* rsv: 1 with group-wise scales */
        }
    };

    /* the pair of stream position q is in A for even q and in B for odd q;
     * loads are unconditional (past the last unit they reload it: in bounds,
     * unused) */
    for (int q = 0; q < U; q += 2) {
        uint32_t xa[NI][8];
        const int j0 = unit_at(q), j1 = unit_at(min(q + 1, U - 1)), j2 = unit_at(min(q + 2, U - 1));
        pair_load<BITS, NI>(B, dc_rows(d, __builtin_amdgcn_readlane(u_l, j1), __builtin_amdgcn_readlane(e_l, j1), row0,
                                       rowbytes),
                            rowbytes, 0, 2, nb);
        dc_act<NI>(xal, j0, nb, xa);
        pair_partials<BITS, NI>(A, xa, 0, nb, P + 2 * j0 * sp, sp);
        pair_load<BITS, NI>(A, dc_rows(d, __builtin_amdgcn_readlane(u_l, j2), __builtin_amdgcn_readlane(e_l, j2), row0,
                                       rowbytes),
                            rowbytes, 0, 2, nb);
        if (q + 1 < U) {
            dc_act<NI>(xal, j1, nb, xa);
            pair_partials<BITS, NI>(B, xa, 0, nb, P + 2 * j1 * sp, sp);
        }
        if (q == 0 && shared) {
            /* the shared expert (streamed first) is folded while the routed
             * pairs load, so the final fold is one round for 8 routed units */
            wave_lds_sync();
            fold_chains(8 * (U - 1), 8 * U);
        }
    }
    wave_lds_sync();
    fold_chains(0, shared ? 8 * (U - 1) : 8 * U);
    wave_lds_sync();
    /* compacted order is slot order: the combine's fma order is kept (every
     * lane runs the chain of row lane & 1; lanes 0 and 1 store) */
    float outv = shared ? ys[2 * n_kept + (lane & 1)] : 0.0f;
    for (int j = 0; j < n_kept; ++j)
        outv = __builtin_fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_l), j)), ys[2 * j + (lane & 1)],
                              outv);
    if (lane < 2)
        d.out[row0 + lane] = outv;
}

static int64_t total_jobs(const FfnArgs& a, int RB)
{
    int64_t n = (int64_t)a.seg[0].max_units * RB;
    if (a.nseg > 1)
        n += (int64_t)a.seg[1].max_units * RB;
    return n;
}

template <int NI, int TMAX>
static void launch_rows_ni(const FfnArgs& a, int32_t bits, bool gate_up, dim3 grid, size_t lds, hipStream_t st)
{
    const dim3 block(64 * kGroups);
    if (gate_up) {
        switch (bits) {
        case 8: hipLaunchKernelGGL((ffn_gate_up_rows<8, NI, TMAX>), grid, block, lds, st, a); break;
        case 4: hipLaunchKernelGGL((ffn_gate_up_rows<4, NI, TMAX>), grid, block, lds, st, a); break;
        default: hipLaunchKernelGGL((ffn_gate_up_rows<2, NI, TMAX>), grid, block, lds, st, a); break;
        }
    } else {
        switch (bits) {
        case 8: hipLaunchKernelGGL((ffn_down_rows<8, NI, TMAX>), grid, block, lds, st, a); break;
        case 4: hipLaunchKernelGGL((ffn_down_rows<4, NI, TMAX>), grid, block, lds, st, a); break;
        default: hipLaunchKernelGGL((ffn_down_rows<2, NI, TMAX>), grid, block, lds, st, a); break;
        }
    }
}

/* The whole-row kernels when their LDS fits, else the octet kernels. */
template <int TMAX>
static void launch_gate_up_t(const FfnArgs& a, int32_t bits, dim3 grid, hipStream_t st)
{
    const dim3 block(64 * kGroups);
    const int nb = a.H / 32;
    if (rows_fit(nb, TMAX)) {
        const size_t lds = rows_lds_words(nb, TMAX) * 4;
        switch (dec_ni(nb)) {
        case 1: launch_rows_ni<1, TMAX>(a, bits, true, grid, lds, st); break;
        case 2: launch_rows_ni<2, TMAX>(a, bits, true, grid, lds, st); break;
        case 4: launch_rows_ni<4, TMAX>(a, bits, true, grid, lds, st); break;
        case 6: launch_rows_ni<6, TMAX>(a, bits, true, grid, lds, st); break;
        default: launch_rows_ni<8, TMAX>(a, bits, true, grid, lds, st); break;
        }
        return;
    }
    switch (bits) {
    case 8: hipLaunchKernelGGL((ffn_gate_up_gemv<8, TMAX>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((ffn_gate_up_gemv<4, TMAX>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((ffn_gate_up_gemv<2, TMAX>), grid, block, 0, st, a); break;
    }
}

template <int TMAX>
static void launch_down_t(const FfnArgs& a, int32_t bits, dim3 grid, hipStream_t st)
{
    const dim3 block(64 * kGroups);
    const int nb = a.I / 32;
    if (rows_fit(nb, TMAX)) {
        const size_t lds = rows_lds_words(nb, TMAX) * 4;
        switch (dec_ni(nb)) {
        case 1: launch_rows_ni<1, TMAX>(a, bits, false, grid, lds, st); break;
        case 2: launch_rows_ni<2, TMAX>(a, bits, false, grid, lds, st); break;
        case 4: launch_rows_ni<4, TMAX>(a, bits, false, grid, lds, st); break;
        case 6: launch_rows_ni<6, TMAX>(a, bits, false, grid, lds, st); break;
        default: launch_rows_ni<8, TMAX>(a, bits, false, grid, lds, st); break;
        }
        return;
    }
    switch (bits) {
    case 8: hipLaunchKernelGGL((ffn_down_gemv<8, TMAX>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((ffn_down_gemv<4, TMAX>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((ffn_down_gemv<2, TMAX>), grid, block, 0, st, a); break;
    }
}

hipError_t launch_ffn_gate_up(const FfnArgs& a, int32_t bits, hipStream_t st)
{
    const int64_t jobs = total_jobs(a, a.I / 32);
    if (jobs == 0)
        return hipSuccess;
    if (a.unit_tokens == 1)
        launch_gate_up_t<1>(a, bits, dim3((uint32_t)jobs), st);
    else
        launch_gate_up_t<kUnitTokens>(a, bits, dim3((uint32_t)jobs), st);
    return hipGetLastError();
}

hipError_t launch_ffn_down(const FfnArgs& a, int32_t bits, hipStream_t st)
{
    const int64_t jobs = total_jobs(a, (a.H + kRowsPerJob - 1) / kRowsPerJob);
    if (jobs == 0)
        return hipSuccess;
    if (a.unit_tokens == 1)
        launch_down_t<1>(a, bits, dim3((uint32_t)jobs), st);
    else
        launch_down_t<kUnitTokens>(a, bits, dim3((uint32_t)jobs), st);
    return hipGetLastError();
}

template <int NI>
static void gate_up_decode_ni(const DecodeArgs& d, int32_t bits, dim3 grid, size_t lds, hipStream_t st)
{
    const dim3 block(64 * kGroups);
    switch (bits) {
    case 8: hipLaunchKernelGGL((ffn_gate_up_decode<8, NI>), grid, block, lds, st, d); break;
    case 4: hipLaunchKernelGGL((ffn_gate_up_decode<4, NI>), grid, block, lds, st, d); break;
    default: hipLaunchKernelGGL((ffn_gate_up_decode<2, NI>), grid, block, lds, st, d); break;
    }
}

template <int NI>
static void down_decode_ni(const DecodeArgs& d, int32_t bits, dim3 grid, size_t lds, hipStream_t st)
{
    const dim3 block(64 * kGroups);
    switch (bits) {
    case 8: hipLaunchKernelGGL((ffn_down_decode<8, NI>), grid, block, lds, st, d); break;
    case 4: hipLaunchKernelGGL((ffn_down_decode<4, NI>), grid, block, lds, st, d); break;
    default: hipLaunchKernelGGL((ffn_down_decode<2, NI>), grid, block, lds, st, d); break;
    }
}

hipError_t launch_ffn_gate_up_decode(const DecodeArgs& d, int32_t bits, hipStream_t st)
{
    /* one-wave jobs of the shared expert (d.hs), then whole jobs */
    const int64_t jobs = (int64_t)(d.k + (d.f.nseg > 1 && !d.hs ? 1 : 0)) * (d.f.I / 32) + (d.hs ? d.f.I / 8 : 0);
    const int nb = d.f.H / 32;
    const dim3 grid((uint32_t)jobs);
    const size_t lds = dec_lds_bytes(nb);
    switch (dec_ni(nb)) {
    case 1: gate_up_decode_ni<1>(d, bits, grid, lds, st); break;
    case 2: gate_up_decode_ni<2>(d, bits, grid, lds, st); break;
    case 4: gate_up_decode_ni<4>(d, bits, grid, lds, st); break;
    case 6: gate_up_decode_ni<6>(d, bits, grid, lds, st); break;
    default: gate_up_decode_ni<8>(d, bits, grid, lds, st); break;
    }
    return hipGetLastError();
}

hipError_t launch_ffn_down_decode(const DecodeArgs& d, int32_t bits, hipStream_t st)
{
    const int64_t jobs = (int64_t)(d.k + (d.f.nseg > 1 ? 1 : 0)) * ((d.f.H + kRowsPerJob - 1) / kRowsPerJob);
    const int nb = d.f.I / 32;
    const dim3 grid((uint32_t)jobs);
    const size_t lds = dec_lds_bytes(nb);
    switch (dec_ni(nb)) {
    case 1: down_decode_ni<1>(d, bits, grid, lds, st); break;
    case 2: down_decode_ni<2>(d, bits, grid, lds, st); break;
    case 4: down_decode_ni<4>(d, bits, grid, lds, st); break;
    case 6: down_decode_ni<6>(d, bits, grid, lds, st); break;
    default: down_decode_ni<8>(d, bits, grid, lds, st); break;
    }
    return hipGetLastError();
}

template <int BITS, int NI, int DW>
static void down_combine_launch(const DecodeArgs& d, dim3 grid, size_t lds, hipStream_t st)
{
    if (lds > 64 * 1024) {
        static bool raised = false; /* once per instantiation */
        if (!raised) {
            (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_down_combine_decode<BITS, NI, DW>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDcLdsMax);
            raised = true;
        }
    }
    hipLaunchKernelGGL((ffn_down_combine_decode<BITS, NI, DW>), grid, dim3(64 * DW), lds, st, d);
}

template <int NI, int DW>
static void down_combine_ni(const DecodeArgs& d, int32_t bits, dim3 grid, size_t lds, hipStream_t st)
{
    switch (bits) {
    case 8: down_combine_launch<8, NI, DW>(d, grid, lds, st); break;
    case 4: down_combine_launch<4, NI, DW>(d, grid, lds, st); break;
    default: down_combine_launch<2, NI, DW>(d, grid, lds, st); break;
    }
}

/* Waves per workgroup of the fused down + combine: kDcWide when the rows
 * divide evenly and its LDS fits a CU, else 4. */
static int dc_waves(const DecodeArgs& d)
{
    const int U = d.k + (d.f.nseg > 1 ? 1 : 0);
    const int nb = d.f.I / 32;
    if (d.f.H % (2 * kDcWide) == 0 && dc_lds_words(U, nb, kDcWide) * 4 <= kDcLdsMax)
        return kDcWide;
    return kGroups;
}

bool down_combine_decode_fits(const DecodeArgs& d)
{
    const int U = d.k + (d.f.nseg > 1 ? 1 : 0);
    /* per-unit values live in lanes: 2U row scales per wave */
    return U <= 32 && d.f.H % (2 * kGroups) == 0 && dc_lds_words(U, d.f.I / 32, kGroups) * 4 <= 64 * 1024;
}

hipError_t launch_ffn_down_combine_decode(const DecodeArgs& d, int32_t bits, hipStream_t st)
{
    const int U = d.k + (d.f.nseg > 1 ? 1 : 0);
    const int nb = d.f.I / 32;
    const int DW = dc_waves(d);
    const dim3 grid((uint32_t)(d.f.H / (2 * DW)));
    const size_t lds = dc_lds_words(U, nb, DW) * 4;
    if (DW == kDcWide) {
        switch (dec_ni(nb)) {
        case 1: down_combine_ni<1, kDcWide>(d, bits, grid, lds, st); break;
        case 2: down_combine_ni<2, kDcWide>(d, bits, grid, lds, st); break;
        case 4: down_combine_ni<4, kDcWide>(d, bits, grid, lds, st); break;
        case 6: down_combine_ni<6, kDcWide>(d, bits, grid, lds, st); break;
        default: down_combine_ni<8, kDcWide>(d, bits, grid, lds, st); break;
        }
    } else {
        switch (dec_ni(nb)) {
        case 1: down_combine_ni<1, kGroups>(d, bits, grid, lds, st); break;
        case 2: down_combine_ni<2, kGroups>(d, bits, grid, lds, st); break;
        case 4: down_combine_ni<4, kGroups>(d, bits, grid, lds, st); break;
        case 6: down_combine_ni<6, kGroups>(d, bits, grid, lds, st); break;
        default: down_combine_ni<8, kGroups>(d, bits, grid, lds, st); break;
        }
    }
    return hipGetLastError();
}

} // namespace coli
