/*
 * ffn_mfma.hip -- gated expert FFN on the integer dot path, grouped-GEMM form
 * on the int8 matrix cores, for the experts of a batch of more than 8 tokens
 * that hold at least the batch's threshold of its tokens (every expert, when
 * the batch averages 8 or more tokens per expert; layer_mfma_min in
 * kernels.h) (prefill batches: "Show HN: 如何在我的低配置电脑上运行 GLM-5.2",
 * implemented features, batched-union MoE item; integer dot-product and
 * quantised-kernel items; Metal section: SwiGLU; resource-policy section:
 * gate and up in one dispatch).
 *
 * Work unit: one expert and up to kMfmaUnitTokens of its sorted positions
 * (up to two N-tiles of 16 tokens).  A 256-thread workgroup covers 64 row
 * dots (gate/up kernel: 32 gate rows and the same 32 up rows, one 32-block of
 * h; down kernel: 64 output rows); wave w owns the 16-row M-tile w.
 *
 * One v_mfma_i32_16x16x32_i8 covers exactly one Q8_0 block (K = 32), so its
 * int32 result is the exact block partial of 16 rows x 16 tokens.  Weights
 * enter as their packed fields shifted to the top of each byte (2^(8-b) * v,
 * see qdot.h) and activations in the matching operand order; the 2^(8-b)
 * factor is taken out of the block scale (exact whenever d * 2^-(8-b) is a
 * normal number; a K step holding any other scale shifts the partials back
 * instead).  The fp32 fold is the canonical one: one chain per (row, token)
 * from +0 over the blocks in ascending order, then the row scale.
 *
 * Memory pipeline.  A K step is 128 bytes of every weight row (8 blocks of
 * int4 / int2 half that, 4 blocks of int8) and the matching activation
 * blocks of the unit's tokens.  Each thread holds two steps of global loads
 * in registers while the workgroup multiplies a third out of LDS, so every
 * workgroup keeps two steps (16 KB of int4 weights) in flight; one barrier
 * per step.  LDS row strides are padded so that the MFMA operand reads of a
 * wave hit distinct banks.
 */
#include "device_common.h"
#include "kernels.h"

namespace coli {

namespace {

constexpr int kTok = kMfmaUnitTokens; /* tokens of a unit (N) */

template <int BITS>
struct Cfg {
    static constexpr int kStep = BITS == 8 ? 4 : 8;                   /* K blocks per step */
    static constexpr int kRowWords = kStep * BITS;                    /* packed words per row and step */
    static constexpr int kRowStride = kRowWords + (BITS == 2 ? 1 : 2); /* LDS words per row */
    static constexpr int kBpt = kStep / 4;                            /* weight blocks per loading thread */
    static constexpr int kXpt = kStep == 8 ? 8 : 4;                   /* activation words per loading thread */
};

/* LDS of the K loop, double-buffered.  GROUPED kernels also stage each
 * weight row's group-wise scale of every block of the step (one word when
 * not grouped, so that the per-row kernels keep their LDS size). */
template <int BITS, bool GROUPED = false>
struct KLds {
    uint32_t a[2][64 * Cfg<BITS>::kRowStride];              /* weight rows, packed words */
    uint32_t b[2][Cfg<BITS>::kStep][4][kTok][2];           /* operand words 2g, 2g+1 per (block, g, token) */
    float ds[2][GROUPED ? 1 : Cfg<BITS>::kStep][kTok];      /* block scale * 2^-(8-b) (per-row kernels) */
    float dr[2][Cfg<BITS>::kStep][kTok];                    /* block scale */
    int flag[2];                                            /* step whose scales need the exact-shift fold */
    float ws[2][GROUPED ? 64 * Cfg<BITS>::kStep : 1];       /* [row][block of the step] weight scale */
};

/* The aligned K loop's weight loads: every instruction reads whole 16-byte
 * chunks of kCR consecutive chunks per row (a row's whole step), kNL
 * instructions per thread; its LDS rows are 16-byte aligned, at a stride
 * whose A-operand reads hit distinct banks. */
template <int BITS>
struct LCfg {
    static constexpr int kCR = Cfg<BITS>::kRowWords / 4; /* 16-byte chunks per row and step */
    static constexpr int kNL = kCR / 4;                  /* weight loads per thread */
    static constexpr int kRowsPerLoad = 256 / kCR;
    static constexpr int kStride = Cfg<BITS>::kRowWords + 4;
    /* activations: a token's step (kStep blocks) is kXC 16-byte chunks, read
     * by kXC consecutive lanes; kNXL loads per thread */
    static constexpr int kXC = 2 * Cfg<BITS>::kStep;
    static constexpr int kNXL = kXC / 8;
    static constexpr int kTokPerLoad = 256 / kXC;
};

/* Token slot of (block j, operand group g) in the aligned loop's B layout:
 * the 16 tokens of a tile are stored XOR-permuted by (j, g), so that the
 * stores of one instruction (one token per 16 lanes, every block and half)
 * spread over the banks while a lane group's reads stay contiguous. */
__device__ __forceinline__ int lean_slot(int tr, int j, int g)
{
    return tr ^ ((2 * j + (g >> 1)) & 15);
}

/* The block scale a thread loads in each step: consecutive threads take
 * consecutive blocks of one token, so a wave's load covers whole token
 * slices (int8: threads 128.. repeat 0..127). */
template <int BITS>
__device__ __forceinline__ int lean_d_token()
{
    const int l = threadIdx.x;
    return Cfg<BITS>::kStep == 8 ? (l >> 3) : ((l >> 2) & 31);
}

template <int BITS>
__device__ __forceinline__ int lean_d_block()
{
    return (int)threadIdx.x & (Cfg<BITS>::kStep - 1);
}

/* LDS of the aligned K loop: the two N-tiles' operands of a lane side by
 * side, so that one read brings both. */
template <int BITS, bool GW = false>
struct __attribute__((aligned(16))) LeanLds {
    __attribute__((aligned(16))) uint32_t a[2][64 * LCfg<BITS>::kStride]; /* weight rows, packed words */
    __attribute__((aligned(16))) uint32_t b[2][Cfg<BITS>::kStep][4][16][2][2]; /* [block][g][token & 15][tile][word] */
    __attribute__((aligned(16))) float ds[2][Cfg<BITS>::kStep][16][2];        /* [block][token & 15][tile] */
    /* GW: each row's group-wise weight scale of each block of the step */
    __attribute__((aligned(16))) float ws[2][Cfg<BITS>::kStep][GW ? 64 : 4]; /* [block][row] */
};

struct EpiLds {
    float v[64][kTok + 1]; /* [row dot][token] */
};

template <int BITS, bool GROUPED = false>
union MfmaShared {
    KLds<BITS, GROUPED> k;
    LeanLds<BITS, GROUPED> l;
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
        pos0 = u * kTok;
        ntok = kTok;
    }
    if (e < 0 || e >= sg.n_mat || pos0 < 0 || pos0 >= sg.rows || ntok <= 0)
        return false;
    ntok = min(min(ntok, kTok), sg.rows - pos0);
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

/* Where a unit's MFMA results belong, for the test-only partial dump: row
 * dot rd < split is weight row wlo + rd of kind klo, else whi + rd - split
 * of kind khi (rows from wmax on do not exist); token t is output row o0 + t
 * (tokens from ntok on do not exist). */
struct MDbg {
    int64_t o0;
    int ntok, split, klo, khi, wlo, whi, wmax;
};

/* The exact partials of one MFMA result (N-tile n, block b; the weights
 * entered as 2^shift times their values). */
__device__ __forceinline__ void mdbg(const FfnArgs& a, const MDbg& m, const i32x4& c, int n, int b, int shift)
{
#ifdef COLI_DEBUG_PARTIALS
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int t = 16 * n + (lane & 15);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int rd = 16 * wv + 4 * (lane >> 4) + v;
        const bool lo = rd < m.split;
        const int wr = lo ? m.wlo + rd : m.whi + rd - m.split;
        if (t < m.ntok && wr < m.wmax)
            dbg_partial(a, lo ? m.klo : m.khi, m.o0 + t, wr, b, c[v] >> shift);
    }
#else
    (void)a; (void)m; (void)c; (void)n; (void)b; (void)shift;
#endif
}

/* One thread's share of a K step's global loads (GROUPED: also the
 * weight row's scales of its kBpt blocks). */
template <int BITS, bool GROUPED = false>
struct Stage {
    uint32_t w[Cfg<BITS>::kBpt * BITS];
    uint32_t x[Cfg<BITS>::kXpt];
    float d;
    float sc[GROUPED ? Cfg<BITS>::kBpt : 1];
};

/* Where a thread loads from.  Weights: row dot (l >> 2), blocks kBpt*(l & 3)
 * .. of the step.  Activations: token (l & 31), block (l >> 5) of the step
 * (int8: block (l >> 6), half ((l >> 5) & 1)).  Block indices past the row
 * are clamped to its last block: those loads stay in bounds and their data
 * is never multiplied. */
struct LoadLane {
    const uint8_t* wrow;
    const int8_t* xrow;
    const float* xdrow;
    int nb;
    const float* wsrow; /* group-wise scales of the weight row (GROUPED kernels; gb == 0: none) */
    int gb;             /* blocks per scale */
};

template <int BITS, bool GROUPED>
__device__ __forceinline__ void fetch(Stage<BITS, GROUPED>& P, const LoadLane& L, int st)
{
    using C = Cfg<BITS>;
    const int l = threadIdx.x;
    const int wb0 = st * C::kStep + C::kBpt * (l & 3);
    if constexpr (GROUPED) {
#pragma unroll
        for (int i = 0; i < C::kBpt; ++i)
            P.sc[i] = L.gb ? L.wsrow[min(wb0 + i, L.nb - 1) / L.gb] : 1.0f; /* per-row: 1 * d = d */
    }
#pragma unroll
    for (int i = 0; i < C::kBpt; ++i) {
        const int b = min(wb0 + i, L.nb - 1);
        const uint8_t* p = L.wrow + (int64_t)b * (4 * BITS);
        if constexpr (BITS == 8) {
            const u32x4 u = reinterpret_cast<const u32x4*>(p)[0];
            const u32x4 v = reinterpret_cast<const u32x4*>(p)[1];
            P.w[0] = u.x; P.w[1] = u.y; P.w[2] = u.z; P.w[3] = u.w;
            P.w[4] = v.x; P.w[5] = v.y; P.w[6] = v.z; P.w[7] = v.w;
        } else if constexpr (BITS == 4) {
            const u32x4 u = reinterpret_cast<const u32x4*>(p)[0];
            P.w[4 * i + 0] = u.x; P.w[4 * i + 1] = u.y; P.w[4 * i + 2] = u.z; P.w[4 * i + 3] = u.w;
        } else {
            const u32x2 u = reinterpret_cast<const u32x2*>(p)[0];
            P.w[2 * i + 0] = u.x; P.w[2 * i + 1] = u.y;
        }
    }
    if constexpr (C::kStep == 8) {
        const int b = min(st * C::kStep + (l >> 5), L.nb - 1);
        const u32x4* q = reinterpret_cast<const u32x4*>(L.xrow + (int64_t)b * 32);
        const u32x4 u = q[0], v = q[1];
        P.x[0] = u.x; P.x[1] = u.y; P.x[2] = u.z; P.x[3] = u.w;
        P.x[4] = v.x; P.x[5] = v.y; P.x[6] = v.z; P.x[7] = v.w;
        P.d = L.xdrow[b];
    } else {
        const int b = min(st * C::kStep + (l >> 6), L.nb - 1);
        const u32x4 u = reinterpret_cast<const u32x4*>(L.xrow + (int64_t)b * 32)[(l >> 5) & 1];
        P.x[0] = u.x; P.x[1] = u.y; P.x[2] = u.z; P.x[3] = u.w;
        P.d = L.xdrow[b];
    }
}

template <int BITS, bool GROUPED>
__device__ __forceinline__ void commit(const Stage<BITS, GROUPED>& P, KLds<BITS, GROUPED>& S, int buf, int st)
{
    using C = Cfg<BITS>;
    constexpr int SHIFT = 8 - BITS;
    const int l = threadIdx.x;
    if constexpr (GROUPED) {
#pragma unroll
        for (int i = 0; i < C::kBpt; ++i)
            S.ws[buf][(l >> 2) * C::kStep + C::kBpt * (l & 3) + i] = P.sc[i];
    }
    uint32_t* ad = &S.a[buf][(l >> 2) * C::kRowStride + C::kBpt * BITS * (l & 3)];
#pragma unroll
    for (int i = 0; i < C::kBpt * BITS; ++i)
        ad[i] = P.w[i];
    const int t = l & 31;
    int j;
    if constexpr (C::kStep == 8) {
        j = l >> 5;
        uint32_t xa[8];
        prep_activation<BITS>(P.x, xa);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            S.b[buf][j][g][t][0] = xa[2 * g];
            S.b[buf][j][g][t][1] = xa[2 * g + 1];
        }
    } else {
        /* int8: natural operand order, half h holds operand groups 2h, 2h+1 */
        j = l >> 6;
        const int h = (l >> 5) & 1;
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
            S.b[buf][j][2 * h + gg][t][0] = P.x[2 * gg];
            S.b[buf][j][2 * h + gg][t][1] = P.x[2 * gg + 1];
        }
    }
    S.dr[buf][j][t] = P.d;
    if constexpr (!GROUPED) {
        const float ds = P.d * (1.0f / (float)(1 << SHIFT));
        S.ds[buf][j][t] = ds;
        if (SHIFT != 0 && P.d != 0.0f && !(ds >= 1.17549435e-38f))
            S.flag[buf] = st;
    }
}

/* A operand of lane group g (elements 8g .. 8g+7 of the block, in the order
 * prep_activation gives the activation codes) from the block's packed words. */
template <int BITS>
__device__ __forceinline__ long a_operand(const uint32_t* w, int g)
{
    uint32_t lo, hi;
    if constexpr (BITS == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(w + 2 * g);
        lo = v.x;
        hi = v.y;
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

/* One block of a K step: the MFMA of each N-tile and its fold into acc. */
template <int BITS, int NT, bool EXACT_SHIFT, class KL>
__device__ __forceinline__ void block_mfma(const KL& S, int buf, int j, const uint32_t* arow,
                                           int r, int g, float (&acc)[2][4], const FfnArgs& a, const MDbg& m, int b)
{
    constexpr int SHIFT = 8 - BITS;
    const long A = a_operand<BITS>(arow + j * BITS, g);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int t = 16 * n + r;
        const uint2 bw = *reinterpret_cast<const uint2*>(&S.b[buf][j][g][t][0]);
        const long B = (long)(((uint64_t)bw.y << 32) | bw.x);
        const i32x4 c = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, i32x4{0, 0, 0, 0}, 0, 0, 0);
        mdbg(a, m, c, n, b, SHIFT);
        if constexpr (!EXACT_SHIFT) {
            const float d = S.ds[buf][j][t];
#pragma unroll
            for (int v = 0; v < 4; ++v)
                acc[n][v] = __builtin_fmaf(d, (float)c[v], acc[n][v]);
        } else {
            const float d = S.dr[buf][j][t];
#pragma unroll
            for (int v = 0; v < 4; ++v)
                acc[n][v] = __builtin_fmaf(d, (float)(c[v] >> SHIFT), acc[n][v]);
        }
    }
}

/* One block with group-wise scales: coefficient s * d (the canonical fp32
 * product, s the row's scale of the block staged in LDS) for each of the
 * lane's row dots 16w + 4(lane/16) + v, on the exact partials (the 2^(8-b)
 * factor of the packed weights shifted back out). */
template <int BITS, int NT>
__device__ __forceinline__ void block_mfma_grouped(const KLds<BITS, true>& S, int buf, int j,
                                                   const uint32_t* arow, int r, int g, float (&acc)[2][4],
                                                   const FfnArgs& a, const MDbg& m, int b)
{
    using C = Cfg<BITS>;
    constexpr int SHIFT = 8 - BITS;
    const int wv = threadIdx.x >> 6;
    const long A = a_operand<BITS>(arow + j * BITS, g);
    float wsv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
        wsv[v] = S.ws[buf][(16 * wv + 4 * g + v) * C::kStep + j];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int t = 16 * n + r;
        const uint2 bw = *reinterpret_cast<const uint2*>(&S.b[buf][j][g][t][0]);
        const long B = (long)(((uint64_t)bw.y << 32) | bw.x);
        const i32x4 c = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, i32x4{0, 0, 0, 0}, 0, 0, 0);
        mdbg(a, m, c, n, b, SHIFT);
        const float d = S.dr[buf][j][t];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            acc[n][v] = __builtin_fmaf(wsv[v] * d, (float)(c[v] >> SHIFT), acc[n][v]);
            asm volatile("" : "+v"(acc[n][v])); /* keeps each block's fold in place */
        }
    }
}

/* Multiplies one K step out of LDS buffer `buf` into acc (NT N-tiles).
 *
 * The common step -- all kStep blocks inside the row, every scale exact
 * after the 2^-(8-b) factor -- runs as straight-line code.  Any other step
 * checks each block: the row end and the shift-back fold. */
template <int BITS, int NT, bool GROUPED>
__device__ __forceinline__ void step(const KLds<BITS, GROUPED>& S, int buf, int st, int nb, float (&acc)[2][4],
                                     int gb, const FfnArgs& a, const MDbg& m)
{
    using C = Cfg<BITS>;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const uint32_t* arow = &S.a[buf][(16 * wv + r) * C::kRowStride];
    const int b0 = st * C::kStep, b1 = b0 + C::kStep;
    if (b0 >= nb)
        return;
    (void)gb;
    if constexpr (GROUPED) {
        /* every segment of a grouped launch: per-row segments carry scale 1 */
        if (b1 <= nb) {
#pragma unroll
            for (int j = 0; j < C::kStep; ++j)
                block_mfma_grouped<BITS, NT>(S, buf, j, arow, r, g, acc, a, m, b0 + j);
            return;
        }
        for (int j = 0; j < C::kStep && b0 + j < nb; ++j)
            block_mfma_grouped<BITS, NT>(S, buf, j, arow, r, g, acc, a, m, b0 + j);
    } else {
        const bool exact_shift = BITS != 8 && __builtin_amdgcn_readfirstlane(S.flag[buf]) == st;
        if (b1 <= nb && !exact_shift) {
#pragma unroll
            for (int j = 0; j < C::kStep; ++j)
                block_mfma<BITS, NT, false>(S, buf, j, arow, r, g, acc, a, m, b0 + j);
            return;
        }
        for (int j = 0; j < C::kStep && b0 + j < nb; ++j) {
            if (exact_shift)
                block_mfma<BITS, NT, true>(S, buf, j, arow, r, g, acc, a, m, b0 + j);
            else
                block_mfma<BITS, NT, false>(S, buf, j, arow, r, g, acc, a, m, b0 + j);
        }
    }
}

/* The K loop shared by both kernels, for NT N-tiles.  Leaves in acc[n][v]
 * the folded sums of row dot 16w + 4(lane/16) + v for token 16n + lane%16.
 *
 * Step st is multiplied out of LDS buffer st & 1.  While an even step is
 * multiplied, P1 holds the loads of st + 1 and P0 those of st + 2 (the roles
 * swap for odd steps).  Every fetch and commit is unconditional -- loads past
 * the last step are clamped in bounds and their LDS copies never multiplied --
 * so the two register sets stay put across iterations and each commit waits
 * only for its own loads. */
template <int BITS, int NT, bool GROUPED>
__device__ __forceinline__ void k_loop_nt(KLds<BITS, GROUPED>& S, const LoadLane& L, float (&acc)[2][4],
                                          const FfnArgs& a, const MDbg& m)
{
    using C = Cfg<BITS>;
    const int nb = L.nb;
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            acc[n][v] = 0.0f;
    const int nsteps = (nb + C::kStep - 1) / C::kStep;
    Stage<BITS, GROUPED> P0, P1;
    fetch<BITS, GROUPED>(P0, L, 0);
    fetch<BITS, GROUPED>(P1, L, 1);
    if (threadIdx.x < 2)
        S.flag[threadIdx.x] = -1;
    __syncthreads();
    commit<BITS, GROUPED>(P0, S, 0, 0);
    fetch<BITS, GROUPED>(P0, L, 2);
    __syncthreads();
    for (int st = 0; st < nsteps; st += 2) {
        step<BITS, NT, GROUPED>(S, 0, st, nb, acc, L.gb, a, m);
        commit<BITS, GROUPED>(P1, S, 1, st + 1);
        fetch<BITS, GROUPED>(P1, L, st + 3);
        __syncthreads();
        step<BITS, NT, GROUPED>(S, 1, st + 1, nb, acc, L.gb, a, m);
        commit<BITS, GROUPED>(P0, S, 0, st + 2);
        fetch<BITS, GROUPED>(P0, L, st + 4);
        __syncthreads();
    }
}

template <int BITS, bool GROUPED>
__device__ __forceinline__ void mfma_k_loop(KLds<BITS, GROUPED>& S, const LoadLane& L, int ntiles,
                                            float (&acc)[2][4], const FfnArgs& a, const MDbg& m)
{
    if (ntiles > 1)
        k_loop_nt<BITS, 2, GROUPED>(S, L, acc, a, m);
    else
        k_loop_nt<BITS, 1, GROUPED>(S, L, acc, a, m);
}

/* ---- the aligned K loop ----------------------------------------------------
 *
 * For rows of a whole, even number of K steps (nb a multiple of 2 kStep:
 * H = 6144 and I = 2048 both are), with per-row weight scales, so a step
 * never checks for the row end.  Every load takes a uniform
 * base (the wave's weight matrix, the activation arrays, advanced by the
 * step index) plus a fixed 32-bit per-thread offset, so a step's addressing
 * costs no vector instructions.  It always folds with the block scale times
 * 2^-(8-b); a step whose scale would not be exact that way is only noted,
 * and the caller then recomputes the unit with the general loop above. */

template <int BITS>
__device__ __forceinline__ bool lean_shape(int nb)
{
    return nb > 0 && nb % (2 * Cfg<BITS>::kStep) == 0;
}

struct LeanLane {
    const uint8_t* wb[2]; /* wave-uniform: matrix window of weight load i */
    const int8_t* x;      /* uniform: activation codes */
    const float* xd;      /* uniform: activation block scales */
    uint32_t wo[2];       /* thread: byte offset of weight load i's chunk of step 0 */
    uint32_t xo[2];       /* thread: element offset of activation load i's chunk of step 0 */
    uint32_t dof;      /* thread: index of its activation block scale of step 0 */
    int nsteps;
    /* grouped launches: the wave's window of group-wise weight scales, the
     * thread's row offset in it (row (l / 4) of the workgroup's 64, ng per
     * row), blocks per scale (0: per-row segment, scale 1) and the divisor
     * for block -> group (umulhi(b, magic) = b / gb exactly for b < 2^16) */
    const float* wsb;
    uint32_t wso, magic;
    int gb, ng;
};

/* Weight scales per thread and step in a grouped launch: 64 rows x kStep
 * blocks over 256 threads. */
template <int BITS>
constexpr int kLeanWsPerThread = Cfg<BITS>::kStep / 4;

template <int BITS, bool GW>
struct LeanStage {
    Stage<BITS, false> p;
    float wsc[GW ? kLeanWsPerThread<BITS> : 1];
};

template <int BITS, int NT, bool GW>
__device__ __forceinline__ void lean_fetch(LeanStage<BITS, GW>& Q, const LeanLane& L, int st)
{
    using C = Cfg<BITS>;
    Stage<BITS, false>& P = Q.p;
    /* steps past the row reload its last step (never multiplied) */
    const int s = min(st, L.nsteps - 1);
    if constexpr (GW) {
        /* thread l: row l / 4, blocks kLeanWsPerThread * (l % 4) + i of the step */
        const uint32_t b0 = (uint32_t)(s * C::kStep + kLeanWsPerThread<BITS> * ((int)threadIdx.x & 3));
        if (kLeanWsPerThread<BITS> == 2 && L.gb == 1 && (reinterpret_cast<uintptr_t>(L.wsb) & 7) == 0) {
            /* one scale per block: the pair of blocks (b0 and the row offset
             * even: nb is a multiple of 16 here) in one 8-byte load */
            const float2 v = *reinterpret_cast<const float2*>(L.wsb + L.wso + min(b0, (uint32_t)L.ng - 2u));
            Q.wsc[0] = v.x;
            Q.wsc[kLeanWsPerThread<BITS> - 1] = v.y;
        } else {
#pragma unroll
            for (int i = 0; i < kLeanWsPerThread<BITS>; ++i) {
                const uint32_t b = b0 + (uint32_t)i;
                const uint32_t g = L.gb == 1 ? b : __umulhi(b, L.magic);
                Q.wsc[i] = L.gb ? L.wsb[L.wso + min(g, (uint32_t)L.ng - 1u)] : 1.0f;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < LCfg<BITS>::kNL; ++i) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(L.wb[i] + (size_t)s * (C::kRowWords * 4) + L.wo[i]);
        P.w[4 * i + 0] = u.x; P.w[4 * i + 1] = u.y; P.w[4 * i + 2] = u.z; P.w[4 * i + 3] = u.w;
    }
    /* one tile: the second load (tokens 16..31) is not needed */
    constexpr int NX = (NT == 1 && LCfg<BITS>::kNXL == 2) ? 1 : LCfg<BITS>::kNXL;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(L.x + (size_t)s * (C::kStep * 32) + L.xo[i]);
        P.x[4 * i + 0] = u.x; P.x[4 * i + 1] = u.y; P.x[4 * i + 2] = u.z; P.x[4 * i + 3] = u.w;
    }
    P.d = L.xd[(size_t)s * C::kStep + L.dof];
}

/* commit() into the aligned loop's layout, without the exact-shift
 * bookkeeping; true when this thread's block scale times 2^-(8-b) is not
 * exact. */
/* prep_activation() of one 16-byte half of a block: the operand words of
 * lane groups 2h and 2h + 1 (h the half). */
template <int BITS>
__device__ __forceinline__ void prep_half(const uint32_t* x, uint32_t (&xa)[4])
{
    if constexpr (BITS == 8) {
        xa[0] = x[0]; xa[1] = x[1]; xa[2] = x[2]; xa[3] = x[3];
    } else if constexpr (BITS == 4) {
        xa[0] = COLI_PERM(x[1], x[0], 0x06040200u);
        xa[1] = COLI_PERM(x[1], x[0], 0x07050301u);
        xa[2] = COLI_PERM(x[3], x[2], 0x06040200u);
        xa[3] = COLI_PERM(x[3], x[2], 0x07050301u);
    } else {
        const uint32_t ab_lo = COLI_PERM(x[1], x[0], 0x05010400u), ab_hi = COLI_PERM(x[1], x[0], 0x07030602u);
        const uint32_t cd_lo = COLI_PERM(x[3], x[2], 0x05010400u), cd_hi = COLI_PERM(x[3], x[2], 0x07030602u);
        xa[0] = COLI_PERM(cd_lo, ab_lo, 0x05040100u);
        xa[1] = COLI_PERM(cd_lo, ab_lo, 0x07060302u);
        xa[2] = COLI_PERM(cd_hi, ab_hi, 0x05040100u);
        xa[3] = COLI_PERM(cd_hi, ab_hi, 0x07060302u);
    }
}

template <int BITS, int NT, bool GW>
__device__ __forceinline__ bool lean_commit(const LeanStage<BITS, GW>& Q, LeanLds<BITS, GW>& S, int buf)
{
    constexpr int SHIFT = 8 - BITS;
    using LC = LCfg<BITS>;
    const Stage<BITS, false>& P = Q.p;
    const int l = threadIdx.x;
    bool bad_ws = false;
    if constexpr (GW) {
        /* a coefficient ws * d * 2^-(8-b) is the canonical product times an
         * exact power of two while both factors lie in [2^-62, 2^62]
         * (or one is zero): the product stays a normal number */
#pragma unroll
        for (int i = 0; i < kLeanWsPerThread<BITS>; ++i) {
            const float v = Q.wsc[i];
            S.ws[buf][kLeanWsPerThread<BITS> * (l & 3) + i][l >> 2] = v;
            const float m = __builtin_fabsf(v);
            bad_ws = bad_ws || (v != 0.0f && !(m >= 0x1p-62f && m <= 0x1p62f));
        }
    }
#pragma unroll
    for (int i = 0; i < LC::kNL; ++i) {
        const int row = i * LC::kRowsPerLoad + l / LC::kCR;
        *reinterpret_cast<u32x4*>(&S.a[buf][row * LC::kStride + 4 * (l % LC::kCR)]) =
            u32x4{P.w[4 * i], P.w[4 * i + 1], P.w[4 * i + 2], P.w[4 * i + 3]};
    }
    constexpr int NX = (NT == 1 && LC::kNXL == 2) ? 1 : LC::kNXL;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
        const int tt = i * LC::kTokPerLoad + l / LC::kXC, c = l % LC::kXC;
        const int jx = c >> 1, h = c & 1;
        uint32_t xa[4];
        prep_half<BITS>(&P.x[4 * i], xa);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int g = 2 * h + k;
            *reinterpret_cast<u32x2*>(&S.b[buf][jx][g][lean_slot(tt & 15, jx, g)][tt >> 4][0]) =
                u32x2{xa[2 * k], xa[2 * k + 1]};
        }
    }
    /* block scales: token lean_d_token(), block lean_d_block() of the step */
    const int t = lean_d_token<BITS>(), tr = t & 15, tn = t >> 4;
    const int j = lean_d_block<BITS>();
    const float ds = P.d * (1.0f / (float)(1 << SHIFT));
    S.ds[buf][j][tr][tn] = ds;
    if constexpr (GW)
        return bad_ws || (P.d != 0.0f && !(ds >= 0x1p-62f && ds <= 0x1p62f));
    return SHIFT != 0 && P.d != 0.0f && !(ds >= 1.17549435e-38f);
}

/* One block's LDS operands for a lane: its weight word(s), the B operand of
 * each N-tile and the tiles' block scales. */
template <int BITS, int NT, bool GW>
struct LeanOps {
    uint32_t w[BITS == 8 ? 2 : 1];
    uint32_t b[2 * NT];
    float d[NT];
};

template <int BITS, int NT, bool GW>
__device__ __forceinline__ void lean_read(const LeanLds<BITS, GW>& S, int buf, int j, const uint32_t* arow, int r,
                                          int g, LeanOps<BITS, NT, GW>& o)
{

    if constexpr (BITS == 8) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(arow + j * BITS + 2 * g);
        o.w[0] = v.x;
        o.w[1] = v.y;
    } else if constexpr (BITS == 4) {
        o.w[0] = arow[j * BITS + g];
    } else {
        o.w[0] = arow[j * BITS + (g >> 1)];
    }
    const int rs = lean_slot(r, j, g);
    if constexpr (NT == 2) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(&S.b[buf][j][g][rs][0][0]);
        o.b[0] = v.x; o.b[1] = v.y; o.b[2] = v.z; o.b[3] = v.w;
        const float2 d = *reinterpret_cast<const float2*>(&S.ds[buf][j][r][0]);
        o.d[0] = d.x;
        o.d[1] = d.y;
    } else {
        const u32x2 v = *reinterpret_cast<const u32x2*>(&S.b[buf][j][g][rs][0][0]);
        o.b[0] = v.x; o.b[1] = v.y;
        o.d[0] = S.ds[buf][j][r][0];
    }
}

template <int BITS, int NT, bool GW>
__device__ __forceinline__ void lean_mfma(const LeanOps<BITS, NT, GW>& o, int g, i32x4 (&c)[NT])
{
    /* the A operand of a_operand(), from the one word lane group g needs */
    uint32_t lo, hi;
    if constexpr (BITS == 8) {
        lo = o.w[0];
        hi = o.w[1];
    } else if constexpr (BITS == 4) {
        lo = o.w[0] & 0xF0F0F0F0u;
        hi = (o.w[0] << 4) & 0xF0F0F0F0u;
    } else {
        const int r0 = 2 * (g & 1);
        lo = (o.w[0] << (2 * r0)) & 0xC0C0C0C0u;
        hi = (o.w[0] << (2 * r0 + 2)) & 0xC0C0C0C0u;
    }
    const long A = (long)(((uint64_t)hi << 32) | lo);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const long B = (long)(((uint64_t)o.b[2 * n + 1] << 32) | o.b[2 * n]);
        c[n] = __builtin_amdgcn_mfma_i32_16x16x32_i8(A, B, i32x4{0, 0, 0, 0}, 0, 0, 0);
    }
}

template <int BITS, int NT, bool GW>
__device__ __forceinline__ void lean_fold(const LeanOps<BITS, NT, GW>& o, const i32x4 (&c)[NT], float (&acc)[2][4],
                                          const LeanLds<BITS, GW>& S, int buf, int j, int g)
{
    float ws[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (GW) {
        /* the group scales of the lane's rows 4g .. 4g+3 for block j, read at
         * the fold (not carried in the operand ring) */
        const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const float4 v = *reinterpret_cast<const float4*>(&S.ws[buf][j][16 * wv + 4 * g]);
        ws[0] = v.x;
        ws[1] = v.y;
        ws[2] = v.z;
        ws[3] = v.w;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            /* GW: the coefficient is the fp32 product of the row's group scale
             * and the token's block scale (times 2^-(8-b), exactly) */
            const float coef = GW ? ws[v] * o.d[n] : o.d[n];
            acc[n][v] = __builtin_fmaf(coef, (float)c[n][v], acc[n][v]);
            if constexpr (GW)
                asm volatile("" : "+v"(acc[n][v])); /* keeps each block's fold in place */
        }
}

/* One K step, software-pipelined over its blocks: while block j
 * multiplies, the operands of block j + 1 are read and block j - 1 is
 * folded, so neither an LDS read nor an MFMA result is waited for right
 * before its use. */
template <int BITS, int NT, bool GW>
__device__ __forceinline__ void lean_step(const LeanLds<BITS, GW>& S, int buf, float (&acc)[2][4], const FfnArgs& a,
                                          const MDbg& m, int st)
{
    using C = Cfg<BITS>;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const uint32_t* arow = &S.a[buf][(16 * wv + r) * LCfg<BITS>::kStride];
    LeanOps<BITS, NT, GW> o[3];
    i32x4 c[2][NT];
    lean_read<BITS, NT, GW>(S, buf, 0, arow, r, g, o[0]);
#pragma unroll
    for (int j = 0; j <= C::kStep; ++j) {
        if (j + 1 < C::kStep)
            lean_read<BITS, NT, GW>(S, buf, j + 1, arow, r, g, o[(j + 1) % 3]);
        __builtin_amdgcn_sched_barrier(0);
        if (j < C::kStep) {
            lean_mfma<BITS, NT, GW>(o[j % 3], g, c[j & 1]);
#pragma unroll
            for (int n = 0; n < NT; ++n)
                mdbg(a, m, c[j & 1][n], n, st * C::kStep + j, 8 - BITS);
        }
        if (j >= 1)
            lean_fold<BITS, NT, GW>(o[(j - 1) % 3], c[(j - 1) & 1], acc, S, buf, j - 1, g);
        __builtin_amdgcn_sched_barrier(0);
    }
}

/* Two steps of loads in registers (stage k holds the steps = k mod 2), one
 * in LDS, one barrier per step; the loop body covers two steps so that
 * stage and LDS buffer indices are compile-time.  (Three or four steps in
 * registers lowered the occupancy and were slower.)  Returns true
 * (uniformly) when some step's scales were not exact with the 2^-(8-b)
 * factor taken out; acc is then void. */
template <int BITS, int NT, bool GW>
__device__ __forceinline__ bool k_loop_lean(LeanLds<BITS, GW>& S, const LeanLane& L, float (&acc)[2][4],
                                            const FfnArgs& a, const MDbg& m)
{
    constexpr int D = 2, U = 2;
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            acc[n][v] = 0.0f;
    LeanStage<BITS, GW> P[D];
#pragma unroll
    for (int k = 0; k < D; ++k)
        lean_fetch<BITS, NT, GW>(P[k], L, k);
    bool bad = lean_commit<BITS, NT, GW>(P[0], S, 0);
    lean_fetch<BITS, NT, GW>(P[0], L, D);
    __syncthreads();
#pragma unroll 1
    for (int st = 0; st < L.nsteps; st += U) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int s = st + i;
            lean_step<BITS, NT, GW>(S, i & 1, acc, a, m, s);
            bad |= lean_commit<BITS, NT, GW>(P[(i + 1) % D], S, (i + 1) & 1);
            lean_fetch<BITS, NT, GW>(P[(i + 1) % D], L, s + 1 + D);
            __syncthreads();
        }
    }
    /* the workgroup's OR of bad, through four words of the block-scale
     * buffers (free after the last step's barrier): no LDS of its own, which
     * keeps the grouped int4 kernels at four workgroups per CU */
    int* red = reinterpret_cast<int*>(&S.ds[0][0][0][0]);
    const bool wbad = __ballot(bad) != 0;
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = wbad ? 1 : 0;
    __syncthreads();
    const bool any = (red[0] | red[1] | red[2] | red[3]) != 0;
    __syncthreads();
    return any;
}

template <int BITS, bool GW>
__device__ __forceinline__ bool mfma_k_loop_lean(LeanLds<BITS, GW>& S, const LeanLane& L, int ntiles,
                                                 float (&acc)[2][4], const FfnArgs& a, const MDbg& m)
{
    if (ntiles > 1)
        return k_loop_lean<BITS, 2, GW>(S, L, acc, a, m);
    return k_loop_lean<BITS, 1, GW>(S, L, acc, a, m);
}

} // namespace

/* GROUPED: a launch whose segments may hold group-wise scales (a separate
 * instantiation, so that the per-row kernels keep their registers). */
template <int BITS, bool GROUPED>
__global__ __launch_bounds__(256) void ffn_gate_up_mfma(FfnArgs a)
{
    __shared__ MfmaShared<BITS, GROUPED> sm;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int RB = a.I / 32;
    MLoc M;
    if (!locate_m(a, blockIdx.x, RB, M))
        return;
    const FfnSeg sg = pick_m(a, M.seg);
    int e, pos0, ntok;
    if (!munit_info(sg, M.unit, e, pos0, ntok))
        return;
    const int nb = a.H / 32;
    const int64_t rowbytes = (int64_t)a.H * BITS / 8;
    const int gbv = GROUPED ? sg.gu_gb : 0;
    const int ntiles = (ntok + 15) / 16;
    const int r = lane & 15, g = lane >> 4;
    const MDbg md = {sg.out_base + pos0, ntok, 32, kDbgGate, kDbgUp, M.rb * 32, M.rb * 32, a.I};
    float acc[2][4];
    bool general = true;
    {
        /* the aligned loop, while every activation offset fits 31 bits */
        if (lean_shape<BITS>(nb) && (int64_t)sg.S * a.H < (int64_t(1) << 31) && nb < 65536) {
            using LC = LCfg<BITS>;
            LeanLane LL;
            LL.gb = GROUPED ? sg.gu_gb : 0;
            LL.ng = LL.gb ? nb / LL.gb : 1;
            LL.magic = LL.gb > 1 ? 0xFFFFFFFFu / (uint32_t)LL.gb + 1u : 0u;
            {
                /* scale rows: thread l takes row l / 4 (rows 0..31 gate, 32..63 up) */
                const int rowt = (int)threadIdx.x >> 2;
                const bool up = __builtin_amdgcn_readfirstlane(rowt) >= 32;
                LL.wsb = LL.gb ? (up ? sg.up_s : sg.gate_s) + ((int64_t)e * a.I + M.rb * 32) * LL.ng : nullptr;
                LL.wso = (uint32_t)(rowt & 31) * (uint32_t)LL.ng;
            }
#pragma unroll
            for (int i = 0; i < LC::kNL; ++i) {
                /* rows 0..31 are gate rows, 32..63 the same up rows; a load's rows
                 * lie on one side within each wave */
                const int row = i * LC::kRowsPerLoad + (int)threadIdx.x / LC::kCR;
                const bool up = __builtin_amdgcn_readfirstlane(row) >= 32;
                LL.wb[i] = (up ? sg.up_w : sg.gate_w) + ((int64_t)e * a.I + M.rb * 32) * rowbytes;
                LL.wo[i] = (uint32_t)(row & 31) * (uint32_t)rowbytes + 16u * (uint32_t)(threadIdx.x % LC::kCR);
            }
            if constexpr (LC::kNL == 1) {
                LL.wb[1] = LL.wb[0];
                LL.wo[1] = LL.wo[0];
            }
            LL.x = a.xq;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tt = (i < LC::kNXL ? i : 0) * LC::kTokPerLoad + (int)threadIdx.x / LC::kXC;
                const int tk = token_of_m(sg, pos0 + (tt < ntok ? tt : 0));
                LL.xo[i] = (uint32_t)tk * (uint32_t)a.H + 16u * (uint32_t)(threadIdx.x % LC::kXC);
            }
            LL.xd = a.xd;
            {
                const int td = lean_d_token<BITS>();
                const int tk = token_of_m(sg, pos0 + (td < ntok ? td : 0));
                LL.dof = (uint32_t)tk * (uint32_t)nb + (uint32_t)lean_d_block<BITS>();
            }
            LL.nsteps = nb / Cfg<BITS>::kStep;
            general = mfma_k_loop_lean<BITS, GROUPED>(sm.l, LL, ntiles, acc, a, md);
        }
    }
    if (general) {
        /* load lanes: row dot l >> 2 (gate rows 0..31, then the same up rows)
         * and token l & 31 (tokens past the unit load its first token); set up
         * here, so that nothing of it is live across the aligned loop */
        const int rd = threadIdx.x >> 2, tl = threadIdx.x & 31;
        LoadLane L;
        L.wrow = (rd < 32 ? sg.gate_w : sg.up_w) + ((int64_t)e * a.I + M.rb * 32 + (rd & 31)) * rowbytes;
        const int tok = token_of_m(sg, pos0 + (tl < ntok ? tl : 0));
        L.xrow = a.xq + (int64_t)tok * a.H;
        L.xdrow = a.xd + (int64_t)tok * nb;
        L.nb = nb;
        L.gb = gbv;
        L.wsrow = L.gb ? (rd < 32 ? sg.gate_s : sg.up_s) + ((int64_t)e * a.I + M.rb * 32 + (rd & 31)) * (nb / L.gb)
                       : nullptr;
        mfma_k_loop<BITS, GROUPED>(sm.k, L, ntiles, acc, a, md);
    }

    /* epilogue: scaled g (row dots 0..31) and u (32..63) through LDS, then
     * h = silu(g) * u and one Q8_0 block of h per token */
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int rdot = 16 * wv + 4 * g + v;
        const float sc =
            gbv ? 1.0f : (rdot < 32 ? sg.gate_s : sg.up_s)[(int64_t)e * a.I + M.rb * 32 + (rdot & 31)];
#pragma unroll
        for (int n = 0; n < 2; ++n)
            if (n < ntiles)
                sm.e.v[rdot][16 * n + r] = sc * acc[n][v];
    }
    __syncthreads();
    /* thread: token t, elements 4q .. 4q+3 of the h block */
    const int t = threadIdx.x >> 3, q = threadIdx.x & 7;
    float h[4];
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float gv = sm.e.v[4 * q + i][t];
        const float uv = sm.e.v[32 + 4 * q + i][t];
        h[i] = canon_silu(gv) * uv;
        am = fmaxf(am, __builtin_fabsf(h[i]));
    }
    am = fmaxf(am, shfl_xor(am, 1));
    am = fmaxf(am, shfl_xor(am, 2));
    am = fmaxf(am, shfl_xor(am, 4));
    if (t < ntok) {
        const float dsc = am / 127.0f;
        const float inv = (am == 0.0f) ? 0.0f : 1.0f / dsc;
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            word |= (uint32_t)(q8_code(h[i], inv) & 0xFF) << (8 * i);
        const int64_t row_out = sg.out_base + pos0 + t;
        *reinterpret_cast<uint32_t*>(a.hq + row_out * a.I + M.rb * 32 + 4 * q) = word;
        if (q == 0)
            a.hd[row_out * (a.I / 32) + M.rb] = dsc;
    }
}

template <int BITS, bool GROUPED>
__global__ __launch_bounds__(256) void ffn_down_mfma(FfnArgs a)
{
    __shared__ MfmaShared<BITS, GROUPED> sm;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int RB = (a.H + 63) / 64;
    MLoc M;
    if (!locate_m(a, blockIdx.x, RB, M))
        return;
    const FfnSeg sg = pick_m(a, M.seg);
    int e, pos0, ntok;
    if (!munit_info(sg, M.unit, e, pos0, ntok))
        return;
    const int nb = a.I / 32;
    const int64_t rowbytes = (int64_t)a.I * BITS / 8;
    const int gbv = GROUPED ? sg.d_gb : 0;
    const int ntiles = (ntok + 15) / 16;
    const int r = lane & 15, g = lane >> 4;
    const MDbg md = {sg.out_base + pos0, ntok, 64, kDbgDown, kDbgDown, M.rb * 64, M.rb * 64, a.H};
    float acc[2][4];
    bool general = true;
    {
        /* the aligned loop, while the weight offsets in one matrix fit 31 bits */
        if (lean_shape<BITS>(nb) && (int64_t)a.H * rowbytes < (int64_t(1) << 31) && nb < 65536) {
            using LC = LCfg<BITS>;
            const int64_t r0 = sg.out_base + pos0;
            LeanLane LL;
            LL.gb = GROUPED ? sg.d_gb : 0;
            LL.ng = LL.gb ? nb / LL.gb : 1;
            LL.magic = LL.gb > 1 ? 0xFFFFFFFFu / (uint32_t)LL.gb + 1u : 0u;
            {
                /* scale rows: thread l takes row l / 4 of the workgroup's 64 */
                const int rw = M.rb * 64 + ((int)threadIdx.x >> 2);
                LL.wsb = LL.gb ? sg.down_s + (int64_t)e * a.H * LL.ng : nullptr;
                LL.wso = (uint32_t)(rw < a.H ? rw : a.H - 1) * (uint32_t)LL.ng;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int rw = M.rb * 64 + (i < LC::kNL ? i : 0) * LC::kRowsPerLoad + (int)threadIdx.x / LC::kCR;
                LL.wb[i] = sg.down_w + (int64_t)e * a.H * rowbytes;
                LL.wo[i] = (uint32_t)(rw < a.H ? rw : 0) * (uint32_t)rowbytes + 16u * (uint32_t)(threadIdx.x % LC::kCR);
            }
            LL.x = a.hq + r0 * a.I;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int tt = (i < LC::kNXL ? i : 0) * LC::kTokPerLoad + (int)threadIdx.x / LC::kXC;
                LL.xo[i] = (uint32_t)(tt < ntok ? tt : 0) * (uint32_t)a.I + 16u * (uint32_t)(threadIdx.x % LC::kXC);
            }
            LL.xd = a.hd + r0 * nb;
            {
                const int td = lean_d_token<BITS>();
                LL.dof = (uint32_t)(td < ntok ? td : 0) * (uint32_t)nb + (uint32_t)lean_d_block<BITS>();
            }
            LL.nsteps = nb / Cfg<BITS>::kStep;
            general = mfma_k_loop_lean<BITS, GROUPED>(sm.l, LL, ntiles, acc, a, md);
        }
    }
    if (general) {
        /* load lanes (set up here: nothing of it is live across the aligned loop) */
        const int rd = threadIdx.x >> 2, tl = threadIdx.x & 31;
        const int row = M.rb * 64 + rd;
        LoadLane L;
        L.wrow = sg.down_w + ((int64_t)e * a.H + (row < a.H ? row : 0)) * rowbytes;
        const int64_t row_in = sg.out_base + pos0 + (tl < ntok ? tl : 0);
        L.xrow = a.hq + row_in * a.I;
        L.xdrow = a.hd + row_in * nb;
        L.nb = nb;
        L.gb = gbv;
        L.wsrow = L.gb ? sg.down_s + ((int64_t)e * a.H + (row < a.H ? row : 0)) * (nb / L.gb) : nullptr;
        mfma_k_loop<BITS, GROUPED>(sm.k, L, ntiles, acc, a, md);
    }

    const int n0 = M.rb * 64 + 16 * wv + 4 * g;
    float sc[4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
        sc[v] = n0 + v < a.H ? (gbv ? 1.0f : sg.down_s[(int64_t)e * a.H + n0 + v]) : 0.0f;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int t = 16 * n + r;
        if (n < ntiles && t < ntok) {
            float* yr = a.y + (int64_t)(sg.out_base + pos0 + t) * a.H + n0;
            if (n0 + 3 < a.H && (a.H & 3) == 0) {
                *reinterpret_cast<float4*>(yr) =
                    make_float4(sc[0] * acc[n][0], sc[1] * acc[n][1], sc[2] * acc[n][2], sc[3] * acc[n][3]);
            } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (n0 + v < a.H)
                        yr[v] = sc[v] * acc[n][v];
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
    const bool grouped = a.seg[0].gu_gb != 0 || (a.nseg > 1 && a.seg[1].gu_gb != 0);
    switch (bits * 2 + (grouped ? 1 : 0)) {
    case 16: hipLaunchKernelGGL((ffn_gate_up_mfma<8, false>), grid, block, 0, st, a); break;
    case 17: hipLaunchKernelGGL((ffn_gate_up_mfma<8, true>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((ffn_gate_up_mfma<4, false>), grid, block, 0, st, a); break;
    case 9: hipLaunchKernelGGL((ffn_gate_up_mfma<4, true>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((ffn_gate_up_mfma<2, false>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((ffn_gate_up_mfma<2, true>), grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_ffn_down_mfma(const FfnArgs& a, int32_t bits, hipStream_t st)
{
    const int64_t jobs = total_mjobs(a, (a.H + 63) / 64);
    if (jobs == 0)
        return hipSuccess;
    const dim3 grid((uint32_t)jobs), block(256);
    const bool grouped = a.seg[0].d_gb != 0 || (a.nseg > 1 && a.seg[1].d_gb != 0);
    switch (bits * 2 + (grouped ? 1 : 0)) {
    case 16: hipLaunchKernelGGL((ffn_down_mfma<8, false>), grid, block, 0, st, a); break;
    case 17: hipLaunchKernelGGL((ffn_down_mfma<8, true>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((ffn_down_mfma<4, false>), grid, block, 0, st, a); break;
    case 9: hipLaunchKernelGGL((ffn_down_mfma<4, true>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((ffn_down_mfma<2, false>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((ffn_down_mfma<2, true>), grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}

} // namespace coli
