/*
 * ffn_gemv.hip -- gated expert FFN on the integer dot path, GEMV form, for
 * experts that hold few tokens of a batch: one-token decode, batches of up to
 * 8 tokens (verify steps), and the experts below the matrix-core threshold
 * in batches that average fewer than 8 tokens per expert.
 *
 * ("Show HN: 如何在我的低配置电脑上运行 GLM-5.2": implemented-features section,
 * integer dot-product item -- Q8_0-style int8 activations -- and quantised-
 * kernel item -- int8 / packed int4 / packed int2 weights, per-row scales,
 * dequantised on use; Metal section: the routed-expert work is a SwiGLU;
 * resource-policy section: gate and up share one dispatch.)
 *
 * A job is one expert, up to kUnitTokens of its tokens and 64 weight rows
 * (gate/up: 32 gate rows and the same 32 up rows, i.e. exactly one 32-block
 * of h; down: 64 output rows), run by a workgroup of four waves; wave w owns
 * 16 whole rows.
 *
 * Loads.  A wave reads its 16 rows in items of two rows by 32 blocks: lane l
 * of item (chunk i, pair p) loads block 32 i + (l mod 32) of row 2p + l/32,
 * so each half wave reads 32 consecutive blocks of one row (512 bytes at
 * int4: whole cache lines).  Items run chunk by chunk -- the eight pairs of
 * chunk 0, then those of chunk 1, ... -- with 2 NI items in flight (NI: the
 * chunks of a row).  Reading whole row spans per instruction streams
 * markedly faster than splitting K across the waves of a job (measured 6.5
 * against 5.5 TB/s on 113 MB).
 *
 * Fold.  Each exact int32 block partial goes to LDS as an fp32 number (exact:
 * |S_b| < 2^20).  After the eight items of a chunk, lane (row, token)
 * continues its row's chain acc = fma(d_b, (float)S_b, acc) over the chunk's
 * 32 blocks in ascending order -- the canonical fold: one chain from +0 over
 * all blocks of the row -- while the next chunk's items load; the row scale
 * multiplies at the end.  Blocks past the row's end hold partial 0 and scale
 * 0, and fma(0, 0, acc) == acc for every value such a chain can hold (it
 * starts at +0 and cannot reach -0), so a ragged last chunk needs no branch.
 *
 * Epilogue of the gate/up kernels: g = row scale * acc (lanes of the 32
 * gate rows), u (the same up rows), h = silu(g) * u, one Q8_0 block of h
 * per token (amax over 32 lanes), codes and scale stored for the down
 * kernels.
 */
#include "device_common.h"
#include "kernels.h"
#include "select.h"

namespace coli {

namespace {

constexpr int kRowsPerJob = 64;
constexpr int kJobWaves = 4;  /* waves of a GEMV workgroup */
constexpr int kWaveRows = 16; /* rows of a job per wave */
constexpr int kChunk = 32;    /* blocks of a row per load item */
constexpr int kTile = kWaveRows * kChunk; /* words of one token's partial tile */

struct JobLoc {
    int seg, unit, rb;
};

/* Matrix index of routed expert id (0 <= id < E) in seg[0]'s banks: the id
 * itself, or its slot in a tiered layer's slot bank; clamped to the bank. */
__device__ __forceinline__ int decode_matrix(const int32_t* slot_of, int id, int E, int n_mat)
{
    const int m = slot_of ? slot_of[min(max(id, 0), E - 1)] : id;
    return min(max(m, 0), n_mat - 1);
}

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

/* int8 chunks (32 blocks of 32 bytes: 1 KB of a row) are loaded in halves
 * of blocks: lane c (of the row's 32 lanes) takes half c & 1 of blocks
 * c >> 1 and 16 + (c >> 1), so that each of its two load instructions reads
 * 512 contiguous bytes of the row (every cache line once; whole blocks per
 * lane would request each line from both instructions).  Blocks past the
 * row's nb read its last block (in bounds; their partials are discarded).
 * The lane then owns one block of the chunk, own8(c). */
/* The split layout is used for int8 rows of four chunks or more (a job's
 * NI): shorter rows have too few blocks per chunk for it to pay (measured
 * slower on rows of one and two chunks). */
template <int BITS, int NI>
constexpr bool kSplit8 = BITS == 8 && NI >= 4;

__device__ __forceinline__ int own8(int c)
{
    return (c & 1) ? 16 + (c >> 1) : (c >> 1);
}

__device__ __forceinline__ void load_chunk8(const uint8_t* row, int chunk0, int c, int nb, uint32_t (&w)[8])
{
    const int b0 = min(chunk0 + (c >> 1), nb - 1), b1 = min(chunk0 + 16 + (c >> 1), nb - 1);
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + b0 * 32 + 16 * (c & 1)));
    const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + b1 * 32 + 16 * (c & 1)));
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

/* The activation words matching load_chunk8's pieces: half c & 1 of blocks
 * chunk0 + (c >> 1) and chunk0 + 16 + (c >> 1) of a staged [block][8] array. */
__device__ __forceinline__ void act_chunk8(const uint32_t* xb, int chunk0, int c, int nb, uint32_t (&x)[8])
{
    const int b0 = min(chunk0 + (c >> 1), nb - 1), b1 = min(chunk0 + 16 + (c >> 1), nb - 1);
    const uint4 u0 = *reinterpret_cast<const uint4*>(xb + b0 * 8 + 4 * (c & 1));
    const uint4 u1 = *reinterpret_cast<const uint4*>(xb + b1 * 8 + 4 * (c & 1));
    x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w;
    x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
}

/* The exact int32 partial of the lane's own block (own8(c)): each half's
 * four byte dots, plus the other half's from the partner lane c ^ 1 (every
 * lane of the wave takes part). */
__device__ __forceinline__ int32_t dot_chunk8(const uint32_t (&w)[8], const uint32_t (&x)[8], int c)
{
    int32_t s0 = 0, s1 = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        s0 = COLI_SDOT4(w[k], x[k], s0);
        s1 = COLI_SDOT4(w[4 + k], x[4 + k], s1);
    }
    s0 += shfl_xor_i(s0, 1);
    s1 += shfl_xor_i(s1, 1);
    return (c & 1) ? s1 : s0;
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

/* Word of partial (row k of the wave's 16, block c of the chunk) in a
 * token's [16][32] tile.  The quads of a row are XOR-permuted by k / 2, so
 * an item's writes (rows 2p and 2p + 1: two 32-word runs) and the fold's
 * quad reads (16 rows, one quad each) both fall on distinct banks. */
__device__ __forceinline__ int ptile(int k, int c)
{
    return k * kChunk + ((((c >> 2) ^ (k >> 1)) & 7) << 2) + (c & 3);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

/* Continues a row's chain over the 32 blocks of one chunk, in ascending
 * order: acc = fma(d_c, S_c, acc).  tile: the token's partial tile (row k);
 * dc: the chunk's 32 block scales (16-byte aligned).  The quad reads run
 * kFoldAhead quads ahead of the fmas.  An empty asm statement that uses
 * acc and may touch memory pins each quad's fmas and reads in place:
 * otherwise the compiler sinks every fma of the loop to its end (the chain
 * is needed only there) and keeps all the chunks' operands live. */
constexpr int kFoldAhead = 3;

__device__ __forceinline__ float fold_chunk(const float* tile, int k, const float* dc, float acc)
{
    const float* row = tile + k * kChunk;
    const int sw = (k >> 1) & 7;
    f32x4 s[8], d[8];
#pragma unroll
    for (int q = 0; q < kFoldAhead; ++q) {
        s[q] = *reinterpret_cast<const f32x4*>(row + ((q ^ sw) << 2));
        d[q] = *reinterpret_cast<const f32x4*>(dc + 4 * q);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        if (q + kFoldAhead < 8) {
            s[q + kFoldAhead] = *reinterpret_cast<const f32x4*>(row + (((q + kFoldAhead) ^ sw) << 2));
            d[q + kFoldAhead] = *reinterpret_cast<const f32x4*>(dc + 4 * (q + kFoldAhead));
        }
        acc = __builtin_fmaf(d[q].x, s[q].x, acc);
        acc = __builtin_fmaf(d[q].y, s[q].y, acc);
        acc = __builtin_fmaf(d[q].z, s[q].z, acc);
        acc = __builtin_fmaf(d[q].w, s[q].w, acc);
        asm volatile("" : "+v"(acc) : : "memory");
    }
    return acc;
}

/* The same with group-wise weight scales: block b's coefficient is the fp32
 * product of the row's group scale and d_b.  wtile holds the chunk's scale
 * of every (row, block), laid out as the partial tile (ptile), so its quad
 * reads are conflict-free like the partials'. */
__device__ __forceinline__ float fold_chunk_grouped(const float* tile, int k, const float* dc, float acc,
                                                    const float* wtile)
{
    const float* row = tile + k * kChunk;
    const float* wrow = wtile + k * kChunk;
    const int sw = (k >> 1) & 7;
    f32x4 s[8], d[8];
#pragma unroll
    for (int q = 0; q < kFoldAhead; ++q) {
        s[q] = *reinterpret_cast<const f32x4*>(row + ((q ^ sw) << 2));
        d[q] = *reinterpret_cast<const f32x4*>(dc + 4 * q);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        if (q + kFoldAhead < 8) {
            s[q + kFoldAhead] = *reinterpret_cast<const f32x4*>(row + (((q + kFoldAhead) ^ sw) << 2));
            d[q + kFoldAhead] = *reinterpret_cast<const f32x4*>(dc + 4 * (q + kFoldAhead));
        }
        /* the coefficients of quad q, formed before its chain steps */
        const f32x4 w = *reinterpret_cast<const f32x4*>(wrow + ((q ^ sw) << 2));
        const float c0 = w.x * d[q].x, c1 = w.y * d[q].y, c2 = w.z * d[q].z, c3 = w.w * d[q].w;
        acc = __builtin_fmaf(c0, s[q].x, acc);
        acc = __builtin_fmaf(c1, s[q].y, acc);
        acc = __builtin_fmaf(c2, s[q].z, acc);
        acc = __builtin_fmaf(c3, s[q].w, acc);
        asm volatile("" : "+v"(acc) : : "memory"); /* as in fold_chunk */
    }
    return acc;
}

/* The group-wise scales of chunk i for a wave's scale tile: lane l takes
 * row l mod 16 (clamped to the rows that exist; ws: the scales of the
 * wave's row 0, ng per row) and blocks 8 (l / 16) .. + 7 of the chunk
 * (block b's scale is the one of group b / gb; blocks past the row take
 * its last one, their d is 0).  Loaded at the chunk's start, stored into
 * the tile before its fold. */
struct ChunkScales {
    float v[8];
};

__device__ __forceinline__ void chunk_scales_load(ChunkScales& S, const float* ws, int ng, int gb, int rows_ok,
                                                  int i, int lane)
{
    /* the lane index through an empty asm, so that the address work of each
     * chunk stays at its chunk instead of being hoisted to the kernel's top
     * and held in registers for every chunk */
    if (gb == 0) {
        /* per-row scales in a grouped launch: coefficient 1 * d_b = d_b */
#pragma unroll
        for (int j = 0; j < 8; ++j)
            S.v[j] = 1.0f;
        return;
    }
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const uint32_t r = (uint32_t)min(ln & 15, max(rows_ok, 1) - 1);
    const int b0 = kChunk * i + 8 * (ln >> 4);
    int g = b0 / gb, rem = b0 - g * gb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        S.v[j] = ws[r * (uint32_t)ng + (uint32_t)min(g, ng - 1)];
        if (++rem == gb) {
            rem = 0;
            ++g;
        }
    }
}

__device__ __forceinline__ void chunk_scales_store(const ChunkScales& S, float* wtile, int lane)
{
    const int r = lane & 15, c0 = 8 * (lane >> 4);
#pragma unroll
    for (int h = 0; h < 2; ++h)
        *reinterpret_cast<f32x4*>(wtile + ptile(r, c0 + 4 * h)) =
            f32x4{S.v[4 * h], S.v[4 * h + 1], S.v[4 * h + 2], S.v[4 * h + 3]};
}

/* Chunks per row for nb blocks, rounded up to an instantiated count. */
inline int gemv_ni(int nb)
{
    const int n = (nb + kChunk - 1) / kChunk;
    return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : n <= 6 ? 6 : 8;
}

/* One load item of a lane: BITS words of one weight block. */
template <int BITS>
struct Item {
    uint32_t w[BITS];
};

/* Items in flight: 2 NI (two chunks' worth at NI = 4 and below). */
template <int BITS, int NI>
struct Ring {
    Item<BITS> it[2 * NI];
};

/* Loads item n = (chunk n / 8, pair n % 8) of a wave's 16 rows: rows0 is
 * row 0 (uniform); rows8, when not null, is where rows 8.. start instead of
 * right after row 7 (then all 16 rows exist).  A load takes the uniform base
 * plus a 32-bit lane offset (16 rows of at most 8 KB).  Loads are
 * unconditional: a lane past the rows or the row's blocks reads the last
 * existing row / block instead (in bounds; its partial is never folded), so
 * no load sits under a branch and each use waits only for its own item. */
template <int BITS, int NI>
__device__ __forceinline__ void item_load(Item<BITS>& W, const uint8_t* rows0, uint32_t rowbytes, int n,
                                          int rows_ok, int nb, const uint8_t* rows8)
{
    const int lane = threadIdx.x & 63;
    const bool hi = rows8 && (n & 7) >= 4; /* uniform */
    const int row = min(2 * (n & 7) + (lane >> 5), max(rows_ok, 1) - 1) - (hi ? 8 : 0);
    if constexpr (kSplit8<BITS, NI>) {
        load_chunk8((hi ? rows8 : rows0) + (uint32_t)row * rowbytes, kChunk * (n >> 3), lane & 31, nb, W.w);
    } else {
        const uint32_t off = (uint32_t)row * rowbytes +
                             (uint32_t)min(kChunk * (n >> 3) + (lane & 31), nb - 1) * (uint32_t)(4 * BITS);
        load_block<BITS>((hi ? rows8 : rows0) + off, W.w);
    }
}

/* Issues the first 2 NI items (before the activations are staged, so the
 * weight stream starts first). */
template <int BITS, int NI>
__device__ __forceinline__ void ring_start(Ring<BITS, NI>& R, const uint8_t* rows0, uint32_t rowbytes, int rows_ok,
                                           int nb, const uint8_t* rows8 = nullptr)
{
#pragma unroll
    for (int n = 0; n < 2 * NI; ++n)
        item_load<BITS, NI>(R.it[n], rows0, rowbytes, n, rows_ok, nb, rows8);
}

/* ---- one token ------------------------------------------------------------
 * Unit u < k is the expert of selection slot u, unit k the shared expert;
 * hq / hd / y row u belongs to unit u, so the combine reads y in slot order.
 * The gate/up kernel selects the experts itself: wave 0 of every routed job
 * runs the top-k over the token's logits (the same selection as
 * router_select_kernel), so no workgroup waits for another, and the first
 * routed job stores ids and weights; meanwhile the other waves stage the
 * token's activation blocks (operand order) and block scales in LDS.
 *
 * (A combine inside the down kernel -- the last unit to finish a row block
 * adding the others' rows -- needs a device-scope release per workgroup,
 * which on this chip writes back the XCD's L2; measured 3x slower than the
 * separate combine launch.) */

/* Dynamic LDS of the one-token kernels, in words: per wave its partial tile
 * (before the K loop wave 0's selection scratch), then the token's
 * activation blocks [32 NI][8] and block scales [32 NI] (zero past nb), the
 * job's row sums [64] and the selected ids [64]. */
__host__ __device__ inline int dec_region()
{
    return kTile > kSelScratch ? kTile : kSelScratch;
}

__host__ __device__ inline int dec_dlen(int nb)
{
    const int n = (nb + kChunk - 1) / kChunk;
    return kChunk * (n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : n <= 6 ? 6 : 8);
}

/* A wave's LDS region; with group-wise scales it also holds the chunk's
 * weight-scale tile (16 rows x 32 blocks, after the partial tile). */
__host__ __device__ inline int dec_region_g(bool grouped)
{
    return grouped ? (dec_region() > 2 * kTile ? dec_region() : 2 * kTile) : dec_region();
}

__host__ __device__ inline size_t dec_lds_bytes(int nb, bool grouped)
{
    return (size_t)(kJobWaves * dec_region_g(grouped) + 9 * dec_dlen(nb) + 64 + 64) * 4;
}

/* Output row, matrix kind and weight rows of a wave's rows 0..7 and 8..15,
 * for the test-only partial dump. */
struct DbgRows {
    int64_t o;
    int kind0, row0, kind8, row8;
};

/* The wave's 16 rows against one token (xal, dl: its staged activation
 * blocks and block scales); R holds items 0 .. 2NI - 1.  Returns on every
 * lane the chain of row (lane mod 16), before the row scale.  P: the wave's
 * partial tile.  GROUPED: ws0 holds the group-wise scales of the wave's
 * row 0 (rows nb / gb apart). */
template <int BITS, int NI, bool GROUPED>
__device__ __forceinline__ float dec_k_loop(Ring<BITS, NI>& R, const uint8_t* rows0, uint32_t rowbytes, int rows_ok,
                                            int nb, const uint32_t* xal, float* P, const float* dl,
                                            const float* ws0, int gb, const FfnArgs& a, const DbgRows& dr,
                                            const uint8_t* rows8 = nullptr)
{
    constexpr int D = 2 * NI, N = 8 * NI;
    const int lane = threadIdx.x & 63, c = lane & 31, k = lane & 15;
    const int ng = GROUPED && gb ? nb / gb : 0;
    float* W = P + kTile; /* GROUPED: the chunk's scale tile */
    ChunkScales CS;
    float acc = 0.0f;
    uint32_t xa[8];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const int i = n >> 3, p = n & 7;
        if (p == 0) {
            /* the lane's activation block of this chunk (int8: the halves
             * matching its weight pieces) */
            if constexpr (kSplit8<BITS, NI>) {
                act_chunk8(xal, kChunk * i, c, nb, xa);
            } else {
                const uint4* src = reinterpret_cast<const uint4*>(xal + (kChunk * i + c) * 8);
                const uint4 u0 = src[0], u1 = src[1];
                xa[0] = u0.x; xa[1] = u0.y; xa[2] = u0.z; xa[3] = u0.w;
                xa[4] = u1.x; xa[5] = u1.y; xa[6] = u1.z; xa[7] = u1.w;
            }
        }
        if constexpr (GROUPED) {
            if (p == 4) /* four items before the fold: late enough to hold few registers */
                chunk_scales_load(CS, ws0, ng, gb, rows_ok, i, lane);
        }
        int32_t s;
        if constexpr (kSplit8<BITS, NI>)
            s = dot_chunk8(R.it[n % D].w, xa, c);
        else
            s = block_dot<BITS>(R.it[n % D].w, xa);
        const int cb = kSplit8<BITS, NI> ? own8(c) : c; /* the lane's block of the chunk */
        const int row = 2 * p + (lane >> 5);
        P[ptile(row, cb)] = kChunk * i + cb < nb ? (float)s : 0.0f;
        if (row < rows_ok && kChunk * i + cb < nb)
            dbg_partial(a, row < 8 ? dr.kind0 : dr.kind8, dr.o, row < 8 ? dr.row0 + row : dr.row8 + row - 8,
                        kChunk * i + cb, s);
        if (n + D < N) /* resolved at compile time */
            item_load<BITS, NI>(R.it[n % D], rows0, rowbytes, n + D, rows_ok, nb, rows8);
        if (p == 7) {
            if constexpr (GROUPED)
                chunk_scales_store(CS, W, lane);
            wave_lds_sync();
            if constexpr (GROUPED)
                acc = fold_chunk_grouped(P, k, dl + kChunk * i, acc, W);
            else
                acc = fold_chunk(P, k, dl + kChunk * i, acc);
            wave_lds_sync(); /* the chunk's partials are read before the next chunk's overwrite them */
        }
    }
    return acc;
}

/* Stages the token's activation blocks (operand order) and block scales:
 * thread `tid` of `nthr` takes blocks tid, tid + nthr, ...; blocks past nb
 * get scale 0 (their codes are never used).  The caller synchronises. */
template <int BITS>
__device__ __forceinline__ void dec_stage(const int8_t* act, const float* scl, int nb, int dlen, int tid, int nthr,
                                          uint32_t* xal, float* dl)
{
    for (int b0 = tid; b0 < dlen; b0 += 2 * nthr) {
        /* two blocks' loads in flight before either is converted */
        uint32_t x[2][8];
        float dv[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int b = min(b0 + r * nthr, nb - 1);
            load_codes(act + (int64_t)b * 32, x[r]);
            dv[r] = scl[b];
        }
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int b = b0 + r * nthr;
            if (b < dlen) {
                uint32_t xa[8];
                prep_dot<BITS>(x[r], xa);
                uint4* dst = reinterpret_cast<uint4*>(xal + b * 8);
                dst[0] = make_uint4(xa[0], xa[1], xa[2], xa[3]);
                dst[1] = make_uint4(xa[4], xa[5], xa[6], xa[7]);
                dl[b] = b < nb ? dv[r] : 0.0f;
            }
        }
    }
}

} // namespace

/* GROUPED: a launch whose segments may hold group-wise scales (a separate
 * instantiation, so that the per-row kernels carry no grouped fold). */
template <int BITS, int NI, bool GROUPED>
__global__ __launch_bounds__(256) void ffn_gate_up_decode(DecodeArgs d)
{
    extern __shared__ __attribute__((aligned(16))) int32_t dec_lds[];
    const FfnArgs& a = d.f;
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int RB = a.I / 32;
    const int nb = a.H / 32, region = dec_region_g(GROUPED), dlen = kChunk * NI;
    float* P = reinterpret_cast<float*>(dec_lds + wv * region);
    uint32_t* xal = reinterpret_cast<uint32_t*>(dec_lds + kJobWaves * region);
    float* dl = reinterpret_cast<float*>(xal + 8 * dlen);
    float* rsum = dl + dlen;
    int32_t* sel_ids = reinterpret_cast<int32_t*>(rsum + 64); /* read by every wave after the barrier */
    const uint32_t rowbytes = (uint32_t)a.H * BITS / 8;
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
        Ring<BITS, NI> R;
        ring_start<BITS, NI>(R, g0, rowbytes, kWaveRows, nb, u0);
        const int r = lane & 15;
        const float sc = (r < 8 ? sh.gate_s : sh.up_s)[8 * m + (r & 7)];
        dec_stage<BITS>(a.xq, a.xd, nb, dlen, lane, 64, xal, dl);
        wave_lds_sync();
        const DbgRows dr = {d.k, kDbgGate, 8 * m, kDbgUp, 8 * m};
        const float v16 =
            dec_k_loop<BITS, NI, false>(R, g0, rowbytes, kWaveRows, nb, xal, P, dl, nullptr, 0, a, dr, u0);
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
    int e = 0;
    if (routed) {
        /* wave 0 alone selects (a chain of wave-wide steps, so it runs best
         * without the other waves issuing the same work) while waves 1..3
         * stage the activations; the scratch is wave 0's (not yet used)
         * partial tile */
        float* sel_s = reinterpret_cast<float*>(dec_lds);
        if (wv == 0) {
            const bool store = u == 0 && rb == 0; /* the others need the ids only */
            select_token(d.logits, d.bias, d.E, d.k, d.rsf, store ? d.ids : sel_ids, store ? d.w : nullptr, sel_s,
                         sel_ids, 1, 0, d.opt);
        } else {
            dec_stage<BITS>(a.xq, a.xd, nb, dlen, threadIdx.x - 64, 192, xal, dl);
        }
        __syncthreads();
        const int sel = sel_ids[u];
        if (sel < 0) /* slot dropped by top-p: the whole workgroup leaves */
            return;
        e = decode_matrix(d.slot_of, sel, d.E, sg.n_mat);
    }
    /* waves 0, 1: gate rows rb*32 + 16w ..; waves 2, 3: the same up rows */
    const uint8_t* rows0 = (wv < 2 ? sg.gate_w : sg.up_w) +
                           ((int64_t)e * a.I + rb * 32 + 16 * (wv & 1)) * rowbytes;
    Ring<BITS, NI> R;
    ring_start<BITS, NI>(R, rows0, rowbytes, kWaveRows, nb);
    /* the epilogue's row scale (lane: row rb*32 + lane%32 of gate, then up),
     * loaded now so that it is in hand after the K loop */
    const int r = rb * 32 + (lane & 31);
    const float sc = sg.gu_gb ? 1.0f : (lane < 32 ? sg.gate_s : sg.up_s)[(int64_t)e * a.I + r];
    if (!routed) {
        dec_stage<BITS>(a.xq, a.xd, nb, dlen, threadIdx.x, 256, xal, dl);
        __syncthreads();
    }
    const float* ws0 = sg.gu_gb ? (wv < 2 ? sg.gate_s : sg.up_s) +
                                      ((int64_t)e * a.I + rb * 32 + 16 * (wv & 1)) * (nb / sg.gu_gb)
                                : nullptr;
    const int kd = wv < 2 ? kDbgGate : kDbgUp, r16 = rb * 32 + 16 * (wv & 1);
    const DbgRows dr = {u, kd, r16, kd, r16 + 8};
    const float v16 =
        dec_k_loop<BITS, NI, GROUPED>(R, rows0, rowbytes, kWaveRows, nb, xal, P, dl, ws0, sg.gu_gb, a, dr);
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

template <int BITS, int NI, bool GROUPED>
__global__ __launch_bounds__(256) void ffn_down_decode(DecodeArgs d)
{
    extern __shared__ __attribute__((aligned(16))) int32_t dec_lds[];
    const FfnArgs& a = d.f;
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int RB = (a.H + kRowsPerJob - 1) / kRowsPerJob;
    const int nunits = d.k + (a.nseg > 1 ? 1 : 0);
    const int u = blockIdx.x / RB, rb = blockIdx.x - (blockIdx.x / RB) * RB;
    if (u >= nunits)
        return;
    const bool routed = u < d.k;
    if (routed && d.ids[u] < 0) /* slot dropped by top-p */
        return;
    const FfnSeg sg = pick(a, routed ? 0 : 1);
    const int e = routed ? decode_matrix(d.slot_of, d.ids[u], d.E, sg.n_mat) : 0;
    const int nb = a.I / 32, region = dec_region_g(GROUPED), dlen = kChunk * NI;
    float* P = reinterpret_cast<float*>(dec_lds + wv * region);
    uint32_t* xal = reinterpret_cast<uint32_t*>(dec_lds + kJobWaves * region);
    float* dl = reinterpret_cast<float*>(xal + 8 * dlen);
    const int row0 = rb * kRowsPerJob + kWaveRows * wv;
    const int rows_ok = min(kWaveRows, max(0, a.H - row0));
    const uint32_t rowbytes = (uint32_t)a.I * BITS / 8;
    const uint8_t* rows0 = sg.down_w + ((int64_t)e * a.H + min(row0, a.H - 1)) * rowbytes;
    Ring<BITS, NI> R;
    ring_start<BITS, NI>(R, rows0, rowbytes, rows_ok, nb);
    dec_stage<BITS>(a.hq + (int64_t)u * a.I, a.hd + (int64_t)u * nb, nb, dlen, threadIdx.x, 256, xal, dl);
    __syncthreads();
    const float* ws0 = sg.d_gb ? sg.down_s + ((int64_t)e * a.H + min(row0, a.H - 1)) * (nb / sg.d_gb) : nullptr;
    const DbgRows dr = {u, kDbgDown, row0, kDbgDown, row0 + 8};
    const float v = dec_k_loop<BITS, NI, GROUPED>(R, rows0, rowbytes, rows_ok, nb, xal, P, dl, ws0, sg.d_gb, a, dr);
    const int n = row0 + lane;
    if (lane < rows_ok)
        a.y[(int64_t)u * a.H + n] = (sg.d_gb ? 1.0f : sg.down_s[(int64_t)e * a.H + n]) * v;
}

namespace {

/* Items a thread stages per round (loads of all issued before any is converted). */
constexpr int kDcStage = 4;

/* ---- units of up to TMAX tokens --------------------------------------------
 * The unit's activation blocks of every token are staged once per job in
 * LDS in operand order; each item then yields the partials of its two rows
 * for every token of the unit, and lane (row k, token t) runs the chain of
 * (k, t).
 *
 * Dynamic LDS, in words: codes [TMAX][nb][8], block scales [TMAX][32 NI]
 * (zero past nb), per wave the partial tiles [TMAX][16][32], and the job's
 * row values [64][TMAX]. */
/* LDS words of the whole-row kernels: codes [tmax][nb][8], scales
 * [tmax][dlen], per wave tmax partial tiles, the row values [64][tmax], and
 * with group-wise scales per wave a scale tile. */
__host__ __device__ inline size_t rows_lds_words(int nb, int tmax, bool grouped)
{
    return (size_t)tmax * nb * 8 + (size_t)tmax * dec_dlen(nb) + (size_t)kJobWaves * tmax * kTile +
           64 * (size_t)tmax + (grouped ? (size_t)kJobWaves * kTile : 0);
}

constexpr size_t kLdsMax = 160 * 1024; /* LDS of one CU (gfx950) */

/* The wave's 16 rows against the unit's ntok tokens; R holds items
 * 0 .. 2NI - 1.  Returns on lane (k = l mod 16, t = l / 16) the chain of
 * row k for token t (lanes of tokens past ntok hold no value).  xal, dls:
 * the staged codes and scales; P: the wave's TMAX partial tiles. */
template <int BITS, int NI, int TMAX, bool GROUPED>
__device__ __forceinline__ float rows_k_loop(Ring<BITS, NI>& R, const uint8_t* rows0, uint32_t rowbytes, int rows_ok,
                                             int nb, int ntok, const uint32_t* xal, const float* dls, float* P,
                                             const float* ws0, int gb, const FfnArgs& a, int64_t o0, int kind,
                                             int wrow0, float* W)
{
    constexpr int D = 2 * NI, N = 8 * NI;
    const int lane = threadIdx.x & 63, c = lane & 31, k = lane & 15;
    const int tf = min(lane >> 4, TMAX - 1); /* token of the lane's chain */
    const int sd = kChunk * NI;
    const int ng = GROUPED && gb ? nb / gb : 0;
    ChunkScales CS;
    float acc = 0.0f;
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const int i = n >> 3, p = n & 7;
        const int b = kChunk * i + c;
        if constexpr (GROUPED) {
            if (p == 4) /* four items before the fold: late enough to hold few registers */
                chunk_scales_load(CS, ws0, ng, gb, rows_ok, i, lane);
        }
        const int bc = min(b, nb - 1);
        const int cb = kSplit8<BITS, NI> ? own8(c) : c; /* the lane's block of the chunk */
        const int bo = kChunk * i + cb;
        const int w = ptile(2 * p + (lane >> 5), cb);
        /* tokens one at a time (a rolled loop keeps one token's operands live) */
#pragma unroll 1
        for (int t = 0; t < ntok; ++t) {
            int32_t s;
            if constexpr (kSplit8<BITS, NI>) {
                uint32_t xa[8];
                act_chunk8(xal + (int64_t)t * nb * 8, kChunk * i, c, nb, xa);
                s = dot_chunk8(R.it[n % D].w, xa, c);
            } else {
                const uint4* src = reinterpret_cast<const uint4*>(xal + ((int64_t)t * nb + bc) * 8);
                const uint4 u0 = src[0], u1 = src[1];
                const uint32_t xa[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
                s = block_dot<BITS>(R.it[n % D].w, xa);
            }
            P[t * kTile + w] = bo < nb ? (float)s : 0.0f;
            if (bo < nb && 2 * p + (lane >> 5) < rows_ok)
                dbg_partial(a, kind, o0 + t, wrow0 + 2 * p + (lane >> 5), bo, s);
        }
        if (n + D < N) /* resolved at compile time */
            item_load<BITS, NI>(R.it[n % D], rows0, rowbytes, n + D, rows_ok, nb, nullptr);
        if (p == 7) {
            if constexpr (GROUPED)
                chunk_scales_store(CS, W, lane);
            wave_lds_sync();
            const float* dc = dls + tf * sd + kChunk * i;
            if constexpr (GROUPED)
                acc = fold_chunk_grouped(P + tf * kTile, k, dc, acc, W);
            else
                acc = fold_chunk(P + tf * kTile, k, dc, acc);
            wave_lds_sync();
        }
    }
    return acc;
}

/* Stages the codes (operand order) and block scales of the unit's tokens;
 * every thread issues up to kDcStage items' loads before converting any.
 * Scales past nb (up to sd per token) are zero. */
template <int BITS, int TMAX>
__device__ __forceinline__ void rows_stage(uint32_t* xal, float* dls, int nb, int sd, int ntok,
                                           const int8_t* const (&act)[TMAX], const float* const (&scl)[TMAX])
{
    const int n_items = ntok * nb;
    for (int i0 = threadIdx.x; i0 < n_items; i0 += 64 * kJobWaves * kDcStage) {
        uint32_t x[kDcStage][8];
        float dv[kDcStage];
#pragma unroll
        for (int r = 0; r < kDcStage; ++r) {
            const int i = i0 + r * 64 * kJobWaves;
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
            const int i = i0 + r * 64 * kJobWaves;
            if (i < n_items) {
                const int t = i / nb, b = i - t * nb;
                uint32_t xa[8];
                prep_dot<BITS>(x[r], xa);
                uint4* dst = reinterpret_cast<uint4*>(xal + (int64_t)i * 8);
                dst[0] = make_uint4(xa[0], xa[1], xa[2], xa[3]);
                dst[1] = make_uint4(xa[4], xa[5], xa[6], xa[7]);
                dls[t * sd + b] = dv[r];
            }
        }
    }
    for (int i = threadIdx.x; i < TMAX * (sd - nb); i += 64 * kJobWaves)
        dls[(i / (sd - nb)) * sd + nb + i % (sd - nb)] = 0.0f;
    __syncthreads();
}

} // namespace

template <int BITS, int NI, int TMAX, bool GROUPED>
__global__ __launch_bounds__(256) void ffn_gate_up_rows(FfnArgs a)
{
    extern __shared__ __attribute__((aligned(16))) int32_t rw_lds[];
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int RB = a.I / 32;
    JobLoc L;
    if (!locate(a, blockIdx.x, RB, L))
        return;
    const FfnSeg sg = pick(a, L.seg);
    int e, pos0, ntok;
    if (!unit_info(sg, L.unit, e, pos0, ntok))
        return;
    ntok = min(ntok, TMAX);
    const int nb = a.H / 32, sd = kChunk * NI;
    const int64_t rowbytes = (int64_t)a.H * BITS / 8;
    uint32_t* xal = reinterpret_cast<uint32_t*>(rw_lds);
    float* dls = reinterpret_cast<float*>(xal + (int64_t)TMAX * nb * 8);
    float* P = dls + TMAX * sd + wv * (TMAX * kTile);
    float* vs = dls + TMAX * sd + kJobWaves * TMAX * kTile;
    float* W = vs + 64 * TMAX + wv * kTile; /* grouped: the wave's scale tile */
    /* waves 0, 1: gate rows rb*32 + 16w ..; waves 2, 3: the same up rows */
    const int rloc = 16 * (wv & 1);
    const uint8_t* rows0 = (wv < 2 ? sg.gate_w : sg.up_w) + ((int64_t)e * a.I + L.rb * 32 + rloc) * rowbytes;
    Ring<BITS, NI> R;
    ring_start<BITS, NI>(R, rows0, rowbytes, kWaveRows, nb);
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
    rows_stage<BITS, TMAX>(xal, dls, nb, sd, ntok, act, scl);
    const int ng = sg.gu_gb ? nb / sg.gu_gb : 0;
    const float* ws0 = sg.gu_gb ? (wv < 2 ? sg.gate_s : sg.up_s) + ((int64_t)e * a.I + L.rb * 32 + rloc) * ng
                                : nullptr;
    const int64_t o0 = sg.out_base + pos0;
    const int kd = wv < 2 ? kDbgGate : kDbgUp, wr0 = L.rb * 32 + rloc;
    const float v = rows_k_loop<BITS, NI, TMAX, GROUPED>(R, rows0, rowbytes, kWaveRows, nb, ntok, xal, dls, P, ws0,
                                                         sg.gu_gb, a, o0, kd, wr0, W);
    /* job row of the wave's row k: gate rows 0..31, up rows 32..63 */
    const int t_l = lane >> 4;
    if (t_l < ntok)
        vs[(16 * wv + (lane & 15)) * TMAX + t_l] = v;
    __syncthreads();
    if (wv != 0)
        return;
    const int nbi = a.I / 32;
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
        if (t < ntok) {
            const float gv = sc * vs[lane * TMAX + t];
            const float u = shfl_xor(gv, 32);
            const float h = canon_silu(gv) * u;
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

template <int BITS, int NI, int TMAX, bool GROUPED>
__global__ __launch_bounds__(256) void ffn_down_rows(FfnArgs a)
{
    extern __shared__ __attribute__((aligned(16))) int32_t rw_lds[];
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int RB = (a.H + kRowsPerJob - 1) / kRowsPerJob;
    JobLoc L;
    if (!locate(a, blockIdx.x, RB, L))
        return;
    const FfnSeg sg = pick(a, L.seg);
    int e, pos0, ntok;
    if (!unit_info(sg, L.unit, e, pos0, ntok))
        return;
    ntok = min(ntok, TMAX);
    const int nb = a.I / 32, sd = kChunk * NI;
    const int64_t rowbytes = (int64_t)a.I * BITS / 8;
    uint32_t* xal = reinterpret_cast<uint32_t*>(rw_lds);
    float* dls = reinterpret_cast<float*>(xal + (int64_t)TMAX * nb * 8);
    float* P = dls + TMAX * sd + wv * (TMAX * kTile);
    float* W = dls + TMAX * sd + kJobWaves * TMAX * kTile + 64 * TMAX + wv * kTile; /* grouped: scale tile */
    const int first = L.rb * kRowsPerJob + kWaveRows * wv;
    const int rows_ok = min(kWaveRows, max(0, a.H - first));
    const uint8_t* rows0 = sg.down_w + ((int64_t)e * a.H + min(first, a.H - 1)) * rowbytes;
    Ring<BITS, NI> R;
    ring_start<BITS, NI>(R, rows0, rowbytes, rows_ok, nb);
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
    rows_stage<BITS, TMAX>(xal, dls, nb, sd, ntok, act, scl);
    const int ng = sg.d_gb ? nb / sg.d_gb : 0;
    const float* ws0 = sg.d_gb ? sg.down_s + ((int64_t)e * a.H + min(first, a.H - 1)) * ng : nullptr;
    const int64_t o0 = sg.out_base + pos0;
    const float v = rows_k_loop<BITS, NI, TMAX, GROUPED>(R, rows0, rowbytes, rows_ok, nb, ntok, xal, dls, P, ws0,
                                                         sg.d_gb, a, o0, kDbgDown, first, W);
    const int t_l = lane >> 4;
    if (t_l < ntok && (lane & 15) < rows_ok)
        a.y[(int64_t)(sg.out_base + pos0 + t_l) * a.H + n] = sc * v;
}

namespace {

/* ---- one token: down projection with the combine --------------------------
 * A workgroup owns 2 DW output rows for all U = k (+1 shared) units; wave w
 * streams rows 2w, 2w+1 of every unit's down matrix as whole-row pairs
 * (pair j = unit j), two units in flight.  All units' h codes are staged in
 * LDS in operand order once per workgroup (measured faster than each lane
 * loading its own h blocks per unit, and than four units in flight).  Lane
 * (unit, row) then runs the canonical chain of its row, and the wave forms
 * out = y_shared + sum_j w_j * y_j for its rows with the same fma order as
 * combine_kernel, so the result is bit-identical to down + combine without
 * the y round trip or the extra launch.
 *
 * kDcWide waves (one workgroup per CU at H = 6144) stage every unit's h once
 * per CU; the vector L1, whose lines bound this kernel, then spends a
 * twelfth as many lines on h as with three 4-wave workgroups per CU. */
constexpr int kDcWide = 12;

/* Row stride of the staged scales and of the partials: a multiple of four
 * words (16-byte quad reads), four words past the row. */
__host__ __device__ inline int dc_sp(int nb)
{
    return ((nb + 3) & ~3) + 4;
}

/* LDS words: h codes [U][nb][8], h scales [U][sp], per wave the partials
 * [2U][sp] and the row values [2U]. */
__host__ __device__ inline size_t dc_lds_words(int U, int nb, int DW)
{
    const size_t sp = (size_t)dc_sp(nb);
    return (size_t)U * nb * 8 + (size_t)U * sp + (size_t)DW * 2 * U * sp + (size_t)DW * 2 * U;
}

/* Row pair of one unit: NI loads per lane (blocks (l & 31) + 32 i of row
 * l / 32 of the pair). */
template <int BITS, int NI>
struct PairLoad {
    uint32_t w[NI][BITS];
};

template <int BITS, int NI>
__device__ __forceinline__ void pair_load(PairLoad<BITS, NI>& L, const uint8_t* rows0, int64_t rowbytes, int nb)
{
    const int lane = threadIdx.x & 63;
    const uint8_t* rp = rows0 + (int64_t)(lane >> 5) * rowbytes;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        if constexpr (kSplit8<BITS, NI>)
            load_chunk8(rp, kChunk * i, lane & 31, nb, L.w[i]);
        else
            load_block<BITS>(rp + (int64_t)min((lane & 31) + kChunk * i, nb - 1) * (4 * BITS), L.w[i]);
    }
}

/* Exact partials of a loaded pair, as fp32, to P[row * sp + b] (o, wrow0:
 * the unit and the pair's first down row, for the test-only dump). */
template <int BITS, int NI>
__device__ __forceinline__ void pair_partials(const PairLoad<BITS, NI>& L, const uint32_t (&xa)[NI][8], int nb,
                                              float* P, int sp, const FfnArgs& a, int o, int wrow0)
{
    const int lane = threadIdx.x & 63;
    const int row = lane >> 5, c = lane & 31;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        if constexpr (kSplit8<BITS, NI>) {
            /* every lane takes part in the halves' exchange */
            const int b = own8(c) + kChunk * i;
            const int32_t s = dot_chunk8(L.w[i], xa[i], c);
            if (b < nb) {
                P[row * sp + b] = (float)s;
                dbg_partial(a, kDbgDown, o, wrow0 + row, b, s);
            }
        } else {
            const int b = c + kChunk * i;
            if (b < nb) {
                const int32_t s = block_dot<BITS>(L.w[i], xa[i]);
                P[row * sp + b] = (float)s;
                dbg_partial(a, kDbgDown, o, wrow0 + row, b, s);
            }
        }
    }
}

/* A whole row's chain over nb blocks: pr the partials, dj the block scales
 * (both 16-byte aligned), in ascending order from acc = +0. */
__device__ __forceinline__ float fold_row(const float* pr, const float* dj, int nb)
{
    float acc = 0.0f;
    int b = 0;
    for (; b + 8 <= nb; b += 8) {
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(pr + b);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(pr + b + 4);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(dj + b);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(dj + b + 4);
        acc = __builtin_fmaf(d0.x, s0.x, acc);
        acc = __builtin_fmaf(d0.y, s0.y, acc);
        acc = __builtin_fmaf(d0.z, s0.z, acc);
        acc = __builtin_fmaf(d0.w, s0.w, acc);
        acc = __builtin_fmaf(d1.x, s1.x, acc);
        acc = __builtin_fmaf(d1.y, s1.y, acc);
        acc = __builtin_fmaf(d1.z, s1.z, acc);
        acc = __builtin_fmaf(d1.w, s1.w, acc);
        asm volatile("" : "+v"(acc) : : "memory"); /* as in fold_chunk */
    }
    for (; b < nb; ++b)
        acc = __builtin_fmaf(dj[b], pr[b], acc);
    return acc;
}

__device__ __forceinline__ float fold_row_grouped(const float* pr, const float* dj, int nb, const float* ws, int gb)
{
    float acc = 0.0f;
    for (int b = 0; b < nb; ++b)
        acc = __builtin_fmaf(group_coef(ws, gb, b, dj[b]), pr[b], acc);
    return acc;
}

template <int BITS, int NI>
__device__ __forceinline__ void dc_act(const uint32_t* xal, int j, int nb, uint32_t (&xa)[NI][8])
{
    const int c = threadIdx.x & 31;
    if constexpr (kSplit8<BITS, NI>) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
            act_chunk8(xal + (int64_t)j * nb * 8, kChunk * i, c, nb, xa[i]);
        return;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const uint4* src = reinterpret_cast<const uint4*>(xal + ((int64_t)j * nb + min(c + kChunk * i, nb - 1)) * 8);
        const uint4 u0 = src[0], u1 = src[1];
        xa[i][0] = u0.x; xa[i][1] = u0.y; xa[i][2] = u0.z; xa[i][3] = u0.w;
        xa[i][4] = u1.x; xa[i][5] = u1.y; xa[i][6] = u1.z; xa[i][7] = u1.w;
    }
}

/* First of this wave's two rows of the down matrix of unit u (u = slot, or
 * k for the shared expert) whose matrix index is e. */
__device__ __forceinline__ const uint8_t* dc_rows(const DecodeArgs& d, int u, int e, int row0, int64_t rowbytes)
{
    const FfnArgs& a = d.f;
    const uint8_t* w = u < d.k ? a.seg[0].down_w : a.seg[1].down_w;
    return w + ((int64_t)e * a.H + row0) * rowbytes;
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

} // namespace

template <int BITS, int NI, int DW>
__global__ __launch_bounds__(64 * DW) void ffn_down_combine_decode(DecodeArgs d)
{
    extern __shared__ __attribute__((aligned(16))) int32_t dc_lds[];
    const FfnArgs& a = d.f;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const bool shared = a.nseg > 1;
    /* slots dropped by top-p are neither streamed nor combined: the units are
     * the kept routed slots in slot order, then the shared expert */
    const bool all_kept = !(d.opt.top_p > 0.0f && d.opt.top_p < 1.0f);
    const uint64_t kept = all_kept ? 0 : __ballot(lane < d.k && d.ids[lane] >= 0);
    const int n_kept = all_kept ? d.k : __popcll(kept);
    const int U = n_kept + (shared ? 1 : 0);
    const int nb = a.I / 32, sp = dc_sp(nb);
    uint32_t* xal = reinterpret_cast<uint32_t*>(dc_lds);    /* [U][nb][8] */
    float* dls = reinterpret_cast<float*>(xal + U * nb * 8); /* [U][sp] */
    float* P0 = dls + U * sp;                                /* [DW][2U][sp] */
    float* P = P0 + wv * (2 * U * sp);
    float* ys = P0 + DW * 2 * U * sp + wv * 2 * U;
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
        pair_load<BITS, NI>(A, dc_rows(d, d.k, 0, row0, rowbytes), rowbytes, nb);
    /* per-unit values in lane registers, loaded once (U <= 32): lane j holds
     * compacted unit j's unit id, matrix index and routing weight (lane
     * 2j + r gets the row scale of this wave's row r of unit j once h is
     * staged: its address needs the id, and h's loads need nothing) */
    const int u_l = dc_unit(kept, n_kept, d.k, min(lane, U - 1), all_kept);
    const bool rt_l = u_l < d.k;
    const int e_l = rt_l ? decode_matrix(d.slot_of, d.ids[u_l], d.E, a.seg[0].n_mat) : 0;
    const float w_l = rt_l ? d.w[u_l] : 0.0f;
    /* a tiered forward with every expert resident: block 0's first wave
     * leaves the slot cache's state as the plan kernel leaves it after this
     * all-hit batch (every kept slot a hit in slot e_l), after the block's
     * rows */
    const bool note = d.note_hits != 0 && blockIdx.x == 0 && wv == 0;
    const int32_t id_n = note && lane < n_kept ? d.ids[u_l] : 0;
    /* without a shared expert, compacted unit 0's pair is issued before h is staged */
    if (!shared)
        pair_load<BITS, NI>(A, dc_rows(d, __builtin_amdgcn_readlane(u_l, 0), __builtin_amdgcn_readlane(e_l, 0), row0,
                                       rowbytes),
                            rowbytes, nb);
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

    /* chains [c_begin, c_end) (at most 64): chain rd = (compacted unit
     * rd / 2, row rd % 2) on lane rd - c_begin */
    auto fold_chains = [&](int c_begin, int c_end) {
        const int ci = c_begin + lane;
        const int rd = min(ci, 2 * U - 1);
        /* lane values are read before any branch: every lane is active */
        const int uf = __shfl(u_l, rd >> 1, kWave), ef = __shfl(e_l, rd >> 1, kWave);
        const float rsv = __shfl(rs_l, rd, kWave);
        const int gbf = uf < d.k ? a.seg[0].d_gb : a.seg[1].d_gb;
        const float* pr = P + rd * sp;
        const float* dj = dls + (rd >> 1) * sp;
        float acc;
        if (gbf) {
            /* group-wise scales of (unit, row) */
            const float* ws = (uf < d.k ? a.seg[0].down_s : a.seg[1].down_s) +
                              ((int64_t)ef * a.H + row0 + (rd & 1)) * (nb / gbf);
            acc = fold_row_grouped(pr, dj, nb, ws, gbf);
        } else {
            acc = fold_row(pr, dj, nb);
        }
        if (ci < c_end)
            ys[rd] = rsv * acc; /* rsv: 1 with group-wise scales */
    };

    /* the pair of stream position q is in A for even q and in B for odd q;
     * loads are unconditional (past the last unit they reload it: in bounds,
     * unused) */
    for (int q = 0; q < U; q += 2) {
        uint32_t xa[NI][8];
        const int j0 = unit_at(q), j1 = unit_at(min(q + 1, U - 1)), j2 = unit_at(min(q + 2, U - 1));
        pair_load<BITS, NI>(B, dc_rows(d, __builtin_amdgcn_readlane(u_l, j1), __builtin_amdgcn_readlane(e_l, j1), row0,
                                       rowbytes),
                            rowbytes, nb);
        dc_act<BITS, NI>(xal, j0, nb, xa);
        pair_partials<BITS, NI>(A, xa, nb, P + 2 * j0 * sp, sp, a, __builtin_amdgcn_readlane(u_l, j0), row0);
        pair_load<BITS, NI>(A, dc_rows(d, __builtin_amdgcn_readlane(u_l, j2), __builtin_amdgcn_readlane(e_l, j2), row0,
                                       rowbytes),
                            rowbytes, nb);
        if (q + 1 < U) {
            dc_act<BITS, NI>(xal, j1, nb, xa);
            pair_partials<BITS, NI>(B, xa, nb, P + 2 * j1 * sp, sp, a, __builtin_amdgcn_readlane(u_l, j1), row0);
        }
    }
    /* every chain (at most 64: U <= 32) in one pass, one per lane, after the
     * stream (a fold inside the loop would hold back the next row loads) */
    wave_lds_sync();
    fold_chains(0, 2 * U);
    wave_lds_sync();
    /* compacted order is slot order: the combine's fma order is kept (every
     * lane runs the chain of row lane & 1; lanes 0 and 1 store) */
    float outv = shared ? ys[2 * n_kept + (lane & 1)] : 0.0f;
    for (int j = 0; j < n_kept; ++j)
        outv = __builtin_fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_l), j)), ys[2 * j + (lane & 1)],
                              outv);
    if (lane < 2)
        d.out[row0 + lane] = outv;
    if (note) {
        /* hits are used now (tick), each expert's usage counts its pair, the
         * plan consumes every in-flight mark; a hit still marked in flight is
         * a late hit, which makes the plan two passes */
        TierHdr* hd = d.ts.hdr;
        const bool kl = lane < n_kept;
        const uint32_t tick = hd->tick + 1;
        const unsigned long long plans = hd->plans, pairs = hd->pairs, hits = hd->hits, passes = hd->passes;
        const unsigned long long use = d.ts.usage[kl ? id_n : 0];
        const int32_t infl = d.ts.inflight[kl ? e_l : 0];
        const bool late = __ballot(kl && infl != 0) != 0;
        __builtin_amdgcn_wave_barrier();
        if (kl) {
            d.ts.last_use[e_l] = tick;
            d.ts.usage[id_n] = use + 1ull;
        }
        for (int sl = lane; sl < d.ts.n; sl += 64)
            d.ts.inflight[sl] = 0;
        if (lane == 0) {
            hd->tick = tick;
            hd->plans = plans + 1;
            hd->pairs = pairs + (unsigned long long)n_kept;
            hd->hits = hits + (unsigned long long)n_kept;
            hd->passes = passes + (late ? 2 : 1);
        }
    }
}

static int64_t total_jobs(const FfnArgs& a, int RB)
{
    int64_t n = (int64_t)a.seg[0].max_units * RB;
    if (a.nseg > 1)
        n += (int64_t)a.seg[1].max_units * RB;
    return n;
}

/* Raises a kernel's dynamic LDS limit once, when it needs more than 64 KB. */
static void allow_lds(const void* fn, size_t lds)
{
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsMax);
}

template <int BITS, int NI, int TMAX, bool GROUPED>
static void launch_rows_k(bool gate_up, dim3 grid, size_t lds, const FfnArgs& a, hipStream_t st)
{
    const dim3 block(64 * kJobWaves);
    if (gate_up) {
        allow_lds(reinterpret_cast<const void*>(&ffn_gate_up_rows<BITS, NI, TMAX, GROUPED>), lds);
        hipLaunchKernelGGL((ffn_gate_up_rows<BITS, NI, TMAX, GROUPED>), grid, block, lds, st, a);
    } else {
        allow_lds(reinterpret_cast<const void*>(&ffn_down_rows<BITS, NI, TMAX, GROUPED>), lds);
        hipLaunchKernelGGL((ffn_down_rows<BITS, NI, TMAX, GROUPED>), grid, block, lds, st, a);
    }
}

template <int NI, int TMAX, bool GROUPED>
static void launch_rows_ni(const FfnArgs& a, int32_t bits, bool gate_up, dim3 grid, size_t lds, hipStream_t st)
{
    switch (bits) {
    case 8: launch_rows_k<8, NI, TMAX, GROUPED>(gate_up, grid, lds, a, st); break;
    case 4: launch_rows_k<4, NI, TMAX, GROUPED>(gate_up, grid, lds, a, st); break;
    default: launch_rows_k<2, NI, TMAX, GROUPED>(gate_up, grid, lds, a, st); break;
    }
}

template <int TMAX, bool GROUPED>
static void launch_rows_g(const FfnArgs& a, int32_t bits, bool gate_up, dim3 grid, hipStream_t st)
{
    const int nb = gate_up ? a.H / 32 : a.I / 32;
    const size_t lds = rows_lds_words(nb, TMAX, GROUPED) * 4;
    switch (gemv_ni(nb)) {
    case 1: launch_rows_ni<1, TMAX, GROUPED>(a, bits, gate_up, grid, lds, st); break;
    case 2: launch_rows_ni<2, TMAX, GROUPED>(a, bits, gate_up, grid, lds, st); break;
    case 4: launch_rows_ni<4, TMAX, GROUPED>(a, bits, gate_up, grid, lds, st); break;
    case 6: launch_rows_ni<6, TMAX, GROUPED>(a, bits, gate_up, grid, lds, st); break;
    default: launch_rows_ni<8, TMAX, GROUPED>(a, bits, gate_up, grid, lds, st); break;
    }
}

/* Whether a launch's segments hold group-wise scales (gate/up or down). */
static bool any_grouped(const FfnArgs& a, bool gate_up)
{
    bool g = false;
    for (int i = 0; i < a.nseg && i < 2; ++i)
        g = g || (gate_up ? a.seg[i].gu_gb : a.seg[i].d_gb) != 0;
    return g;
}

template <int TMAX>
static void launch_rows_t(const FfnArgs& a, int32_t bits, bool gate_up, dim3 grid, hipStream_t st)
{
    if (any_grouped(a, gate_up))
        launch_rows_g<TMAX, true>(a, bits, gate_up, grid, st);
    else
        launch_rows_g<TMAX, false>(a, bits, gate_up, grid, st);
}

hipError_t launch_ffn_gate_up(const FfnArgs& a, int32_t bits, hipStream_t st)
{
    const int64_t jobs = total_jobs(a, a.I / 32);
    if (jobs == 0)
        return hipSuccess;
    if (a.unit_tokens == 1)
        launch_rows_t<1>(a, bits, true, dim3((uint32_t)jobs), st);
    else
        launch_rows_t<kUnitTokens>(a, bits, true, dim3((uint32_t)jobs), st);
    return hipGetLastError();
}

hipError_t launch_ffn_down(const FfnArgs& a, int32_t bits, hipStream_t st)
{
    const int64_t jobs = total_jobs(a, (a.H + kRowsPerJob - 1) / kRowsPerJob);
    if (jobs == 0)
        return hipSuccess;
    if (a.unit_tokens == 1)
        launch_rows_t<1>(a, bits, false, dim3((uint32_t)jobs), st);
    else
        launch_rows_t<kUnitTokens>(a, bits, false, dim3((uint32_t)jobs), st);
    return hipGetLastError();
}

template <int NI, bool GROUPED>
static void gate_up_decode_ni(const DecodeArgs& d, int32_t bits, dim3 grid, size_t lds, hipStream_t st)
{
    const dim3 block(64 * kJobWaves);
    switch (bits) {
    case 8: hipLaunchKernelGGL((ffn_gate_up_decode<8, NI, GROUPED>), grid, block, lds, st, d); break;
    case 4: hipLaunchKernelGGL((ffn_gate_up_decode<4, NI, GROUPED>), grid, block, lds, st, d); break;
    default: hipLaunchKernelGGL((ffn_gate_up_decode<2, NI, GROUPED>), grid, block, lds, st, d); break;
    }
}

template <int NI, bool GROUPED>
static void down_decode_ni(const DecodeArgs& d, int32_t bits, dim3 grid, size_t lds, hipStream_t st)
{
    const dim3 block(64 * kJobWaves);
    switch (bits) {
    case 8: hipLaunchKernelGGL((ffn_down_decode<8, NI, GROUPED>), grid, block, lds, st, d); break;
    case 4: hipLaunchKernelGGL((ffn_down_decode<4, NI, GROUPED>), grid, block, lds, st, d); break;
    default: hipLaunchKernelGGL((ffn_down_decode<2, NI, GROUPED>), grid, block, lds, st, d); break;
    }
}

template <bool GROUPED>
static void gate_up_decode_g(const DecodeArgs& d, int32_t bits, dim3 grid, size_t lds, int nb, hipStream_t st)
{
    switch (gemv_ni(nb)) {
    case 1: gate_up_decode_ni<1, GROUPED>(d, bits, grid, lds, st); break;
    case 2: gate_up_decode_ni<2, GROUPED>(d, bits, grid, lds, st); break;
    case 4: gate_up_decode_ni<4, GROUPED>(d, bits, grid, lds, st); break;
    case 6: gate_up_decode_ni<6, GROUPED>(d, bits, grid, lds, st); break;
    default: gate_up_decode_ni<8, GROUPED>(d, bits, grid, lds, st); break;
    }
}

template <bool GROUPED>
static void down_decode_g(const DecodeArgs& d, int32_t bits, dim3 grid, size_t lds, int nb, hipStream_t st)
{
    switch (gemv_ni(nb)) {
    case 1: down_decode_ni<1, GROUPED>(d, bits, grid, lds, st); break;
    case 2: down_decode_ni<2, GROUPED>(d, bits, grid, lds, st); break;
    case 4: down_decode_ni<4, GROUPED>(d, bits, grid, lds, st); break;
    case 6: down_decode_ni<6, GROUPED>(d, bits, grid, lds, st); break;
    default: down_decode_ni<8, GROUPED>(d, bits, grid, lds, st); break;
    }
}

hipError_t launch_ffn_gate_up_decode(const DecodeArgs& d, int32_t bits, hipStream_t st)
{
    /* one-wave jobs of the shared expert (d.hs), then whole jobs */
    const int64_t jobs = (int64_t)(d.k + (d.f.nseg > 1 && !d.hs ? 1 : 0)) * (d.f.I / 32) + (d.hs ? d.f.I / 8 : 0);
    const int nb = d.f.H / 32;
    const dim3 grid((uint32_t)jobs);
    const size_t lds = dec_lds_bytes(nb, any_grouped(d.f, true));
    if (any_grouped(d.f, true))
        gate_up_decode_g<true>(d, bits, grid, lds, nb, st);
    else
        gate_up_decode_g<false>(d, bits, grid, lds, nb, st);
    return hipGetLastError();
}

hipError_t launch_ffn_down_decode(const DecodeArgs& d, int32_t bits, hipStream_t st)
{
    const int64_t jobs = (int64_t)(d.k + (d.f.nseg > 1 ? 1 : 0)) * ((d.f.H + kRowsPerJob - 1) / kRowsPerJob);
    const int nb = d.f.I / 32;
    const dim3 grid((uint32_t)jobs);
    const size_t lds = dec_lds_bytes(nb, any_grouped(d.f, false));
    if (any_grouped(d.f, false))
        down_decode_g<true>(d, bits, grid, lds, nb, st);
    else
        down_decode_g<false>(d, bits, grid, lds, nb, st);
    return hipGetLastError();
}

template <int BITS, int NI, int DW>
static void down_combine_launch(const DecodeArgs& d, dim3 grid, size_t lds, hipStream_t st)
{
    if (lds > 64 * 1024) {
        static bool raised = false; /* once per instantiation */
        if (!raised) {
            allow_lds(reinterpret_cast<const void*>(&ffn_down_combine_decode<BITS, NI, DW>), lds);
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
    if (d.f.H % (2 * kDcWide) == 0 && dc_lds_words(U, nb, kDcWide) * 4 <= kLdsMax)
        return kDcWide;
    return kJobWaves;
}

bool down_combine_decode_fits(const DecodeArgs& d)
{
    const int U = d.k + (d.f.nseg > 1 ? 1 : 0);
    /* per-unit values live in lanes: 2U row chains per wave */
    return U <= 32 && d.f.H % (2 * kJobWaves) == 0 && dc_lds_words(U, d.f.I / 32, kJobWaves) * 4 <= 64 * 1024;
}

hipError_t launch_ffn_down_combine_decode(const DecodeArgs& d, int32_t bits, hipStream_t st)
{
    const int U = d.k + (d.f.nseg > 1 ? 1 : 0);
    const int nb = d.f.I / 32;
    const int DW = dc_waves(d);
    const dim3 grid((uint32_t)(d.f.H / (2 * DW)));
    const size_t lds = dc_lds_words(U, nb, DW) * 4;
    if (DW == kDcWide) {
        switch (gemv_ni(nb)) {
        case 1: down_combine_ni<1, kDcWide>(d, bits, grid, lds, st); break;
        case 2: down_combine_ni<2, kDcWide>(d, bits, grid, lds, st); break;
        case 4: down_combine_ni<4, kDcWide>(d, bits, grid, lds, st); break;
        case 6: down_combine_ni<6, kDcWide>(d, bits, grid, lds, st); break;
        default: down_combine_ni<8, kDcWide>(d, bits, grid, lds, st); break;
        }
    } else {
        switch (gemv_ni(nb)) {
        case 1: down_combine_ni<1, kJobWaves>(d, bits, grid, lds, st); break;
        case 2: down_combine_ni<2, kJobWaves>(d, bits, grid, lds, st); break;
        case 4: down_combine_ni<4, kJobWaves>(d, bits, grid, lds, st); break;
        case 6: down_combine_ni<6, kJobWaves>(d, bits, grid, lds, st); break;
        default: down_combine_ni<8, kJobWaves>(d, bits, grid, lds, st); break;
        }
    }
    return hipGetLastError();
}

} // namespace coli
