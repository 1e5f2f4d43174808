/*
 * kernels.h -- internal launch interface of libcolibri's gfx950 kernels.
 * Host-side argument validation lives in api.hip; every launcher here assumes
 * validated shapes and returns the HIP launch status.
 */
#ifndef COLI_KERNELS_H
#define COLI_KERNELS_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coli {

/* Tokens that one GEMV work unit applies an expert's rows to.  Experts with
 * more tokens are split into several units. */
constexpr int kUnitTokens = 4;

/* Batches of at most this many tokens use the small-batch router kernels
 * (a workgroup per router row; selection and dispatch in one workgroup). */
constexpr int kSmallS = 8;

/* A work unit: expert e applied to sorted positions [pos0, pos0 + ntok). */
struct Unit {
    int32_t e, pos0, ntok, pad;
};

/* One group of experts run by the FFN kernels. */
struct FfnSeg {
    const uint8_t* gate_w;
    const float* gate_s;
    const uint8_t* up_w;
    const float* up_s;
    const uint8_t* down_w;
    const float* down_s;
    const int32_t* sorted; /* pair index per sorted position; nullptr: identity */
    const Unit* units;     /* device unit list; nullptr: one expert, units of kUnitTokens tokens over positions [0, S) */
    const int32_t* n_units; /* device count of `units` */
    int32_t k;              /* token of pair p is p / k */
    int32_t out_base;       /* first row of this group in hq / hd / y */
    int32_t max_units;      /* upper bound on the unit count (grid sizing) */
    int32_t S;              /* tokens of the batch */
    int32_t rows;           /* sorted positions of this group (S*k, or S for identity) */
    int32_t n_mat;          /* matrices in the group's banks */
};

struct FfnArgs {
    FfnSeg seg[2];
    int32_t nseg;
    int32_t unit_tokens; /* most tokens any unit holds: 1 or kUnitTokens */
    int32_t H, I;
    const int8_t* xq; /* [S][H]   */
    const float* xd;  /* [S][H/32] */
    int8_t* hq;       /* [rows][I] */
    float* hd;        /* [rows][I/32] */
    float* y;         /* [rows][H] */
};

/* Upper bound on the number of units of a routed group with P pairs over E
 * experts: sum_e ceil(n_e / U) <= (P + (U - 1) * min(E, P)) / U. */
inline int32_t max_routed_units(int64_t P, int32_t E)
{
    int64_t active = P < E ? P : E;
    return (int32_t)((P + (kUnitTokens - 1) * active) / kUnitTokens);
}

inline int32_t identity_units(int32_t S)
{
    return (S + kUnitTokens - 1) / kUnitTokens;
}

hipError_t launch_quantize_q8_0(const float* x, int64_t n_blocks, int8_t* q, float* d,
                                hipStream_t st);

hipError_t launch_router_logits(const float* x, int32_t S, int32_t H, int32_t E,
                                const float* w, float* logits, hipStream_t st);

hipError_t launch_router_select(const float* logits, const float* bias, int32_t S, int32_t E,
                                int32_t k, float rsf, int32_t* ids, float* weights,
                                hipStream_t st);

/* S <= kSmallS: router logits and Q8_0 quantisation of x in one launch. */
hipError_t launch_route_prep_small(const float* x, int32_t S, int32_t H, int32_t E, const float* w,
                                   float* logits, int8_t* xq, float* xd, hipStream_t st);

/* S <= kSmallS: selection, union dispatch and unit list in one workgroup. */
hipError_t launch_select_dispatch_small(const float* logits, const float* bias, int32_t S, int32_t E,
                                        int32_t k, float rsf, int32_t* ids, float* weights,
                                        int32_t* offsets, int32_t* sorted, int32_t* inv,
                                        int32_t* active, int32_t* n_active, Unit* units,
                                        int32_t* n_units, hipStream_t st);

/* Union dispatch; `units` / `n_units` may be null (then no unit list). */
hipError_t launch_dispatch(const int32_t* ids, int32_t S, int32_t k, int32_t E,
                           int32_t* offsets, int32_t* sorted, int32_t* inv, int32_t* active,
                           int32_t* n_active, Unit* units, int32_t* n_units, hipStream_t st);

/* Unit list from expert offsets (for a caller-provided dispatch), at most
 * max_units units. */
hipError_t launch_schedule(const int32_t* offsets, int32_t n_mat, int32_t max_units, Unit* units,
                           int32_t* n_units, hipStream_t st);

hipError_t launch_ffn_gate_up(const FfnArgs& a, int32_t bits, hipStream_t st);
hipError_t launch_ffn_down(const FfnArgs& a, int32_t bits, hipStream_t st);

hipError_t launch_combine(const float* y, const int32_t* inv, const float* w, int32_t S,
                          int32_t k, int32_t H, int32_t shared_row0, float* out, hipStream_t st);

} // namespace coli

#endif
