/*
 * colibri_debug.h -- the test-only build of libcolibri (libcolibri_debug.so).
 *
 * The same kernels as libcolibri.so, compiled with COLI_DEBUG_PARTIALS: every
 * FFN kernel (one-token, whole-row and both matrix-core K loops) also stores
 * the exact int32 block partials S_b = sum over a 32-element block of weight
 * code times activation code ("Show HN: 如何在我的低配置电脑上运行 GLM-5.2",
 * section 已实现的功能, integer dot-product item) that it computes for one
 * requested slice, so that tests can compare them with the oracle's directly.
 * Every call of colibri.h is exported by this library too, with identical
 * results; only tests load it.
 */
#ifndef COLIBRI_DEBUG_H
#define COLIBRI_DEBUG_H

#include "colibri.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Selects the slice that later layer forwards and expert FFN calls in this
 * process dump: matrix kind (0 gate, 1 up, 2 down), output rows [o0, o1) of
 * the intermediate rows (the sorted pair positions, then the shared expert's
 * rows; for a one-token forward: slot u, then the shared expert as unit
 * top_k), weight rows [r0, r1) of that matrix, blocks [0, nb).  Partial
 * (o, r, b) goes to out[((o - o0) * (r1 - r0) + (r - r0)) * nb + b] (int32,
 * device memory owned by the caller and large enough); entries the kernels do
 * not compute are left as they were.  out == NULL switches the dump off.
 * The selection is process-wide host state, read when a call enqueues its
 * kernels.  COLI_E_INVAL: a kind other than 0..2, a reversed range or a
 * negative nb.
 */
int colibri_debug_partials(int32_t* out, int32_t kind, int32_t o0, int32_t o1, int32_t r0, int32_t r1,
                           int32_t nb);

#ifdef __cplusplus
}
#endif

#endif
