/*
 * colibri_probes.h -- measurement kernels (libcolibri_probes.so) used by the
 * benchmark to report achievable device rates beside the published MI355X
 * peaks: an HBM read stream and the int8 and bf16 matrix-core loops.  They compute
 * nothing of the layer.  Pointers are device memory owned by the caller;
 * work is enqueued on `stream` (a hipStream_t); returns 0, 1 for a bad
 * argument (nothing enqueued), 4 for a launch error.
 */
#ifndef COLIBRI_PROBES_H
#define COLIBRI_PROBES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads every byte of buf (bytes a multiple of 16, buf 16-byte aligned) once
 * with 16-byte nontemporal loads from n_blocks workgroups of 256 threads:
 * blocked != 0, workgroup b streams the b-th contiguous span; otherwise the
 * grid strides over the buffer.  sink holds n_blocks words (written only in
 * an unlikely case: it keeps the loads from being removed). */
int colibri_probe_read(const void* buf, size_t bytes, int32_t n_blocks, int32_t blocked, uint32_t* sink,
                       void* stream);

/* The one-token GEMV kernels' weight read pattern without their
 * arithmetic: wave w reads 16 consecutive rows of 512 * ni bytes (ni = 2 or
 * 6) starting at buf + 16 w * 512 * ni, in items of two rows by 512 bytes,
 * chunk-major (chunk_major != 0) or row-major, 2 ni items in flight;
 * n_waves waves in workgroups of four (buf holds n_waves * 16 rows). */
int colibri_probe_rows(const void* buf, int32_t ni, int32_t n_waves, int32_t chunk_major, uint32_t* sink,
                       void* stream);

/* The matrix-core kernels' weight read pattern without their arithmetic:
 * n_rows / 64 workgroups of 256 threads; workgroup g reads rows
 * [64 g, 64 g + 64) of rowbytes bytes (buf holds n_rows * rowbytes) in steps
 * of chunk bytes of every row (chunk = 128, 256 or 512; rowbytes a multiple
 * of 2 chunk), 16 bytes per thread and load, two steps in flight and a
 * barrier per step, with nontemporal loads or not; lds_bytes (<= 64 KB) of
 * unused dynamic LDS per workgroup set the occupancy.  sink: n_rows / 64
 * words. */
int colibri_probe_tile(const void* buf, int32_t rowbytes, int32_t n_rows, int32_t chunk, int32_t nontemporal,
                       int32_t lds_bytes, uint32_t* sink, void* stream);

/* n_blocks workgroups of four waves; each wave issues iters rounds of 8
 * independent v_mfma_i32_16x16x{k}_i8 (k = 32 or 64), i.e. 8 * iters *
 * 16 * 16 * k * 2 integer operations per wave.  sink: n_blocks words. */
int colibri_probe_mfma_i8(int32_t k, int32_t iters, int32_t n_blocks, int32_t* sink, void* stream);

/* As colibri_probe_mfma_i8 for v_mfma_f32_16x16x32_bf16 (K = 32, fp32
 * accumulation): 8 * iters * 16 * 16 * 32 * 2 floating-point operations per
 * wave. */
int colibri_probe_mfma_bf16(int32_t iters, int32_t n_blocks, int32_t* sink, void* stream);

/* One v_mfma_f32_16x16x32_bf16 by one wave: d = c + a b, with a [16][32]
 * and b [32][16] bfloat16 bit patterns and c, d [16][16] fp32, all
 * row-major device arrays.  It shows whether the fp32 sums of integer-valued
 * products come out exact (the exactness a bfloat16 form of the integer
 * block partials would need). */
int colibri_probe_mfma_bf16_block(const uint16_t* a, const uint16_t* b, const float* c, float* d, void* stream);

#ifdef __cplusplus
}
#endif

#endif
