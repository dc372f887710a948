/* libconvrot_ceiling.so: a measurement kernel for the INT8 GEMM's roofline.
 *
 * Not part of the convrot linear layer's interface (include/convrot.h) and not
 * on its hot path: the benchmark times it beside the GEMM to show what rate
 * the matrix cores sustain on the same operand data.
 */
#ifndef CONVROT_CEILING_H
#define CONVROT_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Launches `grid` workgroups of 4 waves (one wave per SIMD), each wave running
 * `iters` iterations of 24 v_mfma_i32_32x32x32_i8 (a 4 x 3 set of 32 x 32
 * int32 accumulators, two alternating 32-wide K slices) on operand fragments
 * read once, before the loop, from the int8 rows of `a` (rows_a rows, row
 * stride lda bytes) and `b` (rows_b, ldb) -- device memory, 16-byte aligned,
 * rows_a and rows_b >= 32, lda and ldb >= 128 and multiples of 16.  `sink`
 * (device, grid * 256 int32) receives one value per lane so that no work is
 * dead.  Asynchronous on `stream` (a hipStream_t, or NULL for the default
 * stream).
 * Returns the int8 operations of the launch (2 per multiply-add), or -1 for an
 * invalid argument or a launch error (then nothing ran). */
int64_t convrot_ceiling_mfma_i8(const int8_t* a, int64_t lda, int64_t rows_a, const int8_t* b,
                                int64_t ldb, int64_t rows_b, int32_t iters, int32_t grid,
                                int32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_CEILING_H */
