/* libconvrot_ceiling.so: measurement kernels for the hot path's rooflines.
 *
 * Not part of the convrot linear layer's interface (include/convrot.h) and not
 * on its hot path: the benchmark times them beside the GEMM and the pack to
 * show what rate the matrix cores sustain on the same operand data, and what
 * rate HBM delivers to a pass with the pack's read:write mix.
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

/* Streams dst_bytes / 16 16-byte chunks into `dst`, each the XOR of `ratio`
 * chunks of `src` (ratio 1, 2 or 4; src holds ratio * dst_bytes bytes, read
 * as ratio contiguous planes of dst_bytes each): a pass that reads
 * ratio * dst_bytes and writes dst_bytes with non-temporal 16-byte accesses,
 * the pack's read:write mix for ratio 2 (bf16 in, int8 out) and 4 (float32
 * in).  `grid` workgroups of 256 threads walk the chunks grid-stride.  src
 * and dst are device memory, 16-byte aligned, not overlapping; dst_bytes is a
 * positive multiple of 16.  Asynchronous on `stream` (a hipStream_t, or NULL).
 * Returns 0, or -1 for an invalid argument or a launch error (then nothing
 * ran). */
int32_t convrot_ceiling_stream(const void* src, void* dst, int64_t dst_bytes, int32_t ratio,
                               int32_t grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_CEILING_H */
