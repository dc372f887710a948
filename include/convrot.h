/*
 * convrot.h — C ABI of libconvrot.so, the INT8 "convrot" linear layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The method is the one described on the stable-diffusion.cpp documentation
 * page "INT8 Convrot Safetensors" (cited below as [ICS] with the section):
 *   - R is block diagonal; each block is R_G, the normalised Kronecker power
 *     of the 4x4 regular Hadamard matrix H4 printed in [ICS, How INT8 convrot
 *     works], applied to every contiguous group of G = 4^n input features;
 *   - weights are rotated offline (W_rot = W R) and quantised per output row
 *     [ICS, Weight quantization];
 *   - activations are rotated at run time (X_rot = X R) and quantised with one
 *     dynamic scale per row, giving the packed activation: int8 rows plus
 *     their float row scales [ICS, Runtime activation quantization];
 *   - A = Q_x Q_w^T accumulates in int32 and Y = A s_x[r] s_w[o] + b[o]
 *     [ICS, Runtime activation quantization].
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates no device memory and keeps no pointer after a call returns.
 *   - Matrices are row-major.  "ld" arguments are row strides in elements.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued asynchronously on it; nothing synchronises.
 *   - Every argument is validated on the host before any HIP call, so an
 *     invalid call returns an error code and launches nothing.  A launch
 *     failure reported by the HIP runtime returns CONVROT_ERR_HIP.  Nothing is
 *     printed and no C++ exception crosses the ABI.  The functions are
 *     reentrant; calls on different streams may overlap.
 *   - Rounding is round-half-away-from-zero; a row whose absmax is zero gets
 *     scale 0 and all-zero codes (the page leaves both open).
 *   - Inputs are assumed finite.
 *
 * Limits (all return an error code when violated):
 *   - group_size G = 4^n with 0 <= n <= 7 (1 .. 16384), and G divides k
 *     ([ICS, Checkpoint format]: a power of four dividing in_features);
 *   - 1 <= k <= CONVROT_MAX_K, so that k * 127 * 127 fits in int32, and
 *     k % 16 == 0 (16-byte rows; an extension limit of this library);
 *   - m, n >= 0 (0 is an empty call that launches nothing) and < 2^31;
 *   - X, codes and weight pointers 16-byte aligned, X row stride a multiple
 *     of 16 bytes; Y needs only 4-byte alignment (any ldy >= n).
 */
#ifndef CONVROT_H
#define CONVROT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CONVROT_MAX_K 133136      /* largest k with k % 16 == 0 and k*127*127 < 2^31 */
#define CONVROT_MAX_LOG4_GROUP 7  /* group sizes 1, 4, 16, ..., 16384 */
#define CONVROT_MAX_GROUPED 8     /* weight matrices per convrot_linear_grouped call */
#define CONVROT_MAX_LORA_RANK 256 /* adapter ranks 16, 32, ..., 256 */

typedef enum convrot_status {
  CONVROT_OK = 0,
  CONVROT_ERR_NULL = 1,           /* a required pointer is NULL */
  CONVROT_ERR_SHAPE = 2,          /* m, n or k out of range, ld < row length */
  CONVROT_ERR_GROUP = 3,          /* G not a power of four in range, or G does not divide k */
  CONVROT_ERR_GROUP_MISMATCH = 4, /* packed activation and weights differ in G or k */
  CONVROT_ERR_DTYPE = 5,          /* unknown or unsupported dtype / activation code */
  CONVROT_ERR_UNSUPPORTED = 6,    /* k % 16 != 0, misaligned pointer or stride */
  CONVROT_ERR_HIP = 7             /* the HIP runtime reported an error */
} convrot_status;

typedef enum convrot_dtype {
  CONVROT_F32 = 0,
  CONVROT_BF16 = 1,
  CONVROT_I32 = 2
} convrot_dtype;

typedef enum convrot_act {
  CONVROT_ACT_NONE = 0,
  CONVROT_ACT_GELU = 1            /* x * Phi(x), erf form; not on the page, used by DiT MLPs */
} convrot_act;

/*
 * The packed runtime activation of [ICS, Runtime activation quantization]:
 * int8 rows and one float32 scale per row.  It may feed any number of
 * convrot_linear calls whose weights share its k and group size.
 *   q     : device int8 [m, k], row stride exactly k bytes (caller-allocated)
 *   scale : device float32 [m]                               (caller-allocated)
 */
typedef struct convrot_packed {
  int8_t* q;
  float* scale;
  int64_t m;
  int64_t k;
  int32_t group_size;
} convrot_packed;

/*
 * Quantised weights of one linear layer, [ICS, Checkpoint format]: an int8
 * [out_features, in_features] matrix and one float scale per output row.
 *   q     : device int8 [n, k], row stride exactly k bytes
 *   scale : device float32 [n]
 *   bias  : device float32 [n], or NULL for no bias
 */
typedef struct convrot_weights {
  const int8_t* q;
  const float* scale;
  const float* bias;
  int64_t n;
  int64_t k;
  int32_t group_size;
} convrot_weights;

/*
 * Offline weight preparation, [ICS, How INT8 convrot works] (W_rot = W R) and
 * [ICS, Weight quantization]:
 *   s_w[o]    = max_i |W_rot[o, i]| / 127          (stored as float32)
 *   Q_w[o, i] = clamp(round(W_rot[o, i] / s_w[o]), -127, 127)
 * The rotation, absmax, division and rounding are done in float64; the float64
 * quotient max/127 is rounded once to float32 and the division uses that
 * stored float32 value.
 *   w         : device float32 [n, k], row stride ldw >= k (input, unchanged)
 *   q_out     : device int8 [n, k], row stride k (output)
 *   scale_out : device float32 [n] (output)
 * Errors: NULL, SHAPE, GROUP, UNSUPPORTED, HIP.
 */
convrot_status convrot_quantize_weights(const float* w, int64_t n, int64_t k, int64_t ldw,
                                        int32_t group_size, int8_t* q_out, float* scale_out,
                                        void* stream);

/*
 * Runtime activation rotation and quantisation into a packed activation,
 * [ICS, Runtime activation quantization]: each row of X is rotated group-wise
 * (X_rot = X R), then
 *   s_x[r]    = max_i |X_rot[r, i]| / 127
 *   Q_x[r, i] = clamp(round(X_rot[r, i] / s_x[r]), -127, 127)
 * in float32: the rotation is a radix-4 butterfly in float32; max/127 and
 * X_rot/s_x are correctly rounded float32 operations.  X is not modified (the
 * unrotated X stays available, e.g. for low-rank adapters).
 *   x       : device [m, k] of x_dtype (CONVROT_F32 or CONVROT_BF16), row stride ldx >= k
 *   out->q, out->scale : caller-allocated device buffers (see convrot_packed);
 *             on success the call sets out->m, out->k and out->group_size.
 * Errors: NULL, SHAPE, GROUP, DTYPE, UNSUPPORTED, HIP.
 */
convrot_status convrot_pack_activations(const void* x, int32_t x_dtype, int64_t m, int64_t k,
                                        int64_t ldx, int32_t group_size, convrot_packed* out,
                                        void* stream);

/*
 * The convrot linear on a packed activation, [ICS, Runtime activation
 * quantization]:
 *   A[r, o] = sum_i Q_x[r, i] Q_w[o, i]               (exact int32)
 *   Y[r, o] = A[r, o] * s_x[r] * s_w[o] + b[o]        (float32; then act)
 * y_dtype CONVROT_F32 writes Y (float32 [m, n], row stride ldy >= n; Y must
 * not overlap the inputs);
 * y_dtype CONVROT_I32 writes the raw int32 A (no scale, bias or act; act must
 * be CONVROT_ACT_NONE).  act CONVROT_ACT_GELU applies x*Phi(x) to Y.
 * The packed activation and the weights must have the same k and the same
 * group size ([ICS, Runtime activation quantization]: a packed tensor is
 * shared only by layers with the same input and group size).
 * Errors: NULL, SHAPE, GROUP_MISMATCH, DTYPE, UNSUPPORTED, HIP.
 */
convrot_status convrot_linear(const convrot_packed* x, const convrot_weights* w, void* y,
                              int32_t y_dtype, int64_t ldy, int32_t act, void* stream);

/*
 * Several convrot linears on ONE packed activation in one launch: the linear
 * layers that share an input and a group size reuse its packed tensor
 * ([ICS, Runtime activation quantization]), e.g. the Q, K and V projections
 * of an attention block.  Weight i writes y[i] (row stride ldy[i] >= w[i].n);
 * semantics per weight are those of convrot_linear, with one y_dtype and one
 * act for all.  Weights with n == 0 are skipped.  The outputs must not
 * overlap one another or any input (short outputs are accumulated in place,
 * as int32 partial sums, before they are scaled).
 *   w   : host array of `count` convrot_weights (device pointers inside)
 *   y   : host array of `count` device output pointers
 *   ldy : host array of `count` row strides
 *   1 <= count <= CONVROT_MAX_GROUPED
 * Errors: NULL, SHAPE, GROUP_MISMATCH, DTYPE, UNSUPPORTED, HIP.
 */
convrot_status convrot_linear_grouped(const convrot_packed* x, const convrot_weights* w,
                                      int32_t count, void* const* y, const int64_t* ldy,
                                      int32_t y_dtype, int32_t act, void* stream);

/*
 * Low-rank adapters ([ICS, Backend support]): LoRA-style adapters are applied
 * at run time without touching the int8 weights; the convrot linear gives the
 * base output and the adapter's correction, computed from the original
 * UNROTATED activation X, is added to it.  In the low-rank form, with down
 * weights A [rank, k], up weights B [n, rank] and a scale (alpha / rank):
 *   U = bf16(scale * X A^T)          (convrot_lora_down)
 *   Y += U B^T                       (fused: convrot_linear_lora;
 *                                     separate: convrot_lora_up_add)
 * Operands are bfloat16 with float32 accumulation; the scale is applied to
 * the float32 sum X A^T, which is then rounded to bfloat16 (nearest even).
 * (The page gives no formula or precision for the adapter path; this is the
 * library's reading.)
 */

/*
 * convrot_lora_down: U = bf16(scale * X A^T).
 *   x : device [m, k] of x_dtype (CONVROT_F32 or CONVROT_BF16), row stride
 *       k <= ldx <= 2^21; float32 X is rounded to bfloat16 (nearest even) first
 *   a : device bfloat16 [rank, k], row stride k
 *   u : device bfloat16 [m, ldu] (output; columns rank .. ldu-1 untouched, so
 *       several adapters' U can share one buffer)
 * Adapters with the same scale on the same X (the Q, K and V projections of
 * one block) can stack their A matrices, up to CONVROT_MAX_LORA_RANK rows in
 * all, into one call that reads X once and writes each adapter's U as a
 * column range of the shared buffer; each U column is computed the same way.
 *   rank a multiple of 16 in 16 .. CONVROT_MAX_LORA_RANK; k % 16 == 0;
 *   rank <= ldu <= 2^20 and ldu % 8 == 0;
 *   x, a, u 16-byte aligned, ldx in whole 16-byte units.
 * Errors: NULL, SHAPE, DTYPE, UNSUPPORTED, HIP.
 */
convrot_status convrot_lora_down(const void* x, int32_t x_dtype, int64_t m, int64_t k,
                                 int64_t ldx, const void* a, int32_t rank, float scale, void* u,
                                 int64_t ldu, void* stream);

/*
 * convrot_lora_up_add: Y[i, o] += sum_j U[i, j] B[o, j], a separate pass over Y.
 *   u : device bfloat16 [m, ldu] (from convrot_lora_down)
 *   b : device bfloat16 [n, rank], row stride rank
 *   y : device float32 [m, n], row stride ldy >= n (updated in place,
 *       typically the output of convrot_linear)
 *   rank and ldu as for convrot_lora_down; u and b 16-byte aligned, y 4-byte
 *   aligned; ceil(m / 128) * ceil(n / 128) <= INT32_MAX (128 x 128 tiles).
 * Errors: NULL, SHAPE, UNSUPPORTED, HIP.
 */
convrot_status convrot_lora_up_add(const void* u, int64_t ldu, const void* b, int64_t m,
                                   int64_t n, int32_t rank, float* y, int64_t ldy, void* stream);

/*
 * One weight's adapter for convrot_linear_lora.
 *   u    : device bfloat16 [m, ldu], this adapter's U from convrot_lora_down
 *   b    : device bfloat16 [n, rank], row stride rank
 *   ldu  : row stride of u in elements, rank <= ldu <= 2^20, ldu % 8 == 0
 *   rank : a multiple of 16 in 16 .. CONVROT_MAX_LORA_RANK, or 0 for a weight
 *          without an adapter (u, b and ldu are then ignored)
 */
typedef struct convrot_lora {
  const void* u;
  const void* b;
  int64_t ldu;
  int32_t rank;
} convrot_lora;

/*
 * convrot_linear_grouped (float32 output) with each weight's adapter added
 * in the GEMM epilogue, so Y is written once:
 *   Y_i = act(A_i s_x s_w,i + b_i + U_i B_i^T)
 * (act applies to the adapted output).  lora: host array of `count` adapters.
 * Errors: those of convrot_linear_grouped; SHAPE or UNSUPPORTED for an
 * adapter's rank, ldu or alignment; NULL for a missing u or b.
 */
convrot_status convrot_linear_lora(const convrot_packed* x, const convrot_weights* w,
                                   const convrot_lora* lora, int32_t count, void* const* y,
                                   const int64_t* ldy, int32_t act, void* stream);

/* A static, human-readable name for a status code (never NULL). */
const char* convrot_status_string(convrot_status status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t convrot_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_H */
