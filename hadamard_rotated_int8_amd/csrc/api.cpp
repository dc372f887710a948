// C ABI of libconvrot.so: argument validation and dispatch to the HIP kernels.
//
// Every check runs on the host before any HIP call, so an invalid call
// returns a status code and touches neither the GPU nor the HIP runtime.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/convrot.h"
#include "kernels.h"

namespace {

constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// log4 of a valid group size (1, 4, ..., 4^7), or -1.
int log4_of(int32_t g) {
  for (int n = 0; n <= CONVROT_MAX_LOG4_GROUP; ++n)
    if (g == (int32_t(1) << (2 * n))) return n;
  return -1;
}

convrot_status check_k_group(int64_t k, int32_t group_size, int* log4g) {
  if (k < 1 || k > CONVROT_MAX_K) return CONVROT_ERR_SHAPE;
  const int n = log4_of(group_size);
  if (n < 0 || k % group_size != 0) return CONVROT_ERR_GROUP;
  if (k % 16 != 0) return CONVROT_ERR_UNSUPPORTED;
  *log4g = n;
  return CONVROT_OK;
}

convrot_status from_hip(hipError_t e) { return e == hipSuccess ? CONVROT_OK : CONVROT_ERR_HIP; }

}  // namespace

namespace {

convrot_status check_out(int32_t y_dtype, int32_t act) {
  if (y_dtype != CONVROT_F32 && y_dtype != CONVROT_I32) return CONVROT_ERR_DTYPE;
  if (act != CONVROT_ACT_NONE && act != CONVROT_ACT_GELU) return CONVROT_ERR_DTYPE;
  if (y_dtype == CONVROT_I32 && act != CONVROT_ACT_NONE) return CONVROT_ERR_DTYPE;
  return CONVROT_OK;
}

// Validate one weight against the packed activation and fill its launch slot.
convrot_status check_weight(const convrot_packed* x, const convrot_weights* w, void* y,
                            int64_t ldy, int32_t y_dtype, convrot::GemmWeight* out) {
  if (!w) return CONVROT_ERR_NULL;
  if (w->k != x->k || w->group_size != x->group_size) return CONVROT_ERR_GROUP_MISMATCH;
  if (w->n < 0 || w->n > kMaxRows || ldy < w->n) return CONVROT_ERR_SHAPE;
  if (w->n > 0 && x->m > 0) {
    if (!w->q || !y) return CONVROT_ERR_NULL;
    if (y_dtype == CONVROT_F32 && !w->scale) return CONVROT_ERR_NULL;
    // y needs only its element alignment; 16-byte rows take the vector-store path.
    if (!aligned16(w->q) || (reinterpret_cast<uintptr_t>(y) & 3u) != 0)
      return CONVROT_ERR_UNSUPPORTED;
  }
  out->qw = w->q;
  out->sw = w->scale;
  out->bias = w->bias;
  out->y = y;
  out->n = w->n;
  out->ldy = ldy;
  return CONVROT_OK;
}

bool lora_rank_ok(int32_t rank) {
  return rank >= 16 && rank <= CONVROT_MAX_LORA_RANK && rank % 16 == 0;
}

// Validate one weight's adapter (rank 0: none) and fill its launch slot.
convrot_status check_lora(const convrot_lora* l, int64_t m, int64_t n, convrot::GemmWeight* out) {
  if (!l) return CONVROT_ERR_NULL;
  if (l->rank == 0) return CONVROT_OK;
  if (!lora_rank_ok(l->rank) || l->ldu < l->rank || l->ldu > convrot::kLoraMaxLdu)
    return CONVROT_ERR_SHAPE;
  if (l->ldu % 8 != 0) return CONVROT_ERR_UNSUPPORTED;
  if (m > 0 && n > 0) {
    if (!l->u || !l->b) return CONVROT_ERR_NULL;
    if (!aligned16(l->u) || !aligned16(l->b)) return CONVROT_ERR_UNSUPPORTED;
  }
  out->lu = static_cast<const uint16_t*>(l->u);
  out->lb = static_cast<const uint16_t*>(l->b);
  out->ldu = l->ldu;
  out->rank = l->rank;
  return CONVROT_OK;
}

// lora: NULL, or one adapter per weight (the float32-output fused path).
convrot_status run_linear(const convrot_packed* x, const convrot_weights* const* w, int32_t count,
                          void* const* y, const int64_t* ldy, int32_t y_dtype, int32_t act,
                          void* stream, const convrot_lora* lora = nullptr) {
  if (!x) return CONVROT_ERR_NULL;
  int log4g = 0;
  convrot_status st = check_k_group(x->k, x->group_size, &log4g);
  if (st != CONVROT_OK) return st;
  if (x->m < 0 || x->m > kMaxRows) return CONVROT_ERR_SHAPE;
  st = check_out(y_dtype, act);
  if (st != CONVROT_OK) return st;
  convrot::GemmArgs a;
  a.qx = x->q;
  a.sx = x->scale;
  a.m = x->m;
  a.k = x->k;
  a.count = 0;
  a.raw_i32 = (y_dtype == CONVROT_I32);
  a.gelu = (act == CONVROT_ACT_GELU);
  a.lora = lora != nullptr;
  for (int32_t i = 0; i < count; ++i) {
    a.w[a.count] = convrot::GemmWeight{};  // (a skipped empty weight may have filled it)
    st = check_weight(x, w[i], y[i], ldy[i], y_dtype, &a.w[a.count]);
    if (st != CONVROT_OK) return st;
    if (lora) {
      st = check_lora(&lora[i], x->m, w[i]->n, &a.w[a.count]);
      if (st != CONVROT_OK) return st;
    }
    if (w[i]->n > 0) ++a.count;  // empty weights launch nothing
  }
  // Adapters of rank 0 add nothing: with no adapter of higher rank the launch
  // is the plain one (same values bit for bit, and the short-output path
  // stays available).
  if (a.lora) {
    a.lora = false;
    for (int i = 0; i < a.count; ++i) a.lora = a.lora || a.w[i].rank > 0;
  }
  if (x->m == 0 || a.count == 0) return CONVROT_OK;
  // The persistent kernel numbers its 256 x 192 output tiles with 32-bit
  // integers (no buffer that large can exist, but the count is checked
  // rather than assumed).
  int64_t tiles = 0;
  for (int i = 0; i < a.count; ++i) tiles += (a.w[i].n + 191) / 192;
  if (tiles * ((x->m + 255) / 256) > int64_t(INT32_MAX)) return CONVROT_ERR_SHAPE;
  if (!x->q) return CONVROT_ERR_NULL;
  if (y_dtype == CONVROT_F32 && !x->scale) return CONVROT_ERR_NULL;
  if (!aligned16(x->q)) return CONVROT_ERR_UNSUPPORTED;
  return from_hip(convrot::launch_gemm(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char* convrot_status_string(convrot_status s) {
  switch (s) {
    case CONVROT_OK: return "ok";
    case CONVROT_ERR_NULL: return "a required pointer is NULL";
    case CONVROT_ERR_SHAPE: return "m, n or k out of range, or ld smaller than the row";
    case CONVROT_ERR_GROUP: return "group size is not a power of four in 1..16384 dividing k";
    case CONVROT_ERR_GROUP_MISMATCH: return "packed activation and weights differ in k or group size";
    case CONVROT_ERR_DTYPE: return "unsupported dtype or activation";
    case CONVROT_ERR_UNSUPPORTED: return "k % 16 != 0, or a pointer or stride is not 16-byte aligned";
    case CONVROT_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t convrot_version(void) { return 100; }

convrot_status convrot_quantize_weights(const float* w, int64_t n, int64_t k, int64_t ldw,
                                        int32_t group_size, int8_t* q_out, float* scale_out,
                                        void* stream) {
  int log4g = 0;
  const convrot_status st = check_k_group(k, group_size, &log4g);
  if (st != CONVROT_OK) return st;
  if (n < 0 || n > kMaxRows || ldw < k) return CONVROT_ERR_SHAPE;
  if (n == 0) return CONVROT_OK;
  if (!w || !q_out || !scale_out) return CONVROT_ERR_NULL;
  if (!aligned16(q_out)) return CONVROT_ERR_UNSUPPORTED;
  return from_hip(convrot::launch_wprep(w, n, k, ldw, log4g, q_out, scale_out,
                                        static_cast<hipStream_t>(stream)));
}

convrot_status convrot_pack_activations(const void* x, int32_t x_dtype, int64_t m, int64_t k,
                                        int64_t ldx, int32_t group_size, convrot_packed* out,
                                        void* stream) {
  if (!out) return CONVROT_ERR_NULL;
  int log4g = 0;
  const convrot_status st = check_k_group(k, group_size, &log4g);
  if (st != CONVROT_OK) return st;
  if (m < 0 || m > kMaxRows || ldx < k) return CONVROT_ERR_SHAPE;
  if (x_dtype != CONVROT_F32 && x_dtype != CONVROT_BF16) return CONVROT_ERR_DTYPE;
  if (m > 0 && (!x || !out->q || !out->scale)) return CONVROT_ERR_NULL;
  const int64_t esize = (x_dtype == CONVROT_F32) ? 4 : 2;
  if (m > 0 && (!aligned16(x) || !aligned16(out->q) || (ldx * esize) % 16 != 0))
    return CONVROT_ERR_UNSUPPORTED;
  out->m = m;
  out->k = k;
  out->group_size = group_size;
  if (m == 0) return CONVROT_OK;
  return from_hip(convrot::launch_pack(x, x_dtype == CONVROT_BF16, ldx, m, k, log4g, out->q,
                                       out->scale, static_cast<hipStream_t>(stream)));
}

convrot_status convrot_lora_down(const void* x, int32_t x_dtype, int64_t m, int64_t k,
                                 int64_t ldx, const void* a, int32_t rank, float scale, void* u,
                                 int64_t ldu, void* stream) {
  if (k < 1 || m < 0 || m > kMaxRows || ldx < k || ldx > convrot::kLoraMaxLdx ||
      !lora_rank_ok(rank) || ldu < rank || ldu > convrot::kLoraMaxLdu)
    return CONVROT_ERR_SHAPE;
  if (x_dtype != CONVROT_F32 && x_dtype != CONVROT_BF16) return CONVROT_ERR_DTYPE;
  if (k % 16 != 0 || ldu % 8 != 0) return CONVROT_ERR_UNSUPPORTED;
  if (m == 0) return CONVROT_OK;
  if (!x || !a || !u) return CONVROT_ERR_NULL;
  const int64_t esize = (x_dtype == CONVROT_F32) ? 4 : 2;
  if (!aligned16(x) || !aligned16(a) || !aligned16(u) || (ldx * esize) % 16 != 0)
    return CONVROT_ERR_UNSUPPORTED;
  return from_hip(convrot::launch_lora_down(x, x_dtype == CONVROT_BF16, ldx, m, k,
                                            static_cast<const uint16_t*>(a), rank, scale,
                                            static_cast<uint16_t*>(u), ldu,
                                            static_cast<hipStream_t>(stream)));
}

convrot_status convrot_lora_up_add(const void* u, int64_t ldu, const void* b, int64_t m,
                                   int64_t n, int32_t rank, float* y, int64_t ldy, void* stream) {
  if (m < 0 || m > kMaxRows || n < 0 || n > kMaxRows || ldy < n || !lora_rank_ok(rank) ||
      ldu < rank || ldu > convrot::kLoraMaxLdu)
    return CONVROT_ERR_SHAPE;
  if (ldu % 8 != 0) return CONVROT_ERR_UNSUPPORTED;
  if (m == 0 || n == 0) return CONVROT_OK;
  if (((m + 127) / 128) * ((n + 127) / 128) > INT32_MAX) return CONVROT_ERR_SHAPE;
  if (!u || !b || !y) return CONVROT_ERR_NULL;
  if (!aligned16(u) || !aligned16(b) || (reinterpret_cast<uintptr_t>(y) & 3u) != 0)
    return CONVROT_ERR_UNSUPPORTED;
  return from_hip(convrot::launch_lora_up_add(static_cast<const uint16_t*>(u), ldu,
                                              static_cast<const uint16_t*>(b), m, n, rank, y, ldy,
                                              static_cast<hipStream_t>(stream)));
}

convrot_status convrot_linear(const convrot_packed* x, const convrot_weights* w, void* y,
                              int32_t y_dtype, int64_t ldy, int32_t act, void* stream) {
  if (!x || !w) return CONVROT_ERR_NULL;
  const convrot_weights* ws[1] = {w};
  void* ys[1] = {y};
  const int64_t lds[1] = {ldy};
  return run_linear(x, ws, 1, ys, lds, y_dtype, act, stream);
}

convrot_status convrot_linear_grouped(const convrot_packed* x, const convrot_weights* w,
                                      int32_t count, void* const* y, const int64_t* ldy,
                                      int32_t y_dtype, int32_t act, void* stream) {
  if (!x || !w || !y || !ldy) return CONVROT_ERR_NULL;
  if (count < 1 || count > CONVROT_MAX_GROUPED) return CONVROT_ERR_SHAPE;
  const convrot_weights* ws[CONVROT_MAX_GROUPED];
  for (int32_t i = 0; i < count; ++i) ws[i] = &w[i];
  return run_linear(x, ws, count, y, ldy, y_dtype, act, stream);
}

convrot_status convrot_linear_lora(const convrot_packed* x, const convrot_weights* w,
                                   const convrot_lora* lora, int32_t count, void* const* y,
                                   const int64_t* ldy, int32_t act, void* stream) {
  if (!x || !w || !lora || !y || !ldy) return CONVROT_ERR_NULL;
  if (count < 1 || count > CONVROT_MAX_GROUPED) return CONVROT_ERR_SHAPE;
  const convrot_weights* ws[CONVROT_MAX_GROUPED];
  for (int32_t i = 0; i < count; ++i) ws[i] = &w[i];
  return run_linear(x, ws, count, y, ldy, CONVROT_F32, act, stream, lora);
}

}  // extern "C"
