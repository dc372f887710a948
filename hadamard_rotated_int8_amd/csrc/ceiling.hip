// Measurement kernels for the hot path's rooflines (not on the hot path; built
// into libconvrot_ceiling.so, which only the benchmark loads): the matrix
// cores' rate for the INT8 GEMM and HBM's for the activation pack.
//
// A register-only loop of v_mfma_i32_32x32x32_i8 in the GEMM's per-wave shape:
// one workgroup of 4 waves per CU (one wave per SIMD), each wave keeping a
// 4 x 3 set of 32 x 32 accumulators (the GEMM's 128 x 96 wave tile) and two
// fragment sets that alternate from one 32-wide K slice to the next, as the
// GEMM's sub-steps do.  The fragments are read once from real operand rows
// (packed activation codes and weight codes), so the multipliers see
// code-shaped data: the chip's power draw, and with it the clock the matrix
// cores sustain, depends on the operand bits.  No loads, LDS traffic or
// stores run inside the loop, so its rate is the matrix cores' ceiling for
// this operand data at the clock the chip holds under it.
//
// A streaming pass with the pack's read:write mix: every 16-byte chunk of the
// destination receives the XOR of R source chunks (R = 2 for bf16 input and
// int8 output, 4 for float32 input), with non-temporal 16-byte loads and
// stores, grid-stride, each lane holding the loads of two destination chunks
// in flight before it stores them.  No arithmetic to speak of, so its rate is
// what HBM delivers to a pass that moves the pack's bytes in the pack's
// proportions.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/convrot_ceiling.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kFM = 4, kFN = 3, kSets = 2;

// Fragment (set s, block f) of a wave: lane l reads 16 bytes of row
// (32 * (wave * 8 + 4 * s + f) + l % 32) mod rows, at byte 64 * s + 16 * (l / 32)
// of the row (rows are at least 128 bytes, 16-byte aligned).
__device__ __forceinline__ v4i fragment(const int8_t* base, int64_t ld, int64_t rows, int wave,
                                        int s, int f, int lane) {
  const int64_t row = (int64_t(32) * (wave * 8 + 4 * s + f) + (lane & 31)) % rows;
  return *reinterpret_cast<const v4i*>(base + row * ld + 64 * s + 16 * (lane >> 5));
}

__global__ __launch_bounds__(256, 1) void mfma_loop_kernel(const int8_t* a, int64_t lda,
                                                          int64_t rows_a, const int8_t* b,
                                                          int64_t ldb, int64_t rows_b, int iters,
                                                          int* sink) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  v4i xf[kSets][kFM], wf[kSets][kFN];
#pragma unroll
  for (int s = 0; s < kSets; ++s) {
#pragma unroll
    for (int i = 0; i < kFM; ++i) xf[s][i] = fragment(a, lda, rows_a, wave, s, i, lane);
#pragma unroll
    for (int j = 0; j < kFN; ++j) wf[s][j] = fragment(b, ldb, rows_b, wave, s, j, lane);
  }
  v16i acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[i][j] = v16i{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < kSets; ++s)
#pragma unroll
      for (int i = 0; i < kFM; ++i)
#pragma unroll
        for (int j = 0; j < kFN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf[s][i], wf[s][j], acc[i][j], 0, 0, 0);
  }
  // Fold the accumulators into one value per lane so that no MFMA is dead code.
  int r = 0;
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) r ^= acc[i][j][e] + e;
  sink[int64_t(wave) * 64 + lane] = r;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Source plane j (j < R) holds chunks j * n16 .. j * n16 + n16 - 1, so every
// load instruction of a wave reads 1 KB contiguous.
template <int R>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4* __restrict__ src,
                                                    u32x4* __restrict__ dst, int64_t n16) {
  constexpr int kInFlight = 2;  // destination chunks per lane and round
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += kInFlight * stride) {
    u32x4 v[kInFlight][R];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int64_t c = i + u * stride;
#pragma unroll
      for (int j = 0; j < R; ++j)
        v[u][j] = c < n16 ? __builtin_nontemporal_load(src + j * n16 + c) : u32x4{};
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int64_t c = i + u * stride;
      u32x4 x = v[u][0];
#pragma unroll
      for (int j = 1; j < R; ++j) x ^= v[u][j];
      if (c < n16) __builtin_nontemporal_store(x, dst + c);
    }
  }
}

}  // namespace

extern "C" int32_t convrot_ceiling_stream(const void* src, void* dst, int64_t dst_bytes,
                                          int32_t ratio, int32_t grid, void* stream) {
  if (!src || !dst || dst_bytes < 16 || dst_bytes % 16) return -1;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) return -1;
  if (grid < 1 || grid > 65536) return -1;
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  const int64_t n16 = dst_bytes / 16;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  switch (ratio) {
    case 1: hipLaunchKernelGGL(stream_kernel<1>, dim3(grid), dim3(256), 0, st, s, d, n16); break;
    case 2: hipLaunchKernelGGL(stream_kernel<2>, dim3(grid), dim3(256), 0, st, s, d, n16); break;
    case 4: hipLaunchKernelGGL(stream_kernel<4>, dim3(grid), dim3(256), 0, st, s, d, n16); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int64_t convrot_ceiling_mfma_i8(const int8_t* a, int64_t lda, int64_t rows_a,
                                           const int8_t* b, int64_t ldb, int64_t rows_b,
                                           int32_t iters, int32_t grid, int32_t* sink,
                                           void* stream) {
  if (!a || !b || !sink) return -1;
  if (rows_a < 32 || rows_b < 32 || lda < 128 || ldb < 128 || lda % 16 || ldb % 16) return -1;
  if ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b)) & 15u) return -1;
  if (iters < 1 || grid < 1 || grid > 65536) return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a, lda, rows_a, b, ldb, rows_b, iters, sink);
  if (hipGetLastError() != hipSuccess) return -1;
  // int8 operations (a multiply-add counts 2) the launch performs
  return int64_t(grid) * 4 * iters * kSets * kFM * kFN * (int64_t(2) * 32 * 32 * 32);
}
