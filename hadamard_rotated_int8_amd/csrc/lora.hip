// Low-rank adapter correction on the unrotated activation.
//
// The stable-diffusion.cpp page "INT8 Convrot Safetensors" (section "Backend
// support") applies LoRA-style adapters at run time: the convrot linear gives
// the base output, and the adapter's correction is computed from the
// original, unrotated activation X and added to it.  In the low-rank form,
// with down weights A [r, K], up weights B [N, r] and a scalar scale:
//   U = bf16(scale * X A^T)    (lora_down_kernel; bfloat16 [M, r])
//   Y[m, n] += U B^T           (lora_up_add_kernel, on the convrot output Y;
//                               the GEMM can also add it in its epilogue)
// Both are small dense contractions on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16, float32 accumulation).  Operands go straight
// from global memory (mostly L2: A, B and U are small) into the MFMA
// register layout -- each lane reads 16 contiguous bytes of one row -- so no
// LDS staging is needed for the operands.
#include "common.h"
#include "kernels.h"

namespace convrot {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kLoraMaxBlocks = kLoraMaxRank / 32;

// float32 -> bfloat16 bits, round to nearest even (finite inputs).
CR_DEVICE unsigned short bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (unsigned short)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

CR_DEVICE bf16x8 as_bf16x8(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight consecutive features of one row as MFMA operand bits (zero when the
// row or the features are out of range).
CR_DEVICE u16x8 load8(const uint16_t* __restrict__ p, bool ok) {
  if (!ok) return u16x8{};
  return __builtin_bit_cast(u16x8, *reinterpret_cast<const u32x4*>(p));
}
CR_DEVICE u16x8 load8(const float* __restrict__ p, bool ok) {
  u16x8 r{};
  if (!ok) return r;
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
  const f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
  r[0] = bf16_bits(a.x); r[1] = bf16_bits(a.y); r[2] = bf16_bits(a.z); r[3] = bf16_bits(a.w);
  r[4] = bf16_bits(b.x); r[5] = bf16_bits(b.y); r[6] = bf16_bits(b.z); r[7] = bf16_bits(b.w);
  return r;
}

// U[32-row block] = X A^T.  A workgroup of 4 waves owns 32 rows; the 16-wide
// K steps are dealt round robin over the waves, and the four partial sums
// are added in LDS in wave order (deterministic).  NB = ceil(r / 32) column
// blocks of U.  MFMA operand layout: lane l holds row l % 32, features
// 8 (l / 32) .. 8 (l / 32) + 7 of the step; accumulator register i of lane l
// is row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32.
template <typename InT, int NB>
__global__ __launch_bounds__(256) void lora_down_kernel(const InT* __restrict__ x, int64_t ldx,
                                                        int m, int k,
                                                        const uint16_t* __restrict__ a, int r,
                                                        float scale, uint16_t* __restrict__ u,
                                                        int64_t ldu) {
  __shared__ float part[4][NB][16][64];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = blockIdx.x * 32;
  const int lr = lane & 31, kh = (lane >> 5) * 8;
  const int row = row0 + lr;
  const InT* xr = x + (int64_t)(row < m ? row : 0) * ldx;
  f32x16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x16{};
  const int nsteps = (k + 15) / 16;
  for (int s = wave; s < nsteps; s += 4) {
    const int kk = s * 16 + kh;
    const bool kok = kk < k;  // k is a multiple of 16, so a lane's 8 features are all in or all out
    const bf16x8 xa = as_bf16x8(load8(xr + kk, kok && row < m));
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int ar = b * 32 + lr;
      const bf16x8 ab = as_bf16x8(load8(a + (int64_t)(ar < r ? ar : 0) * k + kk, kok && ar < r));
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa, ab, acc[b], 0, 0, 0);
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) part[wave][b][i][lane] = acc[b][i];
  __syncthreads();
  // Wave w finishes column blocks w, w + 4, ...: sum the four partials in
  // wave order, scale, round to bfloat16, store.
  for (int b = wave; b < NB; b += 4) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float v = scale * (((part[0][b][i][lane] + part[1][b][i][lane]) +
                                part[2][b][i][lane]) + part[3][b][i][lane]);
      const int orow = row0 + 8 * (i / 4) + 4 * (lane >> 5) + (i & 3);
      const int ocol = b * 32 + lr;
      if (orow < m && ocol < r) u[(int64_t)orow * ldu + ocol] = bf16_bits(v);
    }
  }
}

// Y[128 x 128 tile] += U B^T.  Each wave owns 64 x 64 (2 x 2 blocks of
// 32 x 32); the rank r is the contraction length (steps of 16).  The tile's
// Y values are read, updated and written back (float32).
__global__ __launch_bounds__(256) void lora_up_add_kernel(const uint16_t* __restrict__ u,
                                                          const uint16_t* __restrict__ bw,
                                                          int64_t ldu, int m, int n, int r,
                                                          float* __restrict__ y, int64_t ldy) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tiles_n = (n + 127) / 128;
  const int m0 = int(blockIdx.x / unsigned(tiles_n)) * 128 + (wave >> 1) * 64;
  const int n0 = int(blockIdx.x % unsigned(tiles_n)) * 128 + (wave & 1) * 64;
  const int lr = lane & 31, kh = (lane >> 5) * 8;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  for (int k0 = 0; k0 < r; k0 += 16) {  // uniform trip count (r % 16 == 0)
    const int kk = k0 + kh;
    bf16x8 ua[2], bb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = m0 + i * 32 + lr;
      ua[i] = as_bf16x8(load8(u + (int64_t)(row < m ? row : 0) * ldu + kk, row < m));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + j * 32 + lr;
      bb[j] = as_bf16x8(load8(bw + (int64_t)(col < n ? col : 0) * r + kk, col < n));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ua[i], bb[j], acc[i][j], 0, 0, 0);
  }
  // Read every Y value of the wave first, then update and write.
  float yv[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + i * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e & 3);
        const int col = n0 + j * 32 + lr;
        yv[i][j][e] = (row < m && col < n) ? y[(int64_t)row * ldy + col] : 0.f;
      }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + i * 32 + 8 * (e / 4) + 4 * (lane >> 5) + (e & 3);
        const int col = n0 + j * 32 + lr;
        if (row < m && col < n)
          y[(int64_t)row * ldy + col] = yv[i][j][e] + acc[i][j][e];
      }
}

template <typename InT, int NB>
hipError_t launch_down_t(const void* x, int64_t ldx, int m, int k, const uint16_t* a, int r,
                         float scale, uint16_t* u, int64_t ldu, hipStream_t stream) {
  const int grid = (m + 31) / 32;
  hipLaunchKernelGGL((lora_down_kernel<InT, NB>), dim3(grid), dim3(256), 0, stream,
                     static_cast<const InT*>(x), ldx, m, k, a, r, scale, u, ldu);
  return hipGetLastError();
}

template <typename InT>
hipError_t launch_down(const void* x, int64_t ldx, int m, int k, const uint16_t* a, int r,
                       float scale, uint16_t* u, int64_t ldu, hipStream_t stream) {
  switch ((r + 31) / 32) {
    case 1: return launch_down_t<InT, 1>(x, ldx, m, k, a, r, scale, u, ldu, stream);
    case 2: return launch_down_t<InT, 2>(x, ldx, m, k, a, r, scale, u, ldu, stream);
    case 3: return launch_down_t<InT, 3>(x, ldx, m, k, a, r, scale, u, ldu, stream);
    case 4: return launch_down_t<InT, 4>(x, ldx, m, k, a, r, scale, u, ldu, stream);
    default: return hipErrorInvalidValue;
  }
}
static_assert(kLoraMaxBlocks == 4, "launch_down covers 1..4 column blocks");

}  // namespace

hipError_t launch_lora_down(const void* x, bool bf16, int64_t ldx, int64_t m, int64_t k,
                            const uint16_t* a, int r, float scale, uint16_t* u, int64_t ldu,
                            hipStream_t stream) {
  return bf16 ? launch_down<uint16_t>(x, ldx, int(m), int(k), a, r, scale, u, ldu, stream)
              : launch_down<float>(x, ldx, int(m), int(k), a, r, scale, u, ldu, stream);
}

hipError_t launch_lora_up_add(const uint16_t* u, int64_t ldu, const uint16_t* b, int64_t m,
                              int64_t n, int r, float* y, int64_t ldy, hipStream_t stream) {
  const int64_t tiles = ((m + 127) / 128) * ((n + 127) / 128);
  if (tiles > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lora_up_add_kernel, dim3(unsigned(tiles)), dim3(256), 0, stream, u, b, ldu,
                     int(m), int(n), r, y, ldy);
  return hipGetLastError();
}

}  // namespace convrot
