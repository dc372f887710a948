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
// (v_mfma_f32_32x32x16_bf16, float32 accumulation).  The down projection
// streams X from HBM through LDS stages filled by direct-to-LDS loads (A is
// small and stays in L2): 32 x 32 blocks of U with K split over the waves
// for short X, 128-row blocks for long X.  The up-add pass takes U and B
// (small, L2-resident) straight from global memory into the MFMA registers.
#include "common.h"
#include "kernels.h"

namespace convrot {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));

// float32 -> bfloat16 bits, round to nearest even (v_cvt_pk_bf16_f32).
CR_DEVICE unsigned short bf16_bits(float f) {
  const bf16x2 r = __builtin_convertvector(f32x2{f, 0.f}, bf16x2);
  return __builtin_bit_cast(unsigned short, r.x);
}

CR_DEVICE bf16x8 as_bf16x8(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight consecutive features of one row as MFMA operand bits (zero when the
// row or the features are out of range).
CR_DEVICE u16x8 load8(const uint16_t* __restrict__ p, bool ok) {
  if (!ok) return u16x8{};
  return __builtin_bit_cast(u16x8, *reinterpret_cast<const u32x4*>(p));
}

// U[32 x 32 block] = bf16(scale * X A^T).  The workgroup's 4 waves share the
// 64-wide K blocks round robin and add their partial sums in LDS in wave
// order (deterministic).  Blocks are numbered column block fastest and dealt
// XCD by XCD, so the column blocks of one row block read X through one L2.
//
// Each wave streams its K blocks through a private ring of D LDS stages by
// direct-to-LDS buffer loads: 16 bytes per lane with consecutive lanes on
// consecutive 16-byte chunks of a row, so every instruction reads whole
// 128-byte lines.  The resources span the block's valid rows and features
// past k are given an out-of-range offset, so both read as zero.  Chunk c
// of stage row r sits at slot c ^ swz(r), which spreads the 16 rows a
// quarter-wave reads over all LDS banks.
//
// MFMA operands: for K block kb, lane l (row l % 32 of the block, h = l / 32)
// takes features 32h + 8c .. +7 of the block in MFMA c (c = 0..3); X and A use
// the same assignment, so the four MFMAs sum over all 64 features.
// Accumulator register i of lane l is row 8 (i / 4) + 4 (l / 32) + i % 4,
// column l % 32 of the 32 x 32 block.
template <typename InT, int D>
__global__ __launch_bounds__(256) void lora_down_kernel(const InT* __restrict__ x, int64_t ldx,
                                                        int m, int k,
                                                        const uint16_t* __restrict__ a, int r,
                                                        float scale, uint16_t* __restrict__ u,
                                                        int64_t ldu, int ncb) {
  constexpr int ES = sizeof(InT);
  constexpr int XROW = 64 * ES;           // bytes of X per row and K block
  constexpr int XCH = XROW / 16;          // 16-byte chunks per X row (8 or 16)
  constexpr int XST = 32 * XROW;          // X bytes per stage
  constexpr int STAGE = XST + 32 * 128;   // + A (32 rows x 128 bytes)
  constexpr int XL = XST / 1024, AL = 4;  // load instructions per stage
  constexpr int LPB = XL + AL;
  static_assert((D - 1) * LPB <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) int8_t smem[4 * D * STAGE];
  static_assert(4 * D * STAGE >= 4 * 16 * 64 * 4, "the reduction reuses the stages");

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nrb = (m + 31) / 32;
  const int pos = xcd_slot(blockIdx.x, nrb * ncb);
  const int row0 = (pos / ncb) * 32, col0 = (pos % ncb) * 32;
  const int rows = m - row0 < 32 ? m - row0 : 32;
  const int cols = r - col0 < 32 ? r - col0 : 32;
  const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(x + (int64_t)row0 * ldx, int(rows * ldx * ES));
  const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(a + (int64_t)col0 * k, cols * k * 2);
  const int nkb = (k + 63) / 64;
  const int T = nkb > wave ? (nkb - wave + 3) / 4 : 0;  // this wave's K blocks: wave + 4t
  int8_t* ring = smem + wave * D * STAGE;

  // X rows: lane j of load instruction q fills stage row q*(64/XCH) + j/XCH,
  // slot j%XCH, with global chunk slot ^ swz(row).  Same for A (8 chunks).
  auto xswz = [](int row) { return XCH == 8 ? (row >> 1) & 7 : row & 15; };
  auto aswz = [](int row) { return (row >> 1) & 7; };
  auto issue = [&](int st, int t) {
    const int f0 = (wave + 4 * t) * 64;  // first feature of the K block
    int8_t* xs = ring + st * STAGE;
#pragma unroll
    for (int q = 0; q < XL; ++q) {
      const int row = q * (64 / XCH) + lane / XCH;
      const int ch = (lane % XCH) ^ xswz(row);
      const int f = f0 + ch * (16 / ES);
      const unsigned off = f < k ? unsigned(row * ldx * ES + f * ES) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)(xs + q * 1024), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < AL; ++q) {
      const int row = q * 8 + lane / 8;
      const int ch = (lane % 8) ^ aswz(row);
      const int f = f0 + ch * 8;
      const unsigned off = f < k ? unsigned(row * k * 2 + f * 2) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void*)(xs + XST + q * 1024), 16, off, 0,
                                               0, 0);
    }
  };
  const int lr = lane & 31, h = lane >> 5;
  auto x_operand = [&](const int8_t* xs, int c) -> bf16x8 {
    if constexpr (ES == 2) {
      const int ch = (4 * h + c) ^ xswz(lr);
      return *reinterpret_cast<const bf16x8*>(xs + lr * XROW + ch * 16);
    } else {
      const int c0 = (8 * h + 2 * c) ^ xswz(lr), c1 = (8 * h + 2 * c + 1) ^ xswz(lr);
      const f32x4 lo = *reinterpret_cast<const f32x4*>(xs + lr * XROW + c0 * 16);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(xs + lr * XROW + c1 * 16);
      const bf16x2 p0 = __builtin_convertvector(f32x2{lo.x, lo.y}, bf16x2);
      const bf16x2 p1 = __builtin_convertvector(f32x2{lo.z, lo.w}, bf16x2);
      const bf16x2 p2 = __builtin_convertvector(f32x2{hi.x, hi.y}, bf16x2);
      const bf16x2 p3 = __builtin_convertvector(f32x2{hi.z, hi.w}, bf16x2);
      return bf16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    }
  };
  auto a_operand = [&](const int8_t* as, int c) -> bf16x8 {
    const int ch = (4 * h + c) ^ aswz(lr);
    return *reinterpret_cast<const bf16x8*>(as + lr * 128 + ch * 16);
  };

  f32x16 acc = {};
  auto consume = [&](int st) {
    const int8_t* xs = ring + st * STAGE;
    bf16x8 xo[4], ao[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      xo[c] = x_operand(xs, c);
      ao[c] = a_operand(xs + XST, c);
    }
    wait_lgkm0();
    return [=, &acc]() {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xo[c], ao[c], acc, 0, 0, 0);
    };
  };
#pragma unroll
  for (int st = 0; st < D; ++st) issue(st, st);
  // Rounds of D blocks; blocks past the wave's last one read as zero.  For
  // each stage: wait until only the later stages' loads are in flight, read
  // the fragments, and once they are in registers refill the stage D blocks
  // ahead.  The last round refills nothing, so its waits count down.
  const int rounds = (T + D - 1) / D;
  for (int rd = 0; rd + 1 < rounds; ++rd) {
#pragma unroll
    for (int st = 0; st < D; ++st) {
      waitvm<(D - 1) * LPB>();
      auto mfmas = consume(st);
      __builtin_amdgcn_sched_barrier(0);
      issue(st, rd * D + st + D);
      __builtin_amdgcn_sched_barrier(0);
      mfmas();
    }
  }
  if (rounds > 0) {
    for_each_index(std::make_integer_sequence<int, D>{}, [&](auto stc) {
      constexpr int st = decltype(stc)::value;
      waitvm<(D - 1 - st) * LPB>();
      consume(st)();
    });
  }
  waitvm<0>();  // (a wave without blocks still has its first stages in flight)
  __syncthreads();
  float* part = reinterpret_cast<float*>(smem);  // [4][16][64]
#pragma unroll
  for (int i = 0; i < 16; ++i) part[(wave * 16 + i) * 64 + lane] = acc[i];
  __syncthreads();
  // Wave w finishes registers 4w .. 4w+3: the four partials in wave order,
  // scaled, rounded to bfloat16.
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int i = 4 * wave + ii;
    const float v = scale * (((part[i * 64 + lane] + part[(16 + i) * 64 + lane]) +
                              part[(32 + i) * 64 + lane]) + part[(48 + i) * 64 + lane]);
    const int orow = row0 + 8 * (i / 4) + 4 * h + (i & 3);
    const int ocol = col0 + lr;
    if (orow < m && ocol < r) u[(int64_t)orow * ldu + ocol] = bf16_bits(v);
  }
}

// U[128 x 32 NB block] = bf16(scale * X A^T) for long X (many row blocks):
// each wave owns 32 rows and all NB column blocks of U, so A is read once
// per 128 rows and X once per row.  The 4 waves share a ring of D LDS
// stages (X rows of the block and A rows, 64 features each), filled by
// direct-to-LDS loads spread over the waves; one barrier per K block.
// Operand assignment, swizzle and zero fill as in lora_down_kernel.
template <typename InT, int NB, int D>
__global__ __launch_bounds__(256) void lora_down_rows_kernel(const InT* __restrict__ x,
                                                             int64_t ldx, int m, int k,
                                                             const uint16_t* __restrict__ a,
                                                             int r, float scale,
                                                             uint16_t* __restrict__ u,
                                                             int64_t ldu) {
  constexpr int ES = sizeof(InT);
  constexpr int XROW = 64 * ES;           // bytes of X per row and K block
  constexpr int XCH = XROW / 16;          // 16-byte chunks per X row
  constexpr int XST = 128 * XROW;         // X bytes per stage
  constexpr int STAGE = XST + 32 * NB * 128;
  constexpr int XL = XST / 1024 / 4;      // X load instructions per wave and stage
  constexpr int AL = NB;                  // A load instructions per wave and stage
  constexpr int LPW = XL + AL;
  static_assert((D - 2) * LPW <= 63 && D >= 2, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) int8_t smem[D * STAGE];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = xcd_slot(blockIdx.x, gridDim.x) * 128;
  const int rows = m - row0 < 128 ? m - row0 : 128;
  const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(x + (int64_t)row0 * ldx, int(rows * ldx * ES));
  const __amdgpu_buffer_rsrc_t ar = buffer_rsrc(a, r * k * 2);
  const int nkb = (k + 63) / 64;
  auto xswz = [](int row) { return XCH == 8 ? (row >> 1) & 7 : row & 15; };
  auto aswz = [](int row) { return (row >> 1) & 7; };
  // Load instruction q of a stage (1 KB) is issued by wave q % 4.
  auto issue = [&](int t) {
    const int f0 = t * 64;
    int8_t* st = smem + (t % D) * STAGE;
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int q = wave + 4 * i;
      const int row = q * (64 / XCH) + lane / XCH;
      const int ch = (lane % XCH) ^ xswz(row);
      const int f = f0 + ch * (16 / ES);
      const unsigned off = f < k ? unsigned(row * ldx * ES + f * ES) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)(st + q * 1024), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int q = wave + 4 * i;
      const int row = q * 8 + lane / 8;
      const int ch = (lane % 8) ^ aswz(row);
      const int f = f0 + ch * 8;
      const unsigned off = f < k ? unsigned(row * k * 2 + f * 2) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, (lds_void*)(st + XST + q * 1024), 16, off, 0,
                                               0, 0);
    }
  };
  const int lr = lane & 31, h = lane >> 5;
  const int xrow = wave * 32 + lr;
  auto x_operand = [&](const int8_t* xs, int c) -> bf16x8 {
    if constexpr (ES == 2) {
      const int ch = (4 * h + c) ^ xswz(xrow);
      return *reinterpret_cast<const bf16x8*>(xs + xrow * XROW + ch * 16);
    } else {
      const int c0 = (8 * h + 2 * c) ^ xswz(xrow), c1 = (8 * h + 2 * c + 1) ^ xswz(xrow);
      const f32x4 lo = *reinterpret_cast<const f32x4*>(xs + xrow * XROW + c0 * 16);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(xs + xrow * XROW + c1 * 16);
      const bf16x2 p0 = __builtin_convertvector(f32x2{lo.x, lo.y}, bf16x2);
      const bf16x2 p1 = __builtin_convertvector(f32x2{lo.z, lo.w}, bf16x2);
      const bf16x2 p2 = __builtin_convertvector(f32x2{hi.x, hi.y}, bf16x2);
      const bf16x2 p3 = __builtin_convertvector(f32x2{hi.z, hi.w}, bf16x2);
      return bf16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    }
  };
  auto a_operand = [&](const int8_t* as, int b, int c) -> bf16x8 {
    const int row = b * 32 + lr;
    const int ch = (4 * h + c) ^ aswz(row);
    return *reinterpret_cast<const bf16x8*>(as + row * 128 + ch * 16);
  };

  f32x16 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x16{};
#pragma unroll
  for (int t = 0; t < D - 1; ++t) issue(t);
  for (int t = 0; t < nkb; ++t) {
    // This wave's loads of stage t have landed once only those of the D - 2
    // later stages may be in flight; after the barrier everybody's have, and
    // everybody has finished with stage t - 1, whose slot is refilled.
    waitvm<(D - 2) * LPW>();
    barrier();
    issue(t + D - 1);  // past the last block: out of range, reads zeros
    const int8_t* st = smem + (t % D) * STAGE;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 xo = x_operand(st, c);
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xo, a_operand(st + XST, b, c), acc[b],
                                                         0, 0, 0);
    }
  }
  waitvm<0>();
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int orow = row0 + wave * 32 + 8 * (i / 4) + 4 * h + (i & 3);
      const int ocol = b * 32 + lr;
      if (orow < m && ocol < r) u[(int64_t)orow * ldu + ocol] = bf16_bits(scale * acc[b][i]);
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
hipError_t launch_down_rows(const void* x, int64_t ldx, int m, int k, const uint16_t* a, int r,
                            float scale, uint16_t* u, int64_t ldu, hipStream_t stream) {
  // As many stages of (X 128 rows + A 32 NB rows) x 64 features as fit in
  // 160 KB, at most 4.
  constexpr int STAGE = 128 * 64 * int(sizeof(InT)) + 32 * NB * 128;
  constexpr int D = (160 * 1024 / STAGE) < 4 ? (160 * 1024 / STAGE) : 4;
  const int blocks = (m + 127) / 128;
  hipLaunchKernelGGL((lora_down_rows_kernel<InT, NB, D>), dim3(blocks), dim3(256), 0, stream,
                     static_cast<const InT*>(x), ldx, m, k, a, r, scale, u, ldu);
  return hipGetLastError();
}

template <typename InT>
hipError_t launch_down(const void* x, int64_t ldx, int m, int k, const uint16_t* a, int r,
                       float scale, uint16_t* u, int64_t ldu, hipStream_t stream) {
  // Long X (a 128-row block for every CU): one workgroup per 128 rows and all
  // of U's columns (up to 8 blocks of 32: 128 accumulator registers per
  // lane; a bf16 stage is 48 KB, a float32 one 64 KB).  Otherwise 32 x 32
  // blocks of U, K split over waves.
  if ((m + 127) / 128 >= device_cu_count()) {
    switch ((r + 31) / 32) {
      case 1: return launch_down_rows<InT, 1>(x, ldx, m, k, a, r, scale, u, ldu, stream);
      case 2: return launch_down_rows<InT, 2>(x, ldx, m, k, a, r, scale, u, ldu, stream);
      case 3: return launch_down_rows<InT, 3>(x, ldx, m, k, a, r, scale, u, ldu, stream);
      case 4: return launch_down_rows<InT, 4>(x, ldx, m, k, a, r, scale, u, ldu, stream);
      case 5: return launch_down_rows<InT, 5>(x, ldx, m, k, a, r, scale, u, ldu, stream);
      case 6: return launch_down_rows<InT, 6>(x, ldx, m, k, a, r, scale, u, ldu, stream);
      case 7: return launch_down_rows<InT, 7>(x, ldx, m, k, a, r, scale, u, ldu, stream);
      case 8: return launch_down_rows<InT, 8>(x, ldx, m, k, a, r, scale, u, ldu, stream);
      default: return hipErrorInvalidValue;
    }
  }
  const int ncb = (r + 31) / 32;
  const int64_t blocks = int64_t((m + 31) / 32) * ncb;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  constexpr int D = sizeof(InT) == 2 ? 4 : 3;  // LDS stages per wave (128 KB / 144 KB)
  hipLaunchKernelGGL((lora_down_kernel<InT, D>), dim3(unsigned(blocks)), dim3(256), 0, stream,
                     static_cast<const InT*>(x), ldx, m, k, a, r, scale, u, ldu, ncb);
  return hipGetLastError();
}
static_assert(kLoraMaxRank % 16 == 0 && kLoraMaxRank <= 8 * 32,
              "ranks are multiples of 16, at most 8 blocks of 32 U columns");

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
