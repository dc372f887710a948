// INT8 GEMM for outputs with few tiles (short M): split K.
//
// The same computation as gemm.hip, from the stable-diffusion.cpp page
// "INT8 Convrot Safetensors", section "Runtime activation quantization":
//   A[r, o] = sum_i Q_x[r, i] Q_w[o, i]   (int32),  Y = A s_x[r] s_w[o] + b[o].
// The persistent kernel's 256 x 192 tiles leave most of the 256 CUs idle
// when M is a few hundred rows (a 256 x 4096 x 4096 linear has 22 tiles).
// Here the output is cut into 64 x 128 tiles (64 x 64 when that still gives
// no more work items than CUs) and K into equal slices, so that there is
// about one work item per CU:
//   1. zero_kernel clears Y (viewed as int32);
//   2. gemm_split_kernel computes one tile over one K slice and adds its
//      int32 partial sums into Y with atomic adds.  Integer addition is exact
//      and associative, so the result does not depend on the order in which
//      the slices arrive;
//   3. scale_kernel turns each int32 A into A s_x s_w + b in place (the same
//      float32 expression as the persistent kernel's epilogue), then GELU
//      when asked.  With int32 output the last step is skipped.
// With a single slice (tiny outputs, where the extra launches dominate) the
// kernel stores the finished values itself and steps 1 and 3 are skipped.
// Operands are staged through LDS by direct-to-LDS loads of whole 128-byte
// lines, swizzled like the persistent kernel's stages (chunk c of row r at
// slot c ^ (r & 7) ^ ((r >> 3) & 1)), double-buffered (the next step's lines
// load while this step's MFMAs run) with one barrier per 128-byte K step.
// Three, four or six stages measured no faster on any short output; a
// second wave per SIMD did (see the wave layout below).  Rows past M or n
// and bytes past K read as zero.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kSM = 64;                 // tile rows (Q_x)
constexpr int kSK = 128;                // K bytes per step
constexpr int kSStages = 2;
constexpr int kXBytes = kSM * kSK;      // 8 KB

// Tile columns (Q_w rows) SN = 128, or 64 when the wider tiles would leave
// most CUs idle.
template <int SN>
struct SplitCfg {
  static constexpr int kStage = kXBytes + SN * kSK;   // + 8 or 16 KB
  static constexpr int kPieces = kStage / 1024;       // 1 KB direct-to-LDS loads per stage
  static constexpr int kWaves = SN / 16;              // 4 or 8, one 32 x 32 block each
  static constexpr int kLoadsPerWave = kPieces / kWaves;
  static_assert(SN == 64 || SN == 128, "tile columns");
  static_assert(kPieces % kWaves == 0, "pieces split evenly over the waves");
  static_assert((kSStages - 2) * kLoadsPerWave <= kVmMax, "vmcnt range");
};

struct SplitSeg {
  const int8_t* qw;
  const float* sw;   // direct mode: column scales and bias (or null)
  const float* bias;
  int* acc;        // Y viewed as int32
  int64_t ld;      // row stride of Y (elements)
  int n;
  int tiles_n;
  int item0;       // first work item of this weight
};

struct SplitParams {
  const int8_t* qx;
  const float* sx;   // direct mode: row scales
  int M, K;
  int steps;       // K steps per slice
  int slices, tiles_m, nseg;
  SplitSeg seg[kMaxGemmGroup];
};

CR_DEVICE int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Work items are numbered weight, tile column, slice, tile row (fastest),
// and dealt XCD by XCD, so the tile rows that read one slice of Q_w share
// an L2.
// MODE 0: add int32 partial sums atomically; one slice only: 1 stores float32
// A s_x s_w + b, 2 the same through GELU, 3 the int32 A.
template <int MODE, int SN>
__global__ __launch_bounds__(SN * 4) void gemm_split_kernel(const SplitParams p) {
  using C = SplitCfg<SN>;
  constexpr int kStage = C::kStage, kLoadsPerWave = C::kLoadsPerWave, kWaves = C::kWaves;
  __shared__ __attribute__((aligned(1024))) int8_t smem[kSStages * kStage];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = xcd_slot(blockIdx.x, gridDim.x);
  int s = 0;
  for (int i = 1; i < p.nseg; ++i)
    if (item >= p.seg[i].item0) s = i;
  const SplitSeg& sg = p.seg[s];
  const int local = item - sg.item0;
  const int tm = local % p.tiles_m;
  const int rest = local / p.tiles_m;
  const int slice = rest % p.slices;
  const int tn = rest / p.slices;
  const int m0 = tm * kSM, n0 = tn * SN;
  const int K = p.K;
  const int rows = p.M - m0 < kSM ? p.M - m0 : kSM;
  const int cols = sg.n - n0 < SN ? sg.n - n0 : SN;
  const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(p.qx + (int64_t)m0 * K, rows * K);
  const __amdgpu_buffer_rsrc_t wr = buffer_rsrc(sg.qw + (int64_t)n0 * K, cols * K);
  const int kb0 = slice * p.steps * kSK;  // first K byte of the slice

  // Piece q (1 KB: rows 8q .. 8q+7 of the stage; Q_x pieces first) is loaded
  // by wave q % kWaves.  Lane j fills slot j % 8 of row j / 8 with global chunk
  // (j % 8) ^ swz(row).  Steps past the slice read the next slice's bytes
  // into stages that are never consumed; bytes past K read as zero.
  auto issue = [&](int t) {
    int8_t* st = smem + (t % kSStages) * kStage;
    const int kk = kb0 + t * kSK;
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      const int q = wave + kWaves * i;
      const bool is_x = q < kXBytes / 1024;
      const int row = (is_x ? q : q - kXBytes / 1024) * 8 + lane / 8;
      const int chunk = (lane & 7) ^ swz(row);
      const int kc = kk + chunk * 16;
      const unsigned off = kc < K ? unsigned(row * K + kc) : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(is_x ? xr : wr, (lds_void*)(st + q * 1024), 16, off,
                                               0, 0, 0);
    }
  };

  // Wave (wm, wn) = (wave / (SN / 32), wave % (SN / 32)) owns rows
  // 32 wm .. +31 and columns 32 wn .. +31 of the tile: one block of 32 x 32
  // accumulators (eight waves for 64 x 128 tiles, two per SIMD, so one
  // wave's waits are covered by the other's MFMAs: 512 x 3072 x 3072 in 15.1
  // us instead of 18.9 with four waves of two blocks).  Lane l reads row
  // l % 32 of a block, 16-byte chunk 2 kk + l / 32 of the step's K slice kk.
  const int wm = wave / (SN / 32), wn = wave % (SN / 32);
  const int fr = lane & 31, fh = lane >> 5;
  v16i acc = {};
#pragma unroll
  for (int t = 0; t < kSStages - 1; ++t) issue(t);
  for (int t = 0; t < p.steps; ++t) {
    // This wave's pieces of stage t have landed once only those of the
    // stages after it may be in flight; after the barrier everybody's have,
    // and stage t - 1 is free for the refill.
    waitvm<(kSStages - 2) * kLoadsPerWave>();
    barrier();
    issue(t + kSStages - 1);
    const int8_t* st = smem + (t % kSStages) * kStage;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int xrow = wm * 32 + fr;
      const v4i xf = *reinterpret_cast<const v4i*>(st + xrow * kSK + (((2 * kk + fh) ^ swz(xrow)) << 4));
      const int wrow = wn * 32 + fr;
      const v4i wf = *reinterpret_cast<const v4i*>(st + kXBytes + wrow * kSK +
                                                   (((2 * kk + fh) ^ swz(wrow)) << 4));
      acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf, wf, acc, 0, 0, 0);
    }
  }
  waitvm<0>();  // no load into LDS may still be in flight at exit
  // Accumulator register i of lane l: row 8 (i / 4) + 4 (l / 32) + i % 4,
  // column l % 32 of the block.
  const int col = n0 + wn * 32 + fr;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = m0 + wm * 32 + 8 * (i / 4) + 4 * fh + (i & 3);
    if (row < p.M && col < sg.n) {
      if constexpr (MODE == 0) {
        atomicAdd(sg.acc + (int64_t)row * sg.ld + col, acc[i]);
      } else if constexpr (MODE == 3) {
        sg.acc[(int64_t)row * sg.ld + col] = acc[i];
      } else {
        float v = __builtin_fmaf((float)acc[i] * p.sx[row], sg.sw[col],
                                 sg.bias ? sg.bias[col] : 0.f);
        if constexpr (MODE == 2) v = gelu_erf(v);
        reinterpret_cast<float*>(sg.acc)[(int64_t)row * sg.ld + col] = v;
      }
    }
  }
}

// Y[r, c] = 0 for r < m, c < n (row stride ld), grid-stride over rows.
__global__ __launch_bounds__(256) void zero_kernel(int* __restrict__ y, int64_t ld, int m, int n) {
  for (int r = blockIdx.y; r < m; r += gridDim.y)
    for (int c = blockIdx.x * 256 + threadIdx.x; c < n; c += gridDim.x * 256)
      y[(int64_t)r * ld + c] = 0;
}

// Y[r, c] = act(float(A[r, c]) s_x[r] s_w[c] + b[c]) in place.
template <bool GELU>
__global__ __launch_bounds__(256) void scale_kernel(float* __restrict__ y, int64_t ld, int m, int n,
                                                    const float* __restrict__ sx,
                                                    const float* __restrict__ sw,
                                                    const float* __restrict__ bias) {
  for (int r = blockIdx.y; r < m; r += gridDim.y) {
    const float s = sx[r];
    for (int c = blockIdx.x * 256 + threadIdx.x; c < n; c += gridDim.x * 256) {
      float* yp = y + (int64_t)r * ld + c;
      const int a = __float_as_int(*yp);
      float v = __builtin_fmaf((float)a * s, sw[c], bias ? bias[c] : 0.f);
      if (GELU) v = gelu_erf(v);
      *yp = v;
    }
  }
}

dim3 elementwise_grid(int64_t m, int64_t n) {
  const int64_t gx = (n + 255) / 256 < 16 ? (n + 255) / 256 : 16;
  const int64_t gy = m < 4096 ? m : 4096;
  return dim3(unsigned(gx), unsigned(gy));
}

}  // namespace

// Pick the path from estimates fitted to MI355X measurements of the kernels
// at short M (16 .. 768 rows, K 1024 .. 12288, N 512 .. 13824): the
// persistent kernel takes about 3 us + 1.2 us per 128-byte K step for each
// round of 256 x 192 tiles over the CUs; the split path with atomic partial
// sums about 8 us (three launches) plus its operand intake (every 64 x 128
// tile reads 24 KB per K step) at 6.5 TB/s, the rate the CUs' direct-to-LDS
// loads sustain here; one slice with direct stores about 3 us + 0.6 us per
// K step and round of 64 x 128 tiles.  The cheaper split form is taken when
// it is estimated 15 % faster than the persistent kernel, only while that
// kernel has fewer tiles than CUs.  A single slice whose 64 x 64 tiles still
// fit the CUs uses those: twice the work items, each reading 16 KB per K
// step instead of 24 (256 x 4096 x 4096: 14.2 us instead of 20.5).
bool gemm_split_wanted(const GemmArgs& a, int cus, int* slices, int* tile_n) {
  if (a.lora) return false;
  const int64_t steps = (a.k + kSK - 1) / kSK;
  int64_t big = 0, small = 0, narrow = 0;
  for (int i = 0; i < a.count; ++i) {
    big += ((a.m + 255) / 256) * ((a.w[i].n + 191) / 192);
    small += ((a.m + kSM - 1) / kSM) * ((a.w[i].n + 127) / 128);
    narrow += ((a.m + kSM - 1) / kSM) * ((a.w[i].n + 63) / 64);
  }
  if (big >= cus || steps < 2) return false;
  const double main_us = 3.0 + 1.2 * double(steps);
  const double atomic_us = 8.0 + double(small) * double(steps) * SplitCfg<128>::kStage / 6.5e6;
  const double direct_us = 3.0 + 0.6 * double(steps) * double((small + cus - 1) / cus);
  if (!(std::min(atomic_us, direct_us) < 0.85 * main_us)) return false;
  // About one work item per CU (measured 10-15 % faster than two: fewer
  // atomic partial sums), each slice at least 2 K steps; one slice when
  // direct stores are estimated cheaper.
  int64_t s = (cus + small - 1) / small;
  if (s > steps / 2) s = steps / 2;
  if (s < 1 || direct_us <= atomic_us) s = 1;
  *slices = int(s);
  *tile_n = (s == 1 && narrow <= cus) ? 64 : 128;
  return true;
}

namespace {

template <int SN>
hipError_t launch_split_t(const GemmArgs& a, int slices, hipStream_t stream) {
  SplitParams p{};
  p.qx = a.qx;
  p.sx = a.sx;
  p.M = int(a.m);
  p.K = int(a.k);
  const int steps = int((a.k + kSK - 1) / kSK);
  p.steps = (steps + slices - 1) / slices;
  p.slices = (steps + p.steps - 1) / p.steps;
  p.tiles_m = int((a.m + kSM - 1) / kSM);
  p.nseg = a.count;
  // One slice: each tile's sums are final and are stored directly.
  const bool direct = p.slices == 1;
  int items = 0;
  for (int i = 0; i < a.count; ++i) {
    SplitSeg& sg = p.seg[i];
    sg.qw = a.w[i].qw;
    sg.sw = a.w[i].sw;
    sg.bias = a.w[i].bias;
    sg.acc = static_cast<int*>(a.w[i].y);
    sg.ld = a.w[i].ldy;
    sg.n = int(a.w[i].n);
    sg.tiles_n = (sg.n + SN - 1) / SN;
    sg.item0 = items;
    items += sg.tiles_n * p.slices * p.tiles_m;
    if (!direct)
      hipLaunchKernelGGL(zero_kernel, elementwise_grid(a.m, a.w[i].n), dim3(256), 0, stream,
                         sg.acc, sg.ld, p.M, sg.n);
  }
  const dim3 grid(static_cast<unsigned>(items));
  if (!direct)
    hipLaunchKernelGGL((gemm_split_kernel<0, SN>), grid, dim3(SplitCfg<SN>::kWaves * 64), 0,
                       stream, p);
  else if (a.raw_i32)
    hipLaunchKernelGGL((gemm_split_kernel<3, SN>), grid, dim3(SplitCfg<SN>::kWaves * 64), 0,
                       stream, p);
  else if (a.gelu)
    hipLaunchKernelGGL((gemm_split_kernel<2, SN>), grid, dim3(SplitCfg<SN>::kWaves * 64), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((gemm_split_kernel<1, SN>), grid, dim3(SplitCfg<SN>::kWaves * 64), 0,
                       stream, p);
  if (!direct && !a.raw_i32) {
    for (int i = 0; i < a.count; ++i) {
      float* y = static_cast<float*>(a.w[i].y);
      const dim3 eg = elementwise_grid(a.m, a.w[i].n);
      if (a.gelu)
        hipLaunchKernelGGL(scale_kernel<true>, eg, dim3(256), 0, stream, y, a.w[i].ldy, p.M,
                           int(a.w[i].n), a.sx, a.w[i].sw, a.w[i].bias);
      else
        hipLaunchKernelGGL(scale_kernel<false>, eg, dim3(256), 0, stream, y, a.w[i].ldy, p.M,
                           int(a.w[i].n), a.sx, a.w[i].sw, a.w[i].bias);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_split(const GemmArgs& a, int slices, int tile_n, hipStream_t stream) {
  if (tile_n == 64) return launch_split_t<64>(a, slices, stream);
  if (tile_n == 128) return launch_split_t<128>(a, slices, stream);
  return hipErrorInvalidValue;
}

}  // namespace convrot
