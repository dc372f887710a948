// INT8 GEMM on CDNA4 matrix cores with the scale-restoration epilogue fused.
//
// Implements the stable-diffusion.cpp page "INT8 Convrot Safetensors",
// section "Runtime activation quantization":
//   A[r, o] = sum_i Q_x[r, i] Q_w[o, i]         (signed 32-bit accumulation)
//   Y[r, o] = A[r, o] * s_x[r] * s_w[o] + b[o]
// Both operands are int8 rows with K contiguous ("NT"), the natural operand
// layout of the i8 MFMA instructions.
//
// Design (gfx950):
//   * workgroup tile BM x BN (rows of Q_x x rows of Q_w), K step 128, four
//     waves in a 2 x 2 arrangement, each owning a (BM/2) x (BN/2) block of
//     v_mfma_i32_32x32x32_i8 accumulators (in AGPRs);
//   * global -> LDS with direct-to-LDS 16-byte loads (no VGPR staging), double
//     buffered: the loads of K step s+1 are spread over the MFMAs of step s;
//   * LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at slot
//     c ^ (r & 7) ^ ((r >> 3) & 1), so the 16-byte fragment reads of 16
//     consecutive rows hit 16 distinct bank groups;
//   * inside a K step, every MFMA is followed by at most one LDS fragment read
//     for the next 32-wide sub-step (two fragment register sets), with
//     scheduling barriers pinning that order;
//   * the MFMA takes Q_w as its first operand, so each lane ends up holding 4
//     consecutive output columns of one output row: the fused epilogue
//     (int32 -> float, * s_x * s_w + b, optional GELU) leaves as 16-byte
//     stores; s_x, s_w and b of the tile are staged in LDS up front;
//   * the epilogue mode (float, float + GELU, raw int32) is a template
//     parameter, and interior tiles take a path without bounds checks;
//   * workgroups are re-numbered so that each XCD (workgroups are dealt to the
//     8 XCDs round robin) owns a contiguous band of tiles, walked in groups of
//     a few tile rows for L2 reuse.
#include "common.h"
#include "kernels.h"

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;          // K bytes per step (8 chunks of 16)
constexpr int kThreads = 256;     // 4 waves
constexpr int kNumXcd = 8;
constexpr int kDmaStride = 3;     // one direct-to-LDS load per this many MFMAs

enum { kModeF32 = 0, kModeGelu = 1, kModeI32 = 2 };

typedef __attribute__((address_space(3))) void lds_void;

CR_DEVICE void load_lds_16(const void* g, lds_void* l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

struct GemmParams {
  const int8_t* qx;
  const float* sx;
  const int8_t* qw;
  const float* sw;
  const float* bias;
  void* y;
  int M, N, K;
  int64_t ldy;
  int tiles_m, group_m;
  int vec_store;  // y 16-byte aligned and ldy % 4 == 0
};

template <int BM, int BN>
struct Tile {
  static constexpr int WM = BM / 2;        // wave tile rows (Q_x)
  static constexpr int WN = BN / 2;        // wave tile cols (Q_w)
  static constexpr int FM = WM / 32;       // MFMA blocks along M
  static constexpr int FN = WN / 32;       // MFMA blocks along N
  static constexpr int A_BYTES = BM * kBK;
  static constexpr int STAGE = (BM + BN) * kBK;
  static constexpr int PIECES = (BM + BN) / 8;   // 1 KB pieces per stage
  static constexpr int PIECES_PER_WAVE = PIECES / 4;
  static_assert(PIECES % 4 == 0, "tile rows must split over 4 waves");
};

// Map the hardware workgroup id to a tile (tm, tn).
CR_DEVICE void tile_of_block(int bid, int nblk, int tiles_m, int group_m, int& tm, int& tn) {
  // XCD-aware renumbering: block b runs on XCD b % 8; give each XCD a contiguous range.
  const int xcd = bid % kNumXcd;
  const int idx = bid / kNumXcd;
  const int q = nblk / kNumXcd, r = nblk % kNumXcd;
  const int t = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
  // Grouped order: walk group_m tile rows column by column.
  const int tiles_n = nblk / tiles_m;
  const int per_group = group_m * tiles_n;
  const int g = t / per_group;
  const int first = g * group_m;
  const int gm = (tiles_m - first < group_m) ? (tiles_m - first) : group_m;
  const int in = t - g * per_group;
  tm = first + in % gm;
  tn = in / gm;
}

// LDS slot of 16-byte chunk c in tile row r.  Rows are 128 bytes; the slot
// permutation makes the 16-byte fragment reads of 16 consecutive rows hit 16
// distinct 16-byte bank groups (and 8 consecutive rows 8 distinct groups).
CR_DEVICE int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

CR_DEVICE v4i lds_frag(const int8_t* region, int row, int kchunk) {
  return *reinterpret_cast<const v4i*>(region + row * kBK + ((kchunk ^ lds_swz(row)) << 4));
}

CR_DEVICE float gelu_erf(float y) { return 0.5f * y * (1.0f + erff(y * 0.70710678118654752f)); }

template <int BM, int BN, int MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_kernel(const GemmParams p) {
  using T = Tile<BM, BN>;
  constexpr int PPW = T::PIECES_PER_WAVE;
  constexpr int NMF = T::FM * T::FN;       // MFMAs per 32-wide K sub-step
  constexpr int NFR = T::FM + T::FN;       // fragment reads per sub-step
  constexpr int KSUB = kBK / 32;           // sub-steps per K step
  static_assert(NFR <= NMF, "fragment reads must fit between the MFMAs");
  static_assert(PPW * kDmaStride <= NMF * KSUB, "loads must fit between the MFMAs of a K step");
  // One LDS object holds both stages and the epilogue operands: with a second
  // __shared__ array the compiler can no longer tell the fragment reads from
  // the direct-to-LDS writes and puts a wait for global memory before every
  // fragment read.
  __shared__ __attribute__((aligned(1024))) int8_t smem[2 * T::STAGE + (BM + 2 * BN) * 4];
  float* par = reinterpret_cast<float*>(smem + 2 * T::STAGE);  // s_x | s_w | b of the tile

  const int M = p.M, N = p.N, K = p.K;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Stage the epilogue operands of this tile in LDS (visible after the first
  // barrier below).  Rows and columns past the edge read a valid neighbour;
  // they are never stored.
  if (MODE != kModeI32) {
    for (int i = t; i < BM + 2 * BN; i += kThreads) {
      float v;
      if (i < BM) {
        const int m = m0 + i;
        v = p.sx[m < M ? m : M - 1];
      } else {
        const int c = (i < BM + BN) ? i - BM : i - BM - BN;
        const int n = (n0 + c < N) ? n0 + c : N - 1;
        v = (i < BM + BN) ? p.sw[n] : (p.bias ? p.bias[n] : 0.f);
      }
      par[i] = v;
    }
  }

  // Direct-to-LDS load plan: piece p (1 KB = 8 rows x 128 bytes) of a stage is
  // loaded by wave p % 4; lane l fills LDS slot l of the piece, i.e. row
  // 8p + l/8, slot l%8, which holds global chunk (l%8) ^ lds_swz(row).
  const int rip = lane >> 3;
  int kc[PPW];
  const int8_t* row_ptr[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int pc = wave + 4 * i;
    kc[i] = (lane & 7) ^ lds_swz(pc * 8 + rip);
    if (pc < BM / 8) {
      int r = m0 + pc * 8 + rip;
      r = r < M ? r : M - 1;  // rows past M load row M-1; never stored
      row_ptr[i] = p.qx + (int64_t)r * K;
    } else {
      int r = n0 + (pc - BM / 8) * 8 + rip;
      r = r < N ? r : N - 1;
      row_ptr[i] = p.qw + (int64_t)r * K;
    }
  }
  auto dma = [&](int8_t* stage, int i, int k0) {
    int off = k0 + kc[i] * 16;
    off = off < K - 16 ? off : K - 16;  // K tail: stay in bounds, zeroed after the wait
    load_lds_16(row_ptr[i] + off, (lds_void*)(stage + (wave + 4 * i) * 1024));
  };
  auto zero_tail = [&](int8_t* stage, int k0) {
#pragma unroll
    for (int i = 0; i < PPW; ++i)
      if (k0 + kc[i] * 16 >= K)
        *reinterpret_cast<v4i*>(stage + (wave + 4 * i) * 1024 + lane * 16) = v4i{0, 0, 0, 0};
  };

  v16i acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = v16i{};

  const int nk = (K + kBK - 1) / kBK;
  const int frow = lane & 31;   // fragment row inside a 32-row block
  const int fkc = lane >> 5;    // which 16-byte half of a 32-byte K slice
  v4i xf[2][T::FM], wf[2][T::FN];
  auto read_frag = [&](const int8_t* stage, int set, int f, int kk) {
    if (f < T::FM)
      xf[set][f] = lds_frag(stage, wm * T::WM + f * 32 + frow, 2 * kk + fkc);
    else
      wf[set][f - T::FM] =
          lds_frag(stage + T::A_BYTES, wn * T::WN + (f - T::FM) * 32 + frow, 2 * kk + fkc);
  };

#pragma unroll
  for (int i = 0; i < PPW; ++i) dma(smem, i, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (nk == 1) zero_tail(smem, 0);
  __syncthreads();
#pragma unroll
  for (int f = 0; f < NFR; ++f) read_frag(smem, 0, f, 0);

  for (int ks = 0; ks < nk; ++ks) {
    int8_t* cur = smem + (ks & 1) * T::STAGE;
    int8_t* nxt = smem + ((ks + 1) & 1) * T::STAGE;
    // The last step re-loads its own K range into the idle buffer (never read),
    // which keeps the loop body free of branches.
    const int k_next = (ks + 1 < nk ? ks + 1 : ks) * kBK;
    // One basic block: MFMAs interleaved with the fragment reads of the next
    // sub-step and with the direct-to-LDS loads of the next K step (one per
    // kDmaStride MFMAs: issuing them back to back stalls the MFMA stream).
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk) {
      const int c = kk & 1;
#pragma unroll
      for (int idx = 0; idx < NMF; ++idx) {
        const int i = idx / T::FN, j = idx % T::FN;
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wf[c][j], xf[c][i], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (kk + 1 < KSUB && idx < NFR) read_frag(cur, c ^ 1, idx, kk + 1);
        const int slot = kk * NMF + idx;
        if (slot % kDmaStride == 0 && slot / kDmaStride < PPW) dma(nxt, slot / kDmaStride, k_next);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (ks + 2 == nk) zero_tail(nxt, k_next);
    __syncthreads();
    if (ks + 1 < nk) {
#pragma unroll
      for (int f = 0; f < NFR; ++f) read_frag(nxt, 0, f, 0);
    }
  }

  // Epilogue.  Accumulator element (i, j, r) holds output row
  //   m = m0 + wm*WM + i*32 + (lane & 31)
  // and output column
  //   n = n0 + wn*WN + j*32 + 8*(r/4) + 4*(lane/32) + (r%4).
  const bool interior = (m0 + BM <= M) && (n0 + BN <= N) && p.vec_store;
  auto tile_value = [&](int i, int j, int g, float (&o)[4]) {
    const int ml = wm * T::WM + i * 32 + (lane & 31);
    const int nl = wn * T::WN + j * 32 + 8 * g + 4 * (lane >> 5);
    const float sxm = par[ml];
    const float4 swv = *reinterpret_cast<const float4*>(&par[BM + nl]);
    const float4 bv = *reinterpret_cast<const float4*>(&par[BM + BN + nl]);
    const float sv[4] = {swv.x, swv.y, swv.z, swv.w};
    const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float v = (float)acc[i][j][4 * g + c] * sxm;
      v = __builtin_fmaf(v, sv[c], bb[c]);
      if (MODE == kModeGelu) v = gelu_erf(v);
      o[c] = v;
    }
  };
  if (interior) {
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int m = m0 + wm * T::WM + i * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * T::WN + j * 32 + 8 * g + 4 * (lane >> 5);
          if (MODE == kModeI32) {
            int* yr = static_cast<int*>(p.y) + (int64_t)m * p.ldy + n;
            *reinterpret_cast<v4i*>(yr) = v4i{acc[i][j][4 * g + 0], acc[i][j][4 * g + 1],
                                              acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          } else {
            float o[4];
            tile_value(i, j, g, o);
            float* yr = static_cast<float*>(p.y) + (int64_t)m * p.ldy + n;
            *reinterpret_cast<float4*>(yr) = make_float4(o[0], o[1], o[2], o[3]);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int m = m0 + wm * T::WM + i * 32 + (lane & 31);
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * T::WN + j * 32 + 8 * g + 4 * (lane >> 5);
          float o[4];
          if (MODE != kModeI32) tile_value(i, j, g, o);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (n + c >= N) continue;
            if (MODE == kModeI32)
              static_cast<int*>(p.y)[(int64_t)m * p.ldy + n + c] = acc[i][j][4 * g + c];
            else
              static_cast<float*>(p.y)[(int64_t)m * p.ldy + n + c] = o[c];
          }
        }
      }
    }
  }
}

template <int BM, int BN, int MODE>
hipError_t launch_t(const GemmArgs& a, hipStream_t stream) {
  GemmParams p;
  p.qx = a.qx;
  p.sx = a.sx;
  p.qw = a.qw;
  p.sw = a.sw;
  p.bias = a.bias;
  p.y = a.y;
  p.M = int(a.m);
  p.N = int(a.n);
  p.K = int(a.k);
  p.ldy = a.ldy;
  p.tiles_m = int((a.m + BM - 1) / BM);
  const int tiles_n = int((a.n + BN - 1) / BN);
  p.group_m = 4;
  p.vec_store = (reinterpret_cast<uintptr_t>(a.y) % 16 == 0) && (a.ldy % 4 == 0);
  const int nblk = p.tiles_m * tiles_n;
  hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, MODE>), dim3(nblk), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  // 256 x 192 tiles: N = 3072 gives exactly 256 tiles per 4096 rows (one per CU).
  if (a.raw_i32) return launch_t<256, 192, kModeI32>(a, stream);
  if (a.gelu) return launch_t<256, 192, kModeGelu>(a, stream);
  return launch_t<256, 192, kModeF32>(a, stream);
}

}  // namespace convrot
