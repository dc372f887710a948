// INT8 GEMM on CDNA4 matrix cores with the scale-restoration epilogue fused.
//
// Implements the stable-diffusion.cpp page "INT8 Convrot Safetensors",
// section "Runtime activation quantization":
//   A[r, o] = sum_i Q_x[r, i] Q_w[o, i]         (signed 32-bit accumulation)
//   Y[r, o] = A[r, o] * s_x[r] * s_w[o] + b[o]
// Both operands are int8 rows with K contiguous ("NT"), the natural operand
// layout of the i8 MFMA instructions.  Several weight matrices that share one
// packed activation (same input, same group size) run in one launch.
//
// Design (gfx950), a persistent, warp-specialised kernel:
//   * tile 256 (rows of Q_x) x 128 (rows of Q_w), K step 128 bytes;
//   * one workgroup per CU walks a list of tiles; 8 waves per workgroup:
//     - 4 MFMA waves (one per SIMD) each own a 128 x 64 block of
//       v_mfma_i32_32x32x32_i8 accumulators;
//     - 4 loader waves (one per SIMD) stream Q_x / Q_w tiles global -> LDS
//       with direct-to-LDS 16-byte loads into a 3-stage ring, two K steps
//       ahead and across tile boundaries, and also bring s_x, s_w and b of
//       the next tile into a double-buffered LDS area the same way;
//   * one s_barrier per K step hands a stage from the loaders to the MFMA
//     waves and back.  Only the loaders wait on global loads, so the MFMA
//     waves never wait for their own output stores: the epilogue of a tile
//     (int32 -> float, * s_x * s_w + b, optional GELU, 16-byte stores) drains
//     to HBM while the next tile computes;
//   * the MFMA waves arrive at the barrier as soon as their last fragment of
//     a stage is in registers, one 32-wide sub-step before the end of the
//     step, and read the next stage's first fragments under that sub-step's
//     MFMAs;
//   * LDS rows are 128 bytes; the 16-byte chunk c of stage row r sits at slot
//     c ^ (r & 7) ^ ((r >> 3) & 1): the 16-byte fragment reads of 16
//     consecutive rows hit 16 distinct bank groups (no bank conflicts);
//   * the MFMA takes Q_x as its first operand, so for each accumulator
//     register the 32 lanes of a half-wave hold 32 consecutive output columns
//     of one row: every 4-byte store instruction writes whole 128-byte lines;
//   * tiles are dealt so that the workgroups on one XCD (workgroups go to
//     the 8 XCDs round robin) share a few tile rows and columns in L2.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBM = 256;
constexpr int kBN = 128;
constexpr int kBK = 128;                              // bytes of K per step
constexpr int kStages = 3;
constexpr int kThreads = 512;                         // 4 MFMA + 4 loader waves
constexpr int kStageBytes = (kBM + kBN) * kBK;        // 48 KB
constexpr int kPieces = (kBM + kBN) / 8;              // 1 KB pieces per stage
constexpr int kPiecesPerLoader = kPieces / 4;         // 12
constexpr int kParFloats = kBM + 2 * kBN;             // s_x | s_w | b
constexpr int kParBytes = kParFloats * 4;
constexpr int kLdsBytes = kStages * kStageBytes + 2 * kParBytes;
constexpr int kWM = kBM / 2, kWN = kBN / 2;           // MFMA wave tile 128 x 64
constexpr int kFM = kWM / 32, kFN = kWN / 32;         // 4 x 2 MFMA blocks
constexpr int kNumXcd = 8;
constexpr int kGroupM = 4;

enum { kModeF32 = 0, kModeGelu = 1, kModeI32 = 2 };

struct Seg {
  const int8_t* qw;
  const float* sw;
  const float* bias;
  void* y;
  int64_t ldy;
  int n;
  int tn0;  // first global tile column of this weight
};

struct GemmParams {
  const int8_t* qx;
  const float* sx;
  int M, K, nk;
  int nseg;
  int tiles_m, tiles_n, total_tiles;
  Seg seg[kMaxGemmGroup];
};

struct TileInfo {
  int m0, n0, s;
};

// Tile t of the grouped order: kGroupM tile rows are walked column by column.
CR_DEVICE TileInfo tile_info(const GemmParams& p, int t) {
  const int per_group = kGroupM * p.tiles_n;
  const int g = t / per_group;
  const int first = g * kGroupM;
  const int gm = (p.tiles_m - first < kGroupM) ? (p.tiles_m - first) : kGroupM;
  const int in = t - g * per_group;
  const int tm = first + in % gm;
  const int tn = in / gm;
  int s = 0;
  for (int i = 1; i < p.nseg; ++i)
    if (tn >= p.seg[i].tn0) s = i;
  TileInfo ti;
  ti.m0 = tm * kBM;
  ti.n0 = (tn - p.seg[s].tn0) * kBN;
  ti.s = s;
  return ti;
}

// Position of workgroup b inside a round of G tiles: each XCD (b % 8) gets a
// contiguous run of tile indices.
CR_DEVICE int round_slot(int b, int G) {
  const int xcd = b % kNumXcd, idx = b / kNumXcd;
  const int q = G / kNumXcd, r = G % kNumXcd;
  return (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

CR_DEVICE int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

CR_DEVICE v4i lds_frag(const int8_t* stage, int row, int kchunk) {
  return *reinterpret_cast<const v4i*>(stage + row * kBK + ((kchunk ^ lds_swz(row)) << 4));
}

CR_DEVICE float gelu_erf(float y) { return 0.5f * y * (1.0f + erff(y * 0.70710678118654752f)); }

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt_hi[15:14]); issued through the builtin so that the compiler's own wait
// insertion accounts for them.
constexpr int kWaitLgkm0 = 0xC07F;   // lgkmcnt(0)
constexpr int kWaitVm0 = 0x0F70;     // vmcnt(0)
constexpr int kWaitVm12 = 0x0F7C;    // vmcnt(12)

CR_DEVICE void barrier() {
  // A bare s_barrier: the waits each role needs are issued explicitly, and the
  // memory clobber keeps the compiler from moving LDS accesses across it.
  asm volatile("s_barrier" ::: "memory");
}

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(1024))) int8_t smem[kLdsBytes];
  int8_t* const par_base = smem + kStages * kStageBytes;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int G = gridDim.x;
  const int slot = round_slot(blockIdx.x, G);
  const int ntiles = (p.total_tiles - slot + G - 1) / G;  // tiles of this workgroup (>= 1)
  const int nk = p.nk;
  const int g_total = ntiles * nk;
  const int M = p.M, K = p.K;

  if (wave >= 4) {
    // ------------------------------------------------------------ loader waves
    const int lw = wave - 4;
    const int rip = lane >> 3;
    // Piece q = lw + 4i covers stage rows 8q..8q+7; lane l fills slot l of it:
    // row 8q + l/8, slot l%8, holding global 16-byte chunk (l%8) ^ swz(row).
    int kc[kPiecesPerLoader];
#pragma unroll
    for (int i = 0; i < kPiecesPerLoader; ++i)
      kc[i] = (lane & 7) ^ lds_swz((lw + 4 * i) * 8 + rip);

    // The issue stream walks (tile, k step) in order; per tile it computes the
    // source row of every piece once, so a step only adds its K offset.
    const int8_t* rowp[kPiecesPerLoader];
    int is_it = 0, is_ks = 0, is_stage = 0;
    auto setup_tile = [&](int it) {
      const TileInfo ti = tile_info(p, slot + it * G);
      const int8_t* qw = p.seg[ti.s].qw;
      const int n = p.seg[ti.s].n;
#pragma unroll
      for (int i = 0; i < kPiecesPerLoader; ++i) {
        const int q = lw + 4 * i;
        if (q < kBM / 8) {
          int r = ti.m0 + q * 8 + rip;
          r = r < M ? r : M - 1;  // rows past M load row M-1; never stored
          rowp[i] = p.qx + (int64_t)r * K + kc[i] * 16;
        } else {
          int r = ti.n0 + (q - kBM / 8) * 8 + rip;
          r = r < n ? r : n - 1;
          rowp[i] = qw + (int64_t)r * K + kc[i] * 16;
        }
      }
    };
    auto issue_next = [&]() {
      if (is_ks == 0) setup_tile(is_it);
      int8_t* stage = smem + is_stage * kStageBytes;
      const int k0 = is_ks * kBK;
      if (k0 + kBK <= K) {
#pragma unroll
        for (int i = 0; i < kPiecesPerLoader; ++i)
          __builtin_amdgcn_global_load_lds(rowp[i] + k0, (lds_void*)(stage + (lw + 4 * i) * 1024),
                                           16, 0, 0);
      } else {
        // K tail: keep every address in bounds; the chunks past K are zeroed
        // after the loads have landed.
#pragma unroll
        for (int i = 0; i < kPiecesPerLoader; ++i) {
          const int over = k0 + kc[i] * 16 - (K - 16);
          const int8_t* src = rowp[i] + k0 - (over > 0 ? over : 0);
          __builtin_amdgcn_global_load_lds(src, (lds_void*)(stage + (lw + 4 * i) * 1024), 16, 0, 0);
        }
      }
      is_stage = (is_stage == kStages - 1) ? 0 : is_stage + 1;
      if (++is_ks == nk) {
        is_ks = 0;
        ++is_it;
      }
    };
    // s_x, s_w, b of tile `it` into parameter buffer it % 2 (256 lanes x 2 floats).
    auto issue_params = [&](int it) {
      const TileInfo ti = tile_info(p, slot + it * G);
      const float* sw = p.seg[ti.s].sw;
      const float* bias = p.seg[ti.s].bias;
      const int n_lim = p.seg[ti.s].n - 1;
      int8_t* par = par_base + (it & 1) * kParBytes;
      const int L = lw * 64 + lane;
      int m = ti.m0 + L;
      m = m < M ? m : M - 1;
      __builtin_amdgcn_global_load_lds(p.sx + m, (lds_void*)(par + lw * 256), 4, 0, 0);
      int n = ti.n0 + (L < kBN ? L : L - kBN);
      n = n < n_lim ? n : n_lim;
      const float* src2 = (L < kBN || !bias) ? sw + n : bias + n;  // no bias: loaded, unused
      __builtin_amdgcn_global_load_lds(src2, (lds_void*)(par + kBM * 4 + lw * 256), 4, 0, 0);
    };
    // Zero the 16-byte chunks past K of a stage (after its loads have landed).
    auto zero_tail = [&](int stage_idx) {
      const int k0 = (nk - 1) * kBK;
      int8_t* stage = smem + stage_idx * kStageBytes;
#pragma unroll
      for (int i = 0; i < kPiecesPerLoader; ++i)
        if (k0 + kc[i] * 16 >= K)
          *reinterpret_cast<v4i*>(stage + (lw + 4 * i) * 1024 + lane * 16) = v4i{0, 0, 0, 0};
    };
    const bool ragged = (K % kBK) != 0;

    issue_params(0);
    issue_next();  // step 0
    if (g_total > 1) {
      issue_next();  // step 1
      __builtin_amdgcn_s_waitcnt(kWaitVm12);  // params and step 0 landed
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    if (ragged && nk == 1) zero_tail(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    barrier();  // B_0
    int ks1 = (nk > 1) ? 1 : 0;         // k step of step g+1
    int st1 = 1;                        // stage of step g+1
    int pit = 1, pks = 0;               // params: tile pit is due when step g-1 opens a tile
    for (int g = 0; g < g_total; ++g) {
      // After B_g the MFMA waves are done reading stage (g-1) % 3 = (g+2) % 3.
      if (g >= 1 && pks == 0 && pit < ntiles) issue_params(pit);
      if (g >= 1 && ++pks == nk) {
        pks = 0;
        ++pit;
      }
      if (g + 2 < g_total) {
        issue_next();  // step g+2
        __builtin_amdgcn_s_waitcnt(kWaitVm12);  // step g+1 (and params) landed
      } else {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
      }
      if (ragged && g + 1 < g_total && ks1 == nk - 1) zero_tail(st1);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      barrier();  // B_{g+1}
      ks1 = (ks1 == nk - 1) ? 0 : ks1 + 1;
      st1 = (st1 == kStages - 1) ? 0 : st1 + 1;
    }
    return;
  }

  // -------------------------------------------------------------- MFMA waves
  const int wm = wave >> 1, wn = wave & 1;
  const int frow = lane & 31;  // fragment row inside a 32-row block
  const int fkc = lane >> 5;   // 16-byte half of a 32-byte K slice
  v16i acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[i][j] = v16i{};
  v4i xf[2][kFM], wf[2][kFN];
  // Read slot f -> fragment, ordered as the MFMAs of a sub-step consume them:
  // Q_x block 0, Q_w blocks 0 and 1, then Q_x blocks 1..3.
  auto read_frag = [&](const int8_t* stage, int set, int f, int kk) {
    const bool is_x = (f == 0) || (f >= 3);
    const int b = (f == 0) ? 0 : (f <= 2 ? f - 1 : f - 2);
    if (is_x)
      xf[set][b] = lds_frag(stage, wm * kWM + b * 32 + frow, 2 * kk + fkc);
    else
      wf[set][b] = lds_frag(stage, kBM + wn * kWN + b * 32 + frow, 2 * kk + fkc);
  };
  constexpr int NFR = kFM + kFN;  // 6 fragment reads per 32-wide sub-step
  constexpr int NMF = kFM * kFN;  // 8 MFMAs per sub-step

  barrier();  // B_0
#pragma unroll
  for (int f = 0; f < NFR; ++f) read_frag(smem, 0, f, 0);

  int cur_stage = 0, ks = 0, it = 0;
  for (int g = 0; g < g_total; ++g) {
    const int nxt_stage = (cur_stage == kStages - 1) ? 0 : cur_stage + 1;
    const int8_t* cur = smem + cur_stage * kStageBytes;
    const int8_t* nxt = smem + nxt_stage * kStageBytes;
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      const int c = kk & 1;
#pragma unroll
      for (int idx = 0; idx < NMF; ++idx) {
        const int i = idx / kFN, j = idx % kFN;
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf[c][i], wf[c][j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (kk + 1 < kBK / 32 && idx < NFR) read_frag(cur, c ^ 1, idx, kk + 1);
        if (kk == kBK / 32 - 1 && idx == 1) {
          // Every fragment of this stage is in registers: hand the stage back
          // (two MFMAs in flight cover the barrier), then read the next
          // stage's first fragments under the remaining MFMAs.  After the
          // last step this reads a stale stage of the ring: harmless, and it
          // keeps the block free of branches.
          __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
          barrier();  // B_{g+1}
#pragma unroll
          for (int f = 0; f < NFR; ++f) read_frag(nxt, 0, f, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    cur_stage = nxt_stage;
    if (++ks < nk) continue;
    ks = 0;

    // Epilogue of tile `it`.  Accumulator element (i, j, r) holds row
    //   m = m0 + wm*128 + i*32 + 8*(r/4) + 4*(lane/32) + (r%4)
    // and column
    //   n = n0 + wn*64 + j*32 + (lane & 31).
    const TileInfo ti = tile_info(p, slot + it * G);
    const Seg& sg = p.seg[ti.s];
    const float* par = reinterpret_cast<const float*>(par_base + (it & 1) * kParBytes);
    const bool has_bias = sg.bias != nullptr;
    const bool interior = (ti.m0 + kBM <= M) && (ti.n0 + kBN <= sg.n);
    float swj[kFN], bj[kFN];
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const int nl = wn * kWN + j * 32 + (lane & 31);
      swj[j] = par[kBM + nl];
      bj[j] = has_bias ? par[kBM + kBN + nl] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        // rows ml .. ml+3 for r = 4*rq .. 4*rq+3
        const int ml = wm * kWM + i * 32 + 8 * rq + 4 * (lane >> 5);
        const float4 sx4 = *reinterpret_cast<const float4*>(&par[ml]);
        const float sxr[4] = {sx4.x, sx4.y, sx4.z, sx4.w};
#pragma unroll
        for (int j = 0; j < kFN; ++j) {
          const int n = ti.n0 + wn * kWN + j * 32 + (lane & 31);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int m = ti.m0 + ml + rr;
            const int a = acc[i][j][4 * rq + rr];
            if (MODE == kModeI32) {
              int* yr = static_cast<int*>(sg.y) + (int64_t)m * sg.ldy + n;
              if (interior || (m < M && n < sg.n)) *yr = a;
            } else {
              float v = (float)a * sxr[rr];
              v = has_bias ? __builtin_fmaf(v, swj[j], bj[j]) : v * swj[j];
              if (MODE == kModeGelu) v = gelu_erf(v);
              float* yr = static_cast<float*>(sg.y) + (int64_t)m * sg.ldy + n;
              if (interior || (m < M && n < sg.n)) *yr = v;
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j) acc[i][j] = v16i{};
    ++it;
  }
}

int device_cu_count() {
  static std::mutex mu;
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <int MODE>
hipError_t launch_t(const GemmParams& p, hipStream_t stream) {
  const int cus = device_cu_count();
  const int grid = p.total_tiles < cus ? p.total_tiles : cus;
  hipLaunchKernelGGL((gemm_i8_kernel<MODE>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  GemmParams p;
  p.qx = a.qx;
  p.sx = a.sx;
  p.M = int(a.m);
  p.K = int(a.k);
  p.nk = int((a.k + kBK - 1) / kBK);
  p.nseg = a.count;
  p.tiles_m = int((a.m + kBM - 1) / kBM);
  int tn = 0;
  for (int i = 0; i < a.count; ++i) {
    Seg& s = p.seg[i];
    s.qw = a.w[i].qw;
    s.sw = a.w[i].sw;
    s.bias = a.w[i].bias;
    s.y = a.w[i].y;
    s.ldy = a.w[i].ldy;
    s.n = int(a.w[i].n);
    s.tn0 = tn;
    tn += int((a.w[i].n + kBN - 1) / kBN);
  }
  p.tiles_n = tn;
  p.total_tiles = p.tiles_m * tn;
  if (p.total_tiles == 0) return hipSuccess;
  if (a.raw_i32) return launch_t<kModeI32>(p, stream);
  if (a.gelu) return launch_t<kModeGelu>(p, stream);
  return launch_t<kModeF32>(p, stream);
}

}  // namespace convrot
