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
// Design (gfx950): a persistent kernel, one workgroup of 4 waves per CU.
//   * Output tile 256 (rows of Q_x) x BN (rows of Q_w).  Each wave (one per
//     SIMD, so it may use the whole 512-entry register file) owns a
//     128 x BN/2 block of v_mfma_i32_32x32x32_i8 accumulators.  When a tile
//     is complete its accumulators are copied into a second register set and
//     the next tile starts from zero.
//   * The finished tile is stored during the first 8 K steps of the next
//     tile (scaled on the way in the plain float32 mode; in the GELU and
//     adapter modes it was made float32 at its end), 4 fixed groups of
//     2 x FN values per step, one store under every other MFMA of the middle
//     sub-steps.  Those 8 steps are unrolled, so every store names its
//     registers at compile time and the K loop carries no store bookkeeping.
//     Output writes are thus spread over the main loop instead of bursting
//     at tile ends.
//   * K advances 128 bytes per step (four 32-wide sub-steps).  Operands
//     reach LDS by direct-to-LDS buffer loads of whole 128-byte lines, one
//     per operand row and step, through two rings: Q_x in 2 stages (loaded
//     one step ahead), Q_w in 3 stages (two steps ahead).  Each wave's 14
//     loads of a step are spread one per ~3 MFMAs: a load that cannot issue
//     also holds back the MFMAs behind it.  The buffer resources span the
//     tile's valid rows, so rows past M or N read as zero (hardware range
//     check) and need no clamping or clearing; so do the Q_w chunks past K,
//     which zero whatever the Q_x chunks there hold.  A tile has
//     at least 3 K steps (short K is padded with such zero chunks), so the
//     load streams never run more than one tile ahead.
//   * Everything a tile needs from the kernel arguments (buffer resources of
//     the next tile, its scales and bias) is fetched in the tile prologue,
//     outside the K loop, which thus holds no scalar-memory load: the LDS
//     waits the compiler places inside it count exactly.
//   * One s_barrier per step, two MFMAs into the last sub-step: by then every
//     fragment of the stage is in registers; the next stage's first fragments
//     are read under the remaining MFMAs.
//   * LDS rows are 128 bytes; 16-byte chunk c of stage row r sits at slot
//     c ^ (r & 7) ^ ((r >> 3) & 1), so 16 lanes reading 16 consecutive rows
//     touch 16 distinct groups of 4 banks.
//   * The MFMA takes Q_x as its first operand: for each accumulator register
//     the 32 lanes of a half-wave hold 32 consecutive columns of one output
//     row, so every 4-byte store instruction writes whole 128-byte lines.
//     Output stores are non-temporal: Y is written once and should not push
//     the operand slices the other CUs of the XCD still read out of L2.
//   * s_x, s_w and b of a tile reach LDS by direct-to-LDS loads in the tile's
//     prologue (the first tile's with the first operand loads), in a ring of
//     two buffers.
//   * Loads and stores share one in-order counter (vmcnt).  Every wait names
//     exactly the number of instructions issued after the awaited loads (this
//     step's stores and the Q_w loads of two steps ahead).
//   * Tiles are dealt so that the workgroups of one XCD (workgroups go to the
//     8 XCDs round robin) work on neighbouring tile rows and columns, which
//     they then share in that XCD's L2.
//   * Low-rank adapters (the page's section "Backend support": a correction
//     from the unrotated X added to the output): in the adapter modes the
//     finished tile's accumulators are turned into float32 Y values in place
//     (A s_x s_w + b) at the tile end, and the adapter's U B^T is added by
//     bf16 MFMAs that take those registers as their accumulator input; the
//     rank/16 MFMAs per 32x32 block share the int8 accumulator layout.  The
//     deferred stores then write the finished values.
#include <mutex>
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace convrot {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kBM = 256;
constexpr int kBN = 192;       // tile columns
constexpr int kThreads = 256;  // 4 waves
constexpr int kGroupM = 4;
constexpr int kMinSteps = 3;   // K steps per tile at least (see the header comment)

// Output modes.  kModeF32 scales each value as it is stored, and
// kModeF32Gelu applies the GELU there as well; the tile-end modes turn the
// whole tile into float32 values at its end (and add the adapters there),
// and only store them (through the GELU in kModeTileEndGelu).  Without
// adapters, scaling at store time is the faster GELU form: the tile-end
// conversion runs while the matrix cores wait, the store-time work under
// the next tile's MFMAs.
enum { kModeF32 = 0, kModeF32Gelu = 1, kModeI32 = 2, kModeTileEnd = 3, kModeTileEndGelu = 4 };

template <int BN>
struct Cfg {
  static constexpr int BK = 128;                          // bytes of K per step
  static constexpr int XSTAGE = kBM * BK;                 // bytes per Q_x stage (2 stages)
  static constexpr int WSTAGE = BN * BK;                  // bytes per Q_w stage (3 stages)
  static constexpr int WOFF = 2 * XSTAGE;                 // LDS offset of the Q_w ring
  static constexpr int XPW = kBM / 8 / 4;                 // 1 KB pieces (8 rows) per wave, Q_x
  static constexpr int WPW = BN / 8 / 4;                  // ... and Q_w
  static constexpr int XT = XPW / 2;                      // Q_x pieces issued after the barrier
  static constexpr int WN = BN / 2;                       // wave tile columns
  static constexpr int FM = 4, FN = WN / 32;              // 32x32 blocks per wave
  static constexpr int NMF = FM * FN;                     // MFMAs per sub-step
  static constexpr int PR = (kBM + 2 * BN + 255) / 256;   // parameter loads per wave and tile
  static constexpr int PARB = PR * 256 * 4;               // bytes per parameter buffer
  static constexpr int PAR0 = WOFF + 3 * WSTAGE;          // LDS offset of the parameter ring
  static constexpr int NPK = 3;                           // pending groups parked in LDS
  static constexpr int PARK0 = PAR0 + 2 * PARB;           // LDS offset of the parking area
  static constexpr int LDS = PARK0 + NPK * 6 * kThreads * 4;
  static constexpr int NG = 32;                           // store groups per tile
  static constexpr int NV = 2 * FN;                       // values (stores) per group
  static constexpr int GPS = 4;                           // store groups per storing step
  static constexpr int NSS = NG / GPS;                    // K steps that carry stores
  static constexpr int GSUB = GPS / 2;                    // ... per storing sub-step (1 and 2)
  static constexpr int ST = NMF / (GSUB * NV);            // MFMAs per store
  static_assert(kBM % 32 == 0 && BN % 32 == 0, "pieces must split over 4 waves");
  static_assert(FN >= 2 && XT + 2 <= NMF && XPW - XT <= NMF && WPW <= 2 * NMF, "interleave slots");
  static_assert(GPS % 2 == 0 && ST * GSUB * NV == NMF, "stores evenly spread over the middle sub-steps");
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert(FM * FN * 16 == NG * NV, "store groups cover the tile");
  static_assert(WPW + GPS * NV <= kVmMax, "vmcnt range");
  static_assert(NPK <= GPS, "parked groups are stored by the last storing step");
};

struct Seg {
  const int8_t* qw;
  const float* sw;
  const float* bias;
  void* y;
  int64_t ldy;
  int n;
  int tn0;  // first global tile column of this weight
  const uint16_t* lu;  // adapter: U bfloat16 [M, ldu], B bfloat16 [n, rank]
  const uint16_t* lb;
  int ldu, rank;       // rank 0: no adapter
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
template <int BN>
CR_DEVICE TileInfo tile_info(const GemmParams& p, int t) {
  const int per_group = kGroupM * p.tiles_n;
  const int g = t / per_group;
  const int first = g * kGroupM;
  const int gm = (p.tiles_m - first < kGroupM) ? (p.tiles_m - first) : kGroupM;
  const int in = t - g * per_group;
  const int tm = first + in % gm;
  const int tn = in / gm;
  // The segment: unrolled over every slot so that the first-column loads are
  // independent scalar loads issued together (a loop up to nseg waits for
  // each one in turn); segment 0 starts at column 0.
  int s = 0, tn0 = 0;
#pragma unroll
  for (int i = 1; i < kMaxGemmGroup; ++i) {
    const int t0 = p.seg[i].tn0;
    if (i < p.nseg && tn >= t0) {
      s = i;
      tn0 = t0;
    }
  }
  TileInfo ti;
  ti.m0 = tm * kBM;
  ti.n0 = (tn - tn0) * BN;
  ti.s = s;
  return ti;
}


// Slot (MFMA index in [lo, n_slots)) of the i-th of n loads spread evenly
// over a sub-step; -1 for no load at that slot.
constexpr int spread_piece(int idx, int lo, int n_slots, int n) {
  for (int i = 0; i < n; ++i)
    if (idx == lo + ((2 * i + 1) * (n_slots - lo)) / (2 * n)) return i;
  return -1;
}

template <int BN, int MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_kernel(const GemmParams p) {
  using C = Cfg<BN>;
  constexpr int FM = C::FM, FN = C::FN, NV = C::NV, NG = C::NG, NSS = C::NSS;
  constexpr bool LORA = MODE == kModeTileEnd || MODE == kModeTileEndGelu;  // tile-end epilogue
  constexpr bool GELU = MODE == kModeTileEndGelu || MODE == kModeF32Gelu;
  // Scales and bias applied when a value is stored (otherwise the pending
  // values are raw int32 results or finished float32 values).
  constexpr bool SCALE_AT_STORE = MODE == kModeF32 || MODE == kModeF32Gelu;
  __shared__ __attribute__((aligned(1024))) int8_t smem[C::LDS];

  const int lane = threadIdx.x & 63;
  // wave, M and K are re-read through an empty asm statement at the top of
  // every step and tile prologue (see reload_uniforms): values derived from
  // them are then recomputed where they are used instead of being hoisted
  // into the kernel prologue, where they would stay live (and spill) for the
  // whole kernel.
  int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // The grid size and the activation pointers, made opaque once: otherwise
  // the compiler may reload them from the kernel arguments right before a K
  // loop, and a scalar load in flight turns every LDS wait in that loop into
  // a wait for all of them.
  int G = gridDim.x;
  const int8_t* qx = p.qx;
  const float* sx = p.sx;
  asm volatile("" : "+s"(G), "+s"(qx), "+s"(sx));
  const int slot = xcd_slot(blockIdx.x, G);
  const int ntiles = (p.total_tiles - slot + G - 1) / G;  // >= 1: grid <= tiles
  const int nk = p.nk;                                    // >= kMinSteps
  int M = p.M, K = p.K;
  auto reload_uniforms = [&]() { asm volatile("" : "+s"(wave), "+s"(M), "+s"(K)); };

  // ------------------------------------------------------------ loading
  // Piece q = wave + 4i of a stage holds its rows 8q .. 8q+7.  Lane l fills
  // LDS slot l of it: row 8q + l/8, slot l%8, which holds global chunk
  // (l%8) ^ (row & 7) ^ ((row >> 3) & 1) = (l%8) ^ (l/8) ^ (q & 1), and
  // q & 1 = wave & 1 for every piece of a wave.  The two operands are loaded
  // as independent streams (Q_w runs one step further ahead); past the last
  // tile a stream repeats that tile into stages nobody reads any more.
  //
  // A load's byte offset is lane_off (the lane's row within the piece and its
  // chunk, the same for every load of the launch) plus the piece's first row
  // and the step's K offset, which are uniform and go into the instruction's
  // scalar offset: no vector work per load or step.  The range check covers
  // the sum of both offsets, so rows past the tile's last read zeros.  Past K
  // (in a step that BK does not fit into K, and in the zero-padded steps of a
  // short K) the Q_w lanes use an offset outside every resource and read
  // zeros; the Q_x lanes there read the next row's bytes, which only ever
  // meet those zeros.
  auto ld_chunk = [&]() { return (lane & 7) ^ (lane >> 3) ^ (wave & 1); };
  const unsigned lane_off = unsigned((lane >> 3) * K + ld_chunk() * 16);  // < 8 * K <= 2^21
  // ... for the step that holds K's end (if BK does not divide K)
  const unsigned w_part_off = ld_chunk() * 16 < K % C::BK ? lane_off : kOutOfRange;
  struct Stream {
    __amdgpu_buffer_rsrc_t rs, next;  // this tile's rows; the next tile's (set by its prologue)
    int ks, stage;
  };
  auto x_rsrc = [&](int t_it) {
    const TileInfo ti = tile_info<BN>(p, slot + t_it * G);
    const int rows = M - ti.m0 < kBM ? M - ti.m0 : kBM;
    return buffer_rsrc(qx + (int64_t)ti.m0 * K, rows * K);
  };
  auto w_rsrc = [&](int t_it) {
    const TileInfo ti = tile_info<BN>(p, slot + t_it * G);
    const Seg& sg = p.seg[ti.s];
    const int rows = sg.n - ti.n0 < BN ? sg.n - ti.n0 : BN;
    return buffer_rsrc(sg.qw + (int64_t)ti.n0 * K, rows * K);
  };
  Stream xs{x_rsrc(0), x_rsrc(0), 0, 0};
  Stream ws{w_rsrc(0), w_rsrc(0), 0, 0};
  unsigned w_voff = lane_off;  // Q_w lane offset of the step being loaded
  auto begin_w = [&]() {
    const int k0 = ws.ks * C::BK;
    w_voff = k0 + C::BK <= K ? lane_off : k0 < K ? w_part_off : kOutOfRange;
  };
  auto piece_x = [&](int i) {
    int8_t* dst = smem + xs.stage * C::XSTAGE + (wave + 4 * i) * 1024;
    const int soff = xs.ks * C::BK + (wave + 4 * i) * 8 * K;
    const __amdgpu_buffer_rsrc_t rs = xs.rs;  // (a local: the host pass rejects a member)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, lane_off, soff, 0, 0);
  };
  auto piece_w = [&](int i) {
    int8_t* dst = smem + C::WOFF + ws.stage * C::WSTAGE + (wave + 4 * i) * 1024;
    const int soff = ws.ks * C::BK + (wave + 4 * i) * 8 * K;
    const __amdgpu_buffer_rsrc_t rs = ws.rs;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, w_voff, soff, 0, 0);
  };
  auto end_x = [&]() {
    xs.stage ^= 1;
    if (++xs.ks == nk) {
      xs.ks = 0;
      xs.rs = xs.next;
    }
  };
  auto end_w = [&]() {
    ws.stage = ws.stage == 2 ? 0 : ws.stage + 1;
    if (++ws.ks == nk) {
      ws.ks = 0;
      ws.rs = ws.next;
    }
  };
  // s_x | s_w | b of tile t_it into parameter buffer t_it % 2.  Float f of a
  // buffer is loaded by wave (f / 64) % 4, lane f % 64 (padding loads s_x[0]).
  // The section boundaries are multiples of 64, so each wave's 64 floats come
  // from one array: a buffer load through a wave-uniform resource.  (A global
  // load into LDS would do the same work, but the compiler counts it as a flat
  // access still in flight and then waits for all LDS reads, lgkmcnt(0),
  // wherever the K loop needs only the oldest fragments.)
  static_assert(kBM % 64 == 0 && BN % 64 == 0, "a wave's parameter floats share one array");
  auto issue_params = [&](int t_it) {
    const TileInfo ti = tile_info<BN>(p, slot + t_it * G);
    const float* sw = p.seg[ti.s].sw;
    const float* bias = p.seg[ti.s].bias;
    const int n_lim = p.seg[ti.s].n - 1;
    int8_t* par = smem + C::PAR0 + (t_it & 1) * C::PARB;
#pragma unroll
    for (int rd = 0; rd < C::PR; ++rd) {
      // The resource covers the tile's own rows or columns (at most 256
      // floats); idx is relative to the tile's first one.
      const int f0 = rd * 256 + wave * 64;  // uniform
      const int f = f0 + lane;
      const float* src = sx;
      int bytes = 4, idx = 0;
      if (f0 < kBM) {
        const int last = M - 1 - ti.m0;  // >= 0: the tile has rows
        src = sx + ti.m0;
        bytes = (last < kBM ? last + 1 : kBM) * 4;
        idx = f < last ? f : last;
      } else if (f0 < kBM + 2 * BN) {
        const bool is_w = f0 < kBM + BN;
        const int last = n_lim - ti.n0;  // >= 0: the tile has columns
        const int c = is_w ? f - kBM : f - kBM - BN;
        src = ((is_w || !bias) ? sw : bias) + ti.n0;
        bytes = (last < BN ? last + 1 : BN) * 4;
        idx = c < last ? c : last;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(buffer_rsrc(src, bytes), (lds_void*)(par + f0 * 4),
                                               4, idx * 4, 0, 0, 0);
    }
  };

  // ----------------------------------------------------------- fragments
  // Lane l reads row R + l%32 of a 32-row block (R a multiple of 32), 16-byte
  // chunk 2*kk + l/32 of K slice kk.  Since R is a multiple of 32 the row's
  // swizzle depends on l only, so each slice has one per-lane offset and the
  // block adds a uniform R*128.
  const int frow = lane & 31;
  const int fswz = (frow & 7) ^ ((frow >> 3) & 1);
  int fbase[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) fbase[kk] = frow * 128 + (((2 * kk + (lane >> 5)) ^ fswz) << 4);
  // Q_x fragments are single-buffered: x block i is reloaded for the next
  // sub-step right after its last MFMA (sub-steps run i-major), at least
  // NMF - FN MFMAs before it is needed again.  Q_w fragments, used until the
  // end of a sub-step, alternate between two sets.
  v4i xf[FM], wf[2][FN];
  auto read_x = [&](const int8_t* xstage, int i, int kk) {
    xf[i] = *reinterpret_cast<const v4i*>(xstage + fbase[kk] + ((wave >> 1) * 128 + i * 32) * 128);
  };
  auto read_w = [&](const int8_t* wstage, int set, int j, int kk) {
    wf[set][j] = *reinterpret_cast<const v4i*>(wstage + fbase[kk] + ((wave & 1) * C::WN + j * 32) * 128);
  };
  // The fragment reads that follow MFMA idx of a sub-step, for slice kk of
  // the given stages (the next sub-step's slice).
  auto reads_after = [&](int idx, const int8_t* xstage, const int8_t* wstage, int kk) {
    if (idx % FN == FN - 1) read_x(xstage, idx / FN, kk);
    if (idx < FN) read_w(wstage, kk & 1, idx, kk);
  };

  v16i acc[FM][FN];

  // ------------------------------------------------------ pending output
  // The finished tile waits in pend: pend[e][q] is accumulator element
  // (i, j, r) = (q / 8, e / 2, 4*((q / 2) % 4) + 2*(q % 2) + e % 2), i.e.
  // output row pd_row0 + i*32 + 8*((q / 2) % 4) + 2*(q % 2) + e % 2 and
  // column pd_col0 + (e / 2)*32, where pd_row0 = m0 + wm*128 + 4*(lane/32)
  // and pd_col0 = n0 + wn*BN/2 + lane%32.  Group q holds two rows of each of
  // the FN column blocks: NV store instructions, each writing a full
  // 128-byte segment of two output rows.  pend is only ever indexed with
  // compile-time constants (the code that stores it is unrolled), so each
  // value is a register of its own that is free again once stored.  The
  // last NPK groups (stored last) wait in a per-thread LDS area instead: the
  // register file, holding the running tile's accumulators as well, has no
  // room left for them.
  int pend[NG - C::NPK][NV];
  auto park_slot = [&](int q, int e) -> int* {  // q >= NG - NPK
    return reinterpret_cast<int*>(smem + C::PARK0) + ((q - (NG - C::NPK)) * NV + e) * kThreads +
           threadIdx.x;
  };
  // Value e of pending group q (q a constant after unrolling).
  auto pend_get = [&](int q, int e) -> int {
    return q >= NG - C::NPK ? *park_slot(q, e) : pend[q < NG - C::NPK ? q : 0][e];
  };
  int pd_valid = 0, pd_interior = 0, pd_n = 0, pd_par = C::PAR0;
  int pd_row0 = 0, pd_col0 = 0;
  int pd_sxo = 0;              // LDS offset of this lane's s_x for group 0
  int pd_m0w = 0, pd_n0w = 0;  // uniform parts: m0 + wm*128, n0 + wn*BN/2
  int pd_fast = 0;             // interior tile with a row stride that fits the fast path
  unsigned pd_voff = 0;        // lane part of a fast-path store offset, in bytes
  __amdgpu_buffer_rsrc_t pd_rs = buffer_rsrc(nullptr, 0);  // fast path: the wave's 128 rows
  float* pd_y = nullptr;
  int64_t pd_ldy = 0;
  int pd_has_b = 0;             // the pending tile's weight has a bias
  // s_w and b of the lane's columns for the paths that store outside the
  // storing steps (edge tiles, short K, the last tile).
  float pd_sw[FN], pd_b[FN];
  auto load_sw_b = [&]() {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int nl = (wave & 1) * C::WN + j * 32 + (lane & 31);
      pd_sw[j] = *reinterpret_cast<const float*>(smem + pd_par + (kBM + nl) * 4);
      const float bv = *reinterpret_cast<const float*>(smem + pd_par + (kBM + BN + nl) * 4);
      pd_b[j] = pd_has_b ? bv : 0.f;
    }
  };

  auto group_row = [&](int q) {  // output row of element e = 0 of group q
    return pd_row0 + (q >> 3) * 32 + 8 * ((q >> 1) & 3) + 2 * (q & 1);
  };
  auto read_group_sx = [&](int q) -> f32x2 {
    return *reinterpret_cast<const f32x2*>(smem + pd_par + (group_row(q) - pd_row0 + (wave >> 1) * 128 +
                                                               4 * (lane >> 5)) * 4);
  };
  auto scaled_with = [&](int raw, float sx, float sw, float b) -> float {
    if constexpr (MODE == kModeI32) return __int_as_float(raw);
    float v = SCALE_AT_STORE ? __builtin_fmaf((float)raw * sx, sw, b) : __int_as_float(raw);
    if constexpr (GELU) v = gelu_erf(v);
    return v;
  };
  auto scaled = [&](int raw, float sx, int j) -> float { return scaled_with(raw, sx, pd_sw[j], pd_b[j]); };
  // Value e of group q, masked to the matrix (any tile).
  auto store_value = [&](int q, int e, f32x2 sx, float* yrow, int m) {
    const int j = e >> 1, rr = e & 1;
    const float v = scaled(pend_get(q, e), sx[rr], j);
    float* yp = yrow + rr * pd_ldy + j * 32;
    if (m + rr < M && pd_col0 + j * 32 < pd_n) __builtin_nontemporal_store(v, yp);
  };
  auto store_group = [&](int q, f32x2 sx) {
    const int m = group_row(q);
    float* yrow = pd_y + (int64_t)m * pd_ldy + pd_col0;
#pragma unroll
    for (int e = 0; e < NV; ++e) store_value(q, e, sx, yrow, m);
  };
  // Fast path (interior tiles): non-temporal buffer stores through a
  // resource over the wave's 128 rows; the row's byte offset is uniform (the
  // scalar offset), the lane's (4*(lane/32) rows, lane%32 columns) is fixed,
  // and the column block goes into the immediate offset.  No address
  // arithmetic per store beyond one scalar add.
  auto group_rel = [&](int q) {  // row of group q relative to m0 + wm*128
    return (q >> 3) * 32 + 8 * ((q >> 1) & 3) + 2 * (q & 1);
  };
  auto group_off = [&](int q) { return group_rel(q) * (int)pd_ldy * 4; };  // < 2^31 (pd_fast)
  auto store_raw_with = [&](int raw, int goff, f32x2 sx, int e, float sw, float b) {
    const int j = e >> 1, rr = e & 1;
    const float v = scaled_with(raw, sx[rr], sw, b);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), pd_rs, pd_voff + j * 128,
                                          goff + rr * (int)pd_ldy * 4, kNonTemporal);
  };
  auto store_raw = [&](int raw, int goff, f32x2 sx, int e) {
    store_raw_with(raw, goff, sx, e, pd_sw[e >> 1], pd_b[e >> 1]);
  };
  auto store_fast = [&](int q, int goff, f32x2 sx, int e) { store_raw(pend_get(q, e), goff, sx, e); };
  auto store_group_fast = [&](int q) {
    const f32x2 sx = read_group_sx(q);
    const int goff = group_off(q);
#pragma unroll
    for (int e = 0; e < NV; ++e) store_fast(q, goff, sx, e);
  };

  // ------------------------------------------------------------ prologue
  // The first tile's scales and bias, then both operands of steps 0 and 1
  // (both Q_x stages are free at the start, so the kernel's first step need
  // not request the rest of step 1 itself: one cold-load latency instead of
  // two before the loop runs).  Only step 0's operands (and the parameters)
  // are waited for here: step 1's land under step 0, whose closing wait
  // covers them.
  issue_params(0);
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
    for (int i = 0; i < C::XPW; ++i) piece_x(i);
    end_x();
    begin_w();
#pragma unroll
    for (int i = 0; i < C::WPW; ++i) piece_w(i);
    end_w();
  }
  waitvm<C::XPW + C::WPW>();
  wait_lgkm0();
  barrier();
#pragma unroll
  for (int f = 0; f < FM; ++f) read_x(smem, f, 0);
#pragma unroll
  for (int f = 0; f < FN; ++f) read_w(smem + C::WOFF, 0, f, 0);

  int cur_x = 0, cur_w = 0;  // stages of the step being computed

  // One K step into acc; the first step of a tile starts from zero.  Step g
  // computes from Q_x stage g%2 and Q_w stage g%3; during it the rest of Q_x
  // of step g+1 and all of Q_w of step g+2 are requested.  SG >= 0: the step
  // also stores groups 2*SG and 2*SG+1 of the pending tile (fast path).
  // PRO: the kernel's first step, whose step g+1 the prologue loaded whole.
  auto step = [&](auto first_t, auto ss_t, auto pro_t) __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first_t)::value;
    constexpr bool PRO = decltype(pro_t)::value;
    constexpr int SS = decltype(ss_t)::value;   // storing step index, or -1
    constexpr bool STORE = SS >= 0;
    constexpr int GPS = C::GPS;
    constexpr int NST = STORE ? GPS * NV : 0;  // stores issued by this step
    reload_uniforms();
    const int8_t* cx = smem + cur_x * C::XSTAGE;
    const int8_t* cw = smem + C::WOFF + cur_w * C::WSTAGE;
    const int nxt_x = cur_x ^ 1, nxt_w = cur_w == 2 ? 0 : cur_w + 1;
    const int8_t* nx = smem + nxt_x * C::XSTAGE;
    const int8_t* nw = smem + C::WOFF + nxt_w * C::WSTAGE;
    // s_x of the two groups a storing sub-step writes, read one sub-step
    // ahead (only two are live at a time).
    // s_w and b of the lane's columns, from the tile's parameter buffer
    // (kept in LDS, not in registers, between the steps that store).
    float gsw[FN] = {}, gb[FN] = {};
    if constexpr (STORE && SCALE_AT_STORE) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int nl = (wave & 1) * C::WN + j * 32 + (lane & 31);
        gsw[j] = *reinterpret_cast<const float*>(smem + pd_par + (kBM + nl) * 4);
        const float bv = *reinterpret_cast<const float*>(smem + pd_par + (kBM + BN + nl) * 4);
        gb[j] = pd_has_b ? bv : 0.f;
      }
    }
    // The parked groups (the step's last NPK groups) of the last storing
    // step, read from LDS one value per MFMA, PKL MFMAs before the one whose
    // store writes it (enough to cover the LDS latency; a longer lead keeps
    // more of them live in registers at once).
    int pk[C::NPK * NV];
    constexpr int PK0 = GPS - C::NPK;  // first parked group within the step
    constexpr int PKL = 4;
    auto read_parked = [&](int kk, int idx) {  // reads issued under MFMA idx of sub-step kk
      if constexpr (SS == C::NSS - 1) {
#pragma unroll
        for (int v = 0; v < C::NPK * NV; ++v) {
          const int g = PK0 + v / NV;            // group within the step
          const int store_kk = 1 + g / C::GSUB;  // sub-step that stores it
          const int slot = ((g % C::GSUB) * NV + v % NV) * C::ST + C::ST - 1;  // MFMA of its store
          const int at = store_kk * C::NMF + slot - PKL;  // position of the read
          if (kk * C::NMF + idx == at) pk[v] = *park_slot(NG - C::NPK + v / NV, v % NV);
        }
      }
    };
    f32x2 gsx[C::GSUB] = {};
    auto read_gsx = [&](int kk) {
      if constexpr (STORE && SCALE_AT_STORE) {
#pragma unroll
        for (int g = 0; g < C::GSUB; ++g)
          gsx[g] = *reinterpret_cast<const f32x2*>(
              smem + pd_sxo + group_rel(GPS * SS + C::GSUB * (kk - 1) + g) * 4);
      }
    };
    read_gsx(1);

    // Sub-step 0: fragments of sub-step 1, the remaining Q_x of step g+1.
#pragma unroll
    for (int idx = 0; idx < C::NMF; ++idx) {
      const int i = idx / FN, j = idx % FN;
      acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf[i], wf[0][j], FIRST ? v16i{} : acc[i][j],
                                                        0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      reads_after(idx, cx, cw, 1);
      read_parked(0, idx);
      if constexpr (!PRO) {
        const int pc = spread_piece(idx, 0, C::NMF, C::XPW - C::XT);
        if (pc >= 0) piece_x(C::XT + pc);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (!PRO) end_x();
    begin_w();
    __builtin_amdgcn_sched_barrier(0);

    // Sub-steps 1 and 2: fragments, Q_w of step g+2, the step's stores.
#pragma unroll
    for (int kk = 1; kk < 3; ++kk) {
#pragma unroll
      for (int idx = 0; idx < C::NMF; ++idx) {
        const int i = idx / FN, j = idx % FN;
        acc[i][j] =
            __builtin_amdgcn_mfma_i32_32x32x32_i8(xf[i], wf[kk & 1][j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        reads_after(idx, cx, cw, kk + 1);
        if constexpr (STORE) {  // one store per ST MFMAs (constants after unrolling)
          if (idx % C::ST == C::ST - 1) {
            const int sn = idx / C::ST;
            const int g = C::GSUB * (kk - 1) + sn / NV, e = sn % NV;
            const int q = GPS * SS + g;
            const int raw = q >= NG - C::NPK ? pk[(q - (NG - C::NPK)) * NV + e]
                                             : pend[q < NG - C::NPK ? q : 0][e];
            store_raw_with(raw, group_off(q), gsx[sn / NV], e, gsw[e >> 1], gb[e >> 1]);
          }
          if (kk == 1 && idx == C::NMF - 1) read_gsx(2);
          read_parked(kk, idx);
        }
        {
          constexpr int half = C::WPW / 2;
          const int pc = kk == 1 ? spread_piece(idx, 0, C::NMF, half)
                                 : spread_piece(idx, 0, C::NMF, C::WPW - half);
          if (pc >= 0) piece_w(kk == 1 ? pc : half + pc);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    end_w();

    // Sub-step 3: wait, barrier, fragments and first Q_x loads of the next
    // stage.
#pragma unroll
    for (int idx = 0; idx < 2; ++idx) {
      acc[0][idx] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf[0], wf[1][idx], acc[0][idx], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Q_x of step g+1 and (issued a step earlier) Q_w of step g+1 have
    // landed once only this step's stores and Q_w loads may be in flight.
    waitvm<C::WPW + NST>();
    wait_lgkm0();
    barrier();  // the next stages are readable by all, this step's are free
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int idx = 2; idx < C::NMF; ++idx) {
      const int i = idx / FN, j = idx % FN;
      acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(xf[i], wf[1][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      // After the barrier: x block 0 (free since MFMA 2) and the Q_w set of
      // the next step's first sub-step, then x blocks as they free up.
      if (idx % FN == FN - 1) read_x(nx, idx / FN, 0);
      if (idx >= 2 && idx < 2 + FN) read_w(nw, 0, idx - 2, 0);
      {
        const int pc = spread_piece(idx, 2, C::NMF, C::XT);
        if (pc >= 0) piece_x(pc);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    cur_x = nxt_x;
    cur_w = nxt_w;
  };

  // Adapter epilogue of tile t_it: its accumulators become float32 Y values
  // (A s_x s_w + b, from the tile's parameter buffer, the rounding of the
  // store-time path), and U B^T is accumulated onto them.  U and B fragments
  // come straight from global memory (L2) by buffer loads whose resources
  // span the tile's valid rows, so rows past M or n read as zero.  The rank
  // is walked in 16-wide slices (unrolled: rank <= kLoraMaxRank), each
  // requested one slice ahead (deeper prefetch spills in the K loop); the
  // first is requested before the float32 conversion, whose VALU work covers
  // its latency.  These are loads into registers, so the compiler's own
  // waits cover them.
  auto lora_epilogue = [&](int t_it) __attribute__((always_inline)) {
    constexpr int NSL = kLoraMaxRank / 16, PF = 1;
    reload_uniforms();
    // Lane-derived offsets are formed here, from a copy the compiler cannot
    // see through, rather than hoisted out of the tile loop (live across
    // the K loop they would spill).
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const TileInfo ti = tile_info<BN>(p, slot + t_it * G);
    const Seg& sg = p.seg[ti.s];
    const int8_t* par = smem + C::PAR0 + (t_it & 1) * C::PARB;
    const int wm = wave >> 1, wn = wave & 1;
    const int rank = sg.rank;  // 0 or a multiple of 16
    const int rows = M - ti.m0 < kBM ? M - ti.m0 : kBM;
    const int cols = sg.n - ti.n0 < BN ? sg.n - ti.n0 : BN;
    const int ldu = sg.ldu;
    const __amdgpu_buffer_rsrc_t ur = buffer_rsrc(sg.lu + (int64_t)ti.m0 * ldu, rows * ldu * 2);
    const __amdgpu_buffer_rsrc_t br = buffer_rsrc(sg.lb + (int64_t)ti.n0 * rank, cols * rank * 2);
    // Lane l: row l % 32 of a 32-row block, bf16 elements 8 (l / 32) .. +7
    // of a 16-wide rank slice (both operands; the sum runs over all 16).
    const unsigned uoff = unsigned(((wm * 128 + (lane & 31)) * ldu + 8 * (lane >> 5)) * 2);
    const unsigned boff = unsigned(((wn * C::WN + (lane & 31)) * rank + 8 * (lane >> 5)) * 2);
    v4i uf[NSL][FM], bfr[NSL][FN];
    auto load_slice = [&](int sl) {
      if (16 * sl < rank) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
          uf[sl][i] = __builtin_bit_cast(
              v4i, __builtin_amdgcn_raw_buffer_load_b128(
                       ur, uoff + unsigned((i * 32 * ldu + 16 * sl) * 2), 0, 0));
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bfr[sl][j] = __builtin_bit_cast(
              v4i, __builtin_amdgcn_raw_buffer_load_b128(
                       br, boff + unsigned((j * 32 * rank + 16 * sl) * 2), 0, 0));
      }
    };
#pragma unroll
    for (int sl = 0; sl < PF; ++sl) load_slice(sl);

    const bool has_b = sg.bias != nullptr;
    float sw[FN], bb[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int nl = wn * C::WN + j * 32 + (lane & 31);
      sw[j] = *reinterpret_cast<const float*>(par + (kBM + nl) * 4);
      const float bv = *reinterpret_cast<const float*>(par + (kBM + BN + nl) * 4);
      bb[j] = has_b ? bv : 0.f;
    }
    // Register e of block (i, j) is row 8 (e / 4) + e % 4 + 4 (lane / 32) of
    // row block i: four consecutive rows per f32x4 of s_x.
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 sx4 = *reinterpret_cast<const f32x4*>(
            par + (wm * 128 + i * 32 + 8 * r4 + 4 * (lane >> 5)) * 4);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int e = 4 * r4 + rr;
            acc[i][j][e] = __float_as_int(__builtin_fmaf((float)acc[i][j][e] * sx4[rr], sw[j], bb[j]));
          }
      }
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      if (16 * sl < rank) {
        if (sl + PF < NSL) load_slice(sl + PF);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_bit_cast(
                v16i, __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                          __builtin_bit_cast(bf16x8, uf[sl][i]),
                          __builtin_bit_cast(bf16x8, bfr[sl][j]),
                          __builtin_bit_cast(f32x16, acc[i][j]), 0, 0, 0));
      }
    }
  };

  for (int it = 0; it < ntiles; ++it) {
    // Tile prologue: the next tile's operand rows (the load streams enter it
    // during this tile's last steps) and this tile's scales and bias.
    {
      reload_uniforms();
      const int t1 = it + 1 < ntiles ? it + 1 : ntiles - 1;
      xs.next = x_rsrc(t1);
      ws.next = w_rsrc(t1);
      if (it > 0) issue_params(it);  // (the first tile's: in the kernel prologue)
      wait_lgkm0();  // no scalar load stays in flight into the K loop
    }
    if (pd_fast) {
      // The pending interior tile is stored GPS groups per step over the
      // tile's first NSS steps (unrolled: constant register indices).
      for_each_index(std::make_integer_sequence<int, NSS>{}, [&](auto ss) {
        constexpr int S = decltype(ss)::value;
        if (S < nk) step(std::integral_constant<bool, S == 0>{}, ss, std::false_type{});
      });
      for (int ks = NSS; ks < nk; ++ks)
        step(std::false_type{}, std::integral_constant<int, -1>{}, std::false_type{});
      if (nk < NSS) {  // short K: the groups left over
        load_sw_b();
        for_each_index(std::make_integer_sequence<int, NG>{}, [&](auto qc) {
          constexpr int Q = decltype(qc)::value;
          if (Q >= C::GPS * nk) store_group_fast(Q);
        });
        wait_lgkm0();
        barrier();  // the pending tile's parameter buffer is refilled next
      }
    } else {
      if (pd_valid) {  // an edge tile: masked stores, before this tile's steps
        load_sw_b();
        for_each_index(std::make_integer_sequence<int, NG>{}, [&](auto qc) {
          constexpr int Q = decltype(qc)::value;
          store_group(Q, read_group_sx(Q));
        });
      }
      if (it == 0)
        step(std::true_type{}, std::integral_constant<int, -1>{}, std::true_type{});
      else
        step(std::true_type{}, std::integral_constant<int, -1>{}, std::false_type{});
      for (int ks = 1; ks < nk; ++ks)
        step(std::false_type{}, std::integral_constant<int, -1>{}, std::false_type{});
    }

    // The tile is complete and the previous one fully stored: move the
    // accumulators into pend.  The tile's parameters were requested in its
    // prologue and have been waited for since.
    if constexpr (LORA) lora_epilogue(it);
#pragma unroll
    for (int q = 0; q < NG; ++q)
#pragma unroll
      for (int e = 0; e < NV; ++e)
      {
        int v = acc[q >> 3][e >> 1][4 * ((q >> 1) & 3) + 2 * (q & 1) + (e & 1)];
        // Finished values only feed stores, which could take them from the
        // accumulator registers; keep them in ordinary VGPRs, which is where
        // the register file has room next to the running tile.
        if constexpr (LORA) asm volatile("" : "+v"(v));
        if (q >= NG - C::NPK)
          *park_slot(q, e) = v;
        else
          pend[q < NG - C::NPK ? q : 0][e] = v;
      }
    const TileInfo ti = tile_info<BN>(p, slot + it * G);
    const Seg& sg = p.seg[ti.s];
    pd_valid = 1;
    pd_par = C::PAR0 + (it & 1) * C::PARB;
    pd_sxo = pd_par + ((wave >> 1) * 128 + 4 * (lane >> 5)) * 4;
    pd_row0 = ti.m0 + (wave >> 1) * 128 + 4 * (lane >> 5);
    pd_col0 = ti.n0 + (wave & 1) * C::WN + (lane & 31);
    pd_y = static_cast<float*>(sg.y);
    pd_ldy = sg.ldy;
    pd_n = sg.n;
    pd_interior = (ti.m0 + kBM <= M) && (ti.n0 + BN <= sg.n);
    pd_m0w = ti.m0 + (wave >> 1) * 128;
    pd_n0w = ti.n0 + (wave & 1) * C::WN;
    // (128 rows of a stride below 2^22 floats: every offset fits 31 bits)
    pd_fast = pd_interior && sg.ldy < (int64_t(1) << 22);
    pd_voff = unsigned((4 * (lane >> 5)) * (int)(pd_fast ? sg.ldy : 0) + (lane & 31)) * 4u;
    pd_rs = buffer_rsrc(pd_y + (int64_t)pd_m0w * pd_ldy + pd_n0w, pd_fast ? 128 * (int)pd_ldy * 4 : 0);
    pd_has_b = sg.bias != nullptr;
  }
  // The last tile.
  load_sw_b();
  if (pd_fast) {
    for_each_index(std::make_integer_sequence<int, NG>{},
                   [&](auto qc) { store_group_fast(decltype(qc)::value); });
  } else {
    for_each_index(std::make_integer_sequence<int, NG>{}, [&](auto qc) {
      constexpr int Q = decltype(qc)::value;
      store_group(Q, read_group_sx(Q));
    });
  }
  waitvm<0>();  // no load into LDS may still be in flight at exit
}

template <int BN, int MODE>
hipError_t launch_t(GemmParams p, hipStream_t stream) {
  p.tiles_m = (p.M + kBM - 1) / kBM;
  int tn = 0;
  for (int i = 0; i < p.nseg; ++i) {
    p.seg[i].tn0 = tn;
    tn += (p.seg[i].n + BN - 1) / BN;
  }
  p.tiles_n = tn;
  p.total_tiles = p.tiles_m * tn;
  p.nk = (p.K + Cfg<BN>::BK - 1) / Cfg<BN>::BK;
  if (p.nk < kMinSteps) p.nk = kMinSteps;  // the extra steps read zeros
  if (p.total_tiles == 0) return hipSuccess;
  const int cus = device_cu_count();
  const int grid = p.total_tiles < cus ? p.total_tiles : cus;
  hipLaunchKernelGGL((gemm_i8_kernel<BN, MODE>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

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

hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
  int slices = 0, tile_n = 0;
  if (gemm_split_wanted(a, device_cu_count(), &slices, &tile_n))
    return launch_gemm_split(a, slices, tile_n, stream);
  GemmParams p{};
  p.qx = a.qx;
  p.sx = a.sx;
  p.M = int(a.m);
  p.K = int(a.k);
  p.nseg = a.count;
  for (int i = 0; i < a.count; ++i) {
    Seg& s = p.seg[i];
    s.qw = a.w[i].qw;
    s.sw = a.w[i].sw;
    s.bias = a.w[i].bias;
    s.y = a.w[i].y;
    s.ldy = a.w[i].ldy;
    s.n = int(a.w[i].n);
    s.tn0 = 0;
    s.lu = a.w[i].lu;
    s.lb = a.w[i].lb;
    s.ldu = int(a.w[i].ldu);
    s.rank = a.lora ? a.w[i].rank : 0;
  }
  if (a.raw_i32) {
    if (a.lora || a.gelu) return hipErrorInvalidValue;
    return launch_t<kBN, kModeI32>(p, stream);
  }
  if (a.gelu && !a.lora) return launch_t<kBN, kModeF32Gelu>(p, stream);
  if (a.gelu) return launch_t<kBN, kModeTileEndGelu>(p, stream);
  if (a.lora) return launch_t<kBN, kModeTileEnd>(p, stream);
  return launch_t<kBN, kModeF32>(p, stream);
}

}  // namespace convrot
