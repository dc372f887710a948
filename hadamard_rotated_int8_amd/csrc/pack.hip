// Activation pack: group-wise Hadamard rotation + row absmax + int8 codes.
//
// Implements the runtime half of the stable-diffusion.cpp page "INT8 Convrot
// Safetensors", section "Runtime activation quantization": every row of X is
// rotated by the block-diagonal R (R_G = normalised Kronecker power of H4 on
// each contiguous group of G = 4^n features, section "How INT8 convrot works"),
// then one scale per row s = max|X_rot| / 127 and codes
// Q = clamp(round(X_rot / s), -127, 127), packed as int8 rows + float32 scales.
//
// Design (gfx950, one pass over HBM, HBM-bound):
//   * one workgroup per row (rows strided over the grid); T = 64..1024 threads;
//   * a thread owns "chunks" of 16 consecutive features, loaded with 16-byte
//     vector loads (bf16: 2 loads, fp32: 4 loads);
//   * the base-4 digits of the in-group index are transformed in any order
//     (every factor of the Kronecker power is the same H4):
//       digits 0,1 (feature bits 0-3)  : inside the thread's registers,
//       digit 2    (lane bits 0-1)     : DPP quad permutations,
//       digit 3    (lane bits 2-3)     : DPP row rotations (see chunk_of_thread),
//       digit 4    (lane bits 4-5)     : cross-row lane shuffles,
//       digits 5,6 (wave bits)         : through LDS;
//   * the butterfly is unnormalised, y_d = sum(x) - 2 x_{3-d} = 2 (H4 x)_d; the
//     factor 2^n is exact and is taken out of the scale, so every rounding is
//     that of the normalised butterfly;
//   * the row absmax is reduced across the wave in registers (DPP moves and
//     permlane swaps) and then, for rows split over waves, in LDS;
//   * the code decision is made in float32: s = m/127 (IEEE division) and
//     r = RN(1/s) once per row, then per value a code.  Nearly every row:
//     r_up, the nearest float32 above 1/s (so exact ties of x / s round away
//     from zero), and one fused multiply-add rounding x r_up to nearest even,
//     RN(x r_up + 1.5 2^23), the code in its low byte (x r_up is never an
//     exact tie when r_up has at least 9 significant bits); rows whose r is
//     a power of two: trunc(RN(x r + copysign(0.5 - 2^-25, x))), exactly
//     round half away of x / s.  Either equals round(x / s) except within
//     a few ulp of a half-integer; rows with a tiny absmax are pre-scaled by
//     2^64 so that 1/s cannot overflow; the int8 codes leave as 16-byte
//     stores.
//
// Fast path (pack_rows_kernel), used when G <= 1024 and K is a multiple of
// 1024 (every row then splits into whole 64-chunk wave loads): one wave owns
// one row, lane l holds chunks c*64 + l (c < K/1024) with the same lane
// permutation, so all digits live in registers, DPP and lane shuffles; the
// absmax is a wave reduction.  No LDS and no barriers: a workgroup is just
// four independent rows, and every row of the matrix can be in flight at
// once, which is what an HBM-bound pass needs.
//
// G = 64 and 256 (pack_rows_lds_kernel, the common DiT case): the same
// row-per-wave structure, but digits 2-3 reach registers by a 16 x 16
// transpose through LDS inside each group of 16 lanes (rows padded against
// bank conflicts), so every butterfly stage is a register stage; the codes
// return by a byte transpose and leave as 16-byte stores; float32 rows are
// loaded as whole 1 KB lines and handed to their lanes through LDS; rows
// longer than 8192 features are split over 2 or 4 waves whose maxima meet
// in LDS.
#include <atomic>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace convrot {
namespace {

// Radix-4 butterfly on four registers: returns 2 * H4 * x (unnormalised).
CR_DEVICE void h4_reg(float& a, float& b, float& c, float& d) {
  const float s = (a + b) + (c + d);
  const float y0 = __builtin_fmaf(-2.f, d, s);
  const float y1 = __builtin_fmaf(-2.f, c, s);
  const float y2 = __builtin_fmaf(-2.f, b, s);
  const float y3 = __builtin_fmaf(-2.f, a, s);
  a = y0;
  b = y1;
  c = y2;
  d = y3;
}

// Digit held by lane bits 0-1 (natural order): partner 3-d is lane ^ 3.
CR_DEVICE float h4_quad(float x) {
  const float t = x + dpp_f32<kDppQuadSwap1>(x);
  const float s = t + dpp_f32<kDppQuadSwap2>(t);
  return __builtin_fmaf(-2.f, dpp_f32<kDppQuadRev>(x), s);
}

// Digit held by lane bits 2-3.  The lane -> digit map is d = 2*b3 + (b2 ^ b3),
// so the lane holding digit 3-d is lane ^ 8, one row rotation by 8.
CR_DEVICE float h4_row(float x) {
  const float t = x + dpp_f32<kDppRowRor4>(x);
  const float s = t + dpp_f32<kDppRowRor8>(t);
  return __builtin_fmaf(-2.f, dpp_f32<kDppRowRor8>(x), s);
}

// Digit held by lane bits 4-5 (natural order): partner is lane ^ 48.
CR_DEVICE float h4_wave(float x) {
  const float a = __shfl_xor(x, 16);
  const float b = __shfl_xor(x, 32);
  const float c = __shfl_xor(x, 48);
  const float s = (x + a) + (b + c);
  return __builtin_fmaf(-2.f, c, s);
}

// Maximum over the wave of a float that is non-negative and not NaN in every
// lane (a lane's own fmaxf of |x| drops NaNs): such floats order as their
// bit patterns do as unsigned integers, so the cross-lane steps are integer
// maxima, four of them fused with DPP lane moves (quads, then rotations
// inside rows of 16) and two across rows and wave halves by the permlane
// swaps; no LDS round trips on the row's critical path.
CR_DEVICE float wave_max_nonneg(float x) {
  unsigned v = __float_as_uint(x);
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadSwap1, 0xF, 0xF, false));
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadSwap2, 0xF, 0xF, false));
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowRor4, 0xF, 0xF, false));
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowRor8, 0xF, 0xF, false));
  const auto rows = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // rows 2i <-> 2i+1
  v = max((unsigned)rows[0], (unsigned)rows[1]);
  const auto halves = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // lanes 0-31 <-> 32-63
  v = max((unsigned)halves[0], (unsigned)halves[1]);
  return __uint_as_float(v);
}

// Thread t owns chunk (t with bit 2 replaced by bit2 ^ bit3) of each block of
// T chunks, which realises the lane -> digit map used by h4_row.  It permutes
// chunks only inside aligned groups of 16 lanes, so loads stay coalesced.
CR_DEVICE int chunk_of_thread(int t) { return t ^ ((t >> 1) & 4); }

CR_DEVICE void load16(const float* __restrict__ p, float* v) {
  const f32x4* p4 = reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 f = __builtin_nontemporal_load(p4 + i);
    v[4 * i + 0] = f.x;
    v[4 * i + 1] = f.y;
    v[4 * i + 2] = f.z;
    v[4 * i + 3] = f.w;
  }
}

CR_DEVICE void load16(const uint16_t* __restrict__ p, float* v) {
  const u32x4* p4 = reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const u32x4 u = __builtin_nontemporal_load(p4 + i);
    v[8 * i + 0] = bf16_lo(u.x);
    v[8 * i + 1] = bf16_hi(u.x);
    v[8 * i + 2] = bf16_lo(u.y);
    v[8 * i + 3] = bf16_hi(u.y);
    v[8 * i + 4] = bf16_lo(u.z);
    v[8 * i + 5] = bf16_hi(u.z);
    v[8 * i + 6] = bf16_lo(u.w);
    v[8 * i + 7] = bf16_hi(u.w);
  }
}

CR_DEVICE uint32_t pack4(int a, int b, int c, int d) {
  return (uint32_t(a) & 0xFFu) | ((uint32_t(b) & 0xFFu) << 8) | ((uint32_t(c) & 0xFFu) << 16) |
         (uint32_t(d) << 24);
}

// Rotate the 16 values of one chunk along the digits that live in registers
// and in lanes of the same wave.
CR_DEVICE void rotate_in_wave(float* v, int log4g) {
  if (log4g >= 1) {
#pragma unroll
    for (int a = 0; a < 4; ++a) h4_reg(v[4 * a], v[4 * a + 1], v[4 * a + 2], v[4 * a + 3]);
  }
  if (log4g >= 2) {
#pragma unroll
    for (int a = 0; a < 4; ++a) h4_reg(v[a], v[a + 4], v[a + 8], v[a + 12]);
  }
  if (log4g >= 3) {
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = h4_quad(v[e]);
  }
  if (log4g >= 4) {
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = h4_row(v[e]);
  }
  if (log4g >= 5) {
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = h4_wave(v[e]);
  }
}

// Digits 5 and 6 live in wave-index bits 0-1 and 2-3; exchange through LDS.
// Every thread of the block must call this (it contains barriers).
CR_DEVICE void rotate_across_waves(float* v, int log4g, float4* buf, int t) {
  for (int dg = 5; dg < log4g; ++dg) {
    const int sh = 6 + 2 * (dg - 5);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
      buf[t * 4 + i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    __syncthreads();
    const int dd = (t >> sh) & 3;  // uniform per wave (sh >= 6)
    const int base = t & ~(3 << sh);
    // The sum S accumulates in v (own value first, then the other digits in
    // order); x_{3-dd} is read back from LDS for the last step, 4 values at a
    // time, so the stage needs no second 16-value register set.
#pragma unroll
    for (int d2 = 0; d2 < 4; ++d2) {
      if (d2 == dd) continue;
      const int tt = base | (d2 << sh);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 f = buf[tt * 4 + i];
        v[4 * i + 0] += f.x;
        v[4 * i + 1] += f.y;
        v[4 * i + 2] += f.z;
        v[4 * i + 3] += f.w;
      }
    }
    const int tr = base | ((3 - dd) << sh);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 f = buf[tr * 4 + i];
      v[4 * i + 0] = __builtin_fmaf(-2.f, f.x, v[4 * i + 0]);
      v[4 * i + 1] = __builtin_fmaf(-2.f, f.y, v[4 * i + 1]);
      v[4 * i + 2] = __builtin_fmaf(-2.f, f.z, v[4 * i + 2]);
      v[4 * i + 3] = __builtin_fmaf(-2.f, f.w, v[4 * i + 3]);
    }
  }
}

template <typename InT, int CPT>
CR_DEVICE void load_rotate_segment(const InT* __restrict__ xr, int seg, int nch, int log4g,
                                   float (&v)[CPT][16], float4* buf, int t, int T) {
  const int tp = chunk_of_thread(t);
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    // Lanes past the row's last chunk load its first one (any valid address)
    // and zero the values: no divergent branch around the load.
    const int j = (seg * CPT + c) * T + tp;
    const bool ok = j < nch;
    load16(xr + (int64_t)(ok ? j : 0) * 16, v[c]);
#pragma unroll
    for (int e = 0; e < 16; ++e) v[c][e] = ok ? v[c][e] : 0.f;
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) rotate_in_wave(v[c], log4g);
  if (log4g >= 6) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) rotate_across_waves(v[c], log4g, buf, t);
  }
}

// How a row's codes are decided (uniform per row):
//   kCodeNearestEven: code_bits_rne(x, r_up), one operation.  r_up is the
//     smallest float32 above 1/s among r = RN(1/s) and r + 1 ulp (the sign
//     of the exact residual fma(-s, r, 1) tells which side of 1/s r lies):
//     where x / s is exactly a half-integer, x r_up lies strictly above it
//     and rounds away from zero, as the oracle's decision does; r_up has at
//     least 9 significant bits, so x r_up itself is never an exact tie.
//     Values within one ulp of r_up (relative) below a half-integer also
//     round up, as values within half an ulp do in the oracle's float32
//     quotient: a rounding-tie difference.
//   kCodeHalfAway: code_of(x, r), for r = 0 and powers of two (x r is then
//     exact and the decision exactly round half away of x / s, as at unit
//     scale) and the rare r_up without 9 significant bits.
//   kCodeTiny: tiny rows (pre-scaled and clamped).
enum { kCodeNearestEven = 0, kCodeHalfAway = 1, kCodeTiny = 2 };

// Scale of a row from the absmax mx of its unnormalised rotation (2^n X_rot):
// s = (mx 2^-n) / 127, the value stored.  Returns s; sets the row's code
// decision and r, the multiplier it uses: RN(1 / s_un) (s_un = s 2^n, so
// x_un / s_un == x / s exactly; 0 for a zero row), or r_up for
// kCodeNearestEven.  Rows
// whose absmax is below kTinyRowMax are "tiny": r is formed for s_un 2^64
// instead, and their values must be multiplied by 2^64 (exactly) and their
// codes clamped.
CR_DEVICE float row_scale(float mx, int log4g, float& r, int& mode) {
  mx = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mx)));  // uniform: one per row
  const float m = ldexpf(mx, -log4g);
  const float s = m / 127.0f;
  const bool tiny = m < kTinyRowMax;
  float s_un = ldexpf(s, log4g);
  if (tiny) s_un *= kTinyRowScale;
  r = (s_un != 0.f) ? 1.0f / s_un : 0.f;
  const float r_up =
      __uint_as_float(__float_as_uint(r) + (__builtin_fmaf(-s_un, r, 1.0f) > 0.f ? 1u : 0u));
  const bool nearest = !tiny && (__float_as_uint(r) & 0x7FFFFFu) != 0u && no_exact_ties(r_up);
  mode = __builtin_amdgcn_readfirstlane(tiny ? kCodeTiny : nearest ? kCodeNearestEven : kCodeHalfAway);
  if (nearest) r = r_up;
  return s;
}

template <int CPT>
CR_DEVICE float local_absmax(const float (&v)[CPT][16]) {
  float m = 0.f;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[c][e]));
  return m;
}

template <int CPT>
CR_DEVICE void quantize_store(float (&v)[CPT][16], int seg, int nch, float r, int mode,
                              int8_t* __restrict__ qr, int t, int T) {
  const int tp = chunk_of_thread(t);
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int j = (seg * CPT + c) * T + tp;
    if (j >= nch) continue;
    int qi[16];
    if (mode == kCodeNearestEven) {
#pragma unroll
      for (int e = 0; e < 16; ++e) qi[e] = code_bits_rne(v[c][e], r);
    } else if (mode == kCodeHalfAway) {
#pragma unroll
      for (int e = 0; e < 16; ++e) qi[e] = code_of(v[c][e], r);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) qi[e] = code_of_clamped(v[c][e] * kTinyRowScale, r);
    }
    uint4 o;
    o.x = pack4(qi[0], qi[1], qi[2], qi[3]);
    o.y = pack4(qi[4], qi[5], qi[6], qi[7]);
    o.z = pack4(qi[8], qi[9], qi[10], qi[11]);
    o.w = pack4(qi[12], qi[13], qi[14], qi[15]);
    *reinterpret_cast<uint4*>(qr + (int64_t)j * 16) = o;
  }
}

template <typename InT, int CPT>
__global__ __launch_bounds__(1024) void pack_kernel(const InT* __restrict__ x, int64_t ldx,
                                                    int m, int k, int log4g, int nseg,
                                                    int8_t* __restrict__ q,
                                                    float* __restrict__ scale) {
  extern __shared__ float4 lds_buf[];  // T * 16 floats, only when log4g >= 6
  __shared__ float wave_max[16];
  const int T = blockDim.x;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int nwaves = T >> 6;
  const int nch = k >> 4;

  for (int row = blockIdx.x; row < m; row += gridDim.x) {
    const InT* xr = x + (int64_t)row * ldx;
    int8_t* qr = q + (int64_t)row * k;
    float v[CPT][16];
    float mx = 0.f;
    for (int seg = 0; seg < nseg; ++seg) {
      load_rotate_segment<InT, CPT>(xr, seg, nch, log4g, v, lds_buf, t, T);
      mx = fmaxf(mx, local_absmax<CPT>(v));
    }
    mx = wave_max_nonneg(mx);
    if (lane == 0) wave_max[wave] = mx;
    __syncthreads();
    mx = wave_max[0];
    for (int w = 1; w < nwaves; ++w) mx = fmaxf(mx, wave_max[w]);
    __syncthreads();  // wave_max is rewritten for the next row

    int mode;
    float r;
    const float s = row_scale(mx, log4g, r, mode);
    if (t == 0) scale[row] = s;
    if (nseg == 1) {
      quantize_store<CPT>(v, 0, nch, r, mode, qr, t, T);
    } else {
      for (int seg = 0; seg < nseg; ++seg) {
        load_rotate_segment<InT, CPT>(xr, seg, nch, log4g, v, lds_buf, t, T);
        quantize_store<CPT>(v, seg, nch, r, mode, qr, t, T);
      }
    }
  }
}

// ---- fast path helpers: the same transforms in forms that need no register
// copies (every instruction writes a fresh value or folds its lane exchange).

// 2 * H4 on four registers: y_i = S - 2 x_{3-i} with S = (a+b)+(c+d), the
// four products as three-operand FMAs (the two-operand accumulating form
// would need a copy of S for each output).
CR_DEVICE float fma_m2(float x, float s) {
  float y;
  asm("v_fma_f32 %0, %1, -2.0, %2" : "=v"(y) : "v"(x), "v"(s));
  return y;
}
CR_DEVICE void h4_reg_pq(float& a, float& b, float& c, float& d) {
  const float s = (a + b) + (c + d);
  const float y0 = fma_m2(d, s), y1 = fma_m2(c, s), y2 = fma_m2(b, s), y3 = fma_m2(a, s);
  a = y0;
  b = y1;
  c = y2;
  d = y3;
}

template <int kCtrl>
CR_DEVICE float lane_mov(float v) {  // lane exchange that folds into its user
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, true));
}

// Lane digits: y = S - 2 x_rev with S the sum over the digit's four lanes;
// m2 holds -2 in a register so the last step is one fmac with a lane operand.
CR_DEVICE float h4_quad_f(float x, float m2) {
  const float t = x + lane_mov<kDppQuadSwap1>(x);
  const float s = t + lane_mov<kDppQuadSwap2>(t);
  return __builtin_fmaf(lane_mov<kDppQuadRev>(x), m2, s);
}
CR_DEVICE float h4_row_f(float x, float m2) {
  const float t = x + lane_mov<kDppRowRor4>(x);
  const float s = t + lane_mov<kDppRowRor8>(t);
  return __builtin_fmaf(lane_mov<kDppRowRor8>(x), m2, s);
}

CR_DEVICE void rotate_fast(float* v, int log4g, float m2) {
  if (log4g >= 1) {
#pragma unroll
    for (int a = 0; a < 4; ++a) h4_reg_pq(v[4 * a], v[4 * a + 1], v[4 * a + 2], v[4 * a + 3]);
  }
  if (log4g >= 2) {
#pragma unroll
    for (int a = 0; a < 4; ++a) h4_reg_pq(v[a], v[a + 4], v[a + 8], v[a + 12]);
  }
  if (log4g >= 3) {
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = h4_quad_f(v[e], m2);
  }
  if (log4g >= 4) {
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = h4_row_f(v[e], m2);
  }
  if (log4g >= 5) {
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = h4_wave(v[e]);
  }
}

// Four clamped codes (low bytes of a, b, c, d) into one word.
CR_DEVICE uint32_t pack4_perm(int a, int b, int c, int d) {
  const uint32_t lo = __builtin_amdgcn_perm(uint32_t(b), uint32_t(a), 0x0c0c0400u);  // [a0 b0 0 0]
  const uint32_t hi = __builtin_amdgcn_perm(uint32_t(d), uint32_t(c), 0x04000c0cu);  // [0 0 c0 d0]
  return lo | hi;
}

template <typename InT>
struct RawChunk;  // one chunk (16 features) as loaded
template <>
struct RawChunk<uint16_t> {
  u32x4 w[2];
  CR_DEVICE void load(const uint16_t* p) {
    const u32x4* p4 = reinterpret_cast<const u32x4*>(p);
    w[0] = __builtin_nontemporal_load(p4);
    w[1] = __builtin_nontemporal_load(p4 + 1);
  }
  CR_DEVICE void unpack(float* v) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      v[8 * i + 0] = bf16_lo(w[i].x);
      v[8 * i + 1] = bf16_hi(w[i].x);
      v[8 * i + 2] = bf16_lo(w[i].y);
      v[8 * i + 3] = bf16_hi(w[i].y);
      v[8 * i + 4] = bf16_lo(w[i].z);
      v[8 * i + 5] = bf16_hi(w[i].z);
      v[8 * i + 6] = bf16_lo(w[i].w);
      v[8 * i + 7] = bf16_hi(w[i].w);
    }
  }
};
template <>
struct RawChunk<float> {
  f32x4 w[4];
  CR_DEVICE void load(const float* p) {
    const f32x4* p4 = reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __builtin_nontemporal_load(p4 + i);
  }
  CR_DEVICE void unpack(float* v) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[4 * i + 0] = w[i].x;
      v[4 * i + 1] = w[i].y;
      v[4 * i + 2] = w[i].z;
      v[4 * i + 3] = w[i].w;
    }
  }
};

// float32 rows for the LDS kernel, loaded as whole lines.  A lane owns 16
// contiguous features (64 bytes); loading them as four 16-byte pieces per
// lane touches every 128-byte line with four instructions, which measured
// 4.0 TB/s against 6.9 TB/s for instructions that each read 1 KB
// contiguous.  So load instruction i of a chunk set (64 lanes x 16
// features = 4 KB) reads its 1 KB contiguous -- lane j the 16-byte piece
// i*64 + 4 (j % 16) + j / 16 -- and the pieces reach their owners through
// the wave's LDS buffer: piece slot i*64 + j is written by lane j, and lane l
// reads its pieces 4l .. 4l+3 from slots (l / 16)*64 + 16k + l % 16, sixteen
// consecutive slots per quarter-wave (no bank conflicts either way).
struct RawChunkLines {
  f32x4 w[4];
  CR_DEVICE void load(const float* set, int lane) {
    const f32x4* p4 = reinterpret_cast<const f32x4*>(set);
    const int j = 4 * (lane & 15) + (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __builtin_nontemporal_load(p4 + i * 64 + j);
  }
  CR_DEVICE void unpack(float* v, float* buf, int lane) const {
    f32x4* b4 = reinterpret_cast<f32x4*>(buf);
#pragma unroll
    for (int i = 0; i < 4; ++i) b4[i * 64 + lane] = w[i];
    const int base = (lane >> 4) * 64 + (lane & 15);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 q = b4[base + 16 * k];
      v[4 * k + 0] = q.x;
      v[4 * k + 1] = q.y;
      v[4 * k + 2] = q.z;
      v[4 * k + 3] = q.w;
    }
  }
};

// One wave per row at a time; a wave walks rows row0, row0 + W, ... (W waves
// in the grid) and loads the next row while it transforms the current one.
template <typename InT, int CPL>
__global__ __launch_bounds__(256) void pack_rows_kernel(const InT* __restrict__ x, int64_t ldx,
                                                        int m, int k, int log4g,
                                                        int8_t* __restrict__ q,
                                                        float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int nw = gridDim.x * 4;
  int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= m) return;  // the whole wave: no barriers below
  const int lp = chunk_of_thread(lane);
  float m2;
  asm volatile("v_mov_b32 %0, -2.0" : "=v"(m2));  // -2 in a register (see h4_quad_f)
  RawChunk<InT> raw[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) raw[c].load(x + (int64_t)row * ldx + (int64_t)(c * 64 + lp) * 16);
  for (; row < m; row += nw) {
    float v[CPL][16];
#pragma unroll
    for (int c = 0; c < CPL; ++c) raw[c].unpack(v[c]);
    const int nrow = row + nw;
    if (nrow < m) {
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        raw[c].load(x + (int64_t)nrow * ldx + (int64_t)(c * 64 + lp) * 16);
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) rotate_fast(v[c], log4g, m2);
    float mx = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(v[c][e]));
    mx = wave_max_nonneg(mx);
    int mode;
    float r;
    const float s = row_scale(mx, log4g, r, mode);
    if (lane == 0) scale[row] = s;
    int8_t* qr = q + (int64_t)row * k;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      int qi[16];
      if (mode == kCodeNearestEven) {
#pragma unroll
        for (int e = 0; e < 16; ++e) qi[e] = code_bits_rne(v[c][e], r);
      } else if (mode == kCodeHalfAway) {
#pragma unroll
        for (int e = 0; e < 16; ++e) qi[e] = code_of(v[c][e], r);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) qi[e] = code_of_clamped(v[c][e] * kTinyRowScale, r);
      }
      uint4 o;
      o.x = pack4_perm(qi[0], qi[1], qi[2], qi[3]);
      o.y = pack4_perm(qi[4], qi[5], qi[6], qi[7]);
      o.z = pack4_perm(qi[8], qi[9], qi[10], qi[11]);
      o.w = pack4_perm(qi[12], qi[13], qi[14], qi[15]);
      *reinterpret_cast<uint4*>(qr + (int64_t)(c * 64 + lp) * 16) = o;
    }
  }
}

// G = 64 and 256: the digits held by lane bits 0-3 are brought into registers
// by a 16 x 16 transpose through LDS inside each group of 16 lanes, so every
// butterfly stage is a register stage (two adds per element) and the lane
// exchange is LDS traffic instead of VALU work.  The codes return to the
// natural layout by a byte transpose through the same LDS buffer and leave
// as 16-byte stores.  For a row whose absmax m is not tiny, every |x| <= m
// and r = RN(1 / RN(m / 127)), so |x r| <= 127 (1 + 2^-23), which either
// decision rounds to at most 127: the code needs no clamp (tiny rows, whose
// subnormal scale may be rounded by far more, take the clamped path).
// The 16 x 16 float transpose of a 16-lane group: lane li writes its 16
// values as row li (four 16-byte writes) and reads column li back.  Rows are
// kTRow = 20 floats apart, so the 16 row starts of a write fall on 16
// distinct 4-bank groups (with 16-float rows four lanes shared one); the
// column reads stay 16 consecutive floats.  Groups are kTStride floats apart
// (a multiple of 64 banks plus 16, so the four groups' reads do not collide).
constexpr int kTRow = 20;
constexpr int kTStride = 16 * kTRow + 16;

// WPR waves share one row (rows longer than one wave holds): wave w of a
// workgroup takes part w % WPR of row slot w / WPR, the parts' maxima meet in
// LDS (one barrier per row).  All waves of a workgroup then walk the same
// number of rows, so a slot past the last row only joins the barrier.
template <typename InT, int CPL, int WPR>
__global__ __launch_bounds__(256) void pack_rows_lds_kernel(const InT* __restrict__ x,
                                                            int64_t ldx, int m, int k,
                                                            int log4g, int8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  static_assert(WPR == 1 || WPR == 2 || WPR == 4, "waves per row");
  constexpr int RPB = 4 / WPR;  // rows per workgroup at a time
  __shared__ __attribute__((aligned(16))) float tbuf[4][4 * kTStride];
  __shared__ float red[2][4];   // per-wave maxima, by row parity
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int part = wv % WPR;
  const int grp = lane >> 4, li = lane & 15;
  const int nr = gridDim.x * RPB;
  int row = blockIdx.x * RPB + wv / WPR;
  if (WPR == 1 && row >= m) return;  // the whole wave: no barriers below
  // This wave's part of a row: chunks part*CPL*64 .. (part+1)*CPL*64 - 1.
  const int64_t col0 = int64_t(part) * CPL * 64 * 16;
  float* tw = &tbuf[wv][grp * kTStride];
  constexpr bool kLines = std::is_same<InT, float>::value;  // float32: whole-line loads
  static_assert(4 * kTStride * 4 >= 64 * 64, "a wave's buffer holds one chunk set");
  typename std::conditional<kLines, RawChunkLines, RawChunk<InT>>::type raw[CPL];
  auto load_row = [&](int r) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const InT* set = x + (int64_t)r * ldx + col0 + (int64_t)c * 64 * 16;
      if constexpr (kLines)
        raw[c].load(set, lane);
      else
        raw[c].load(set + lane * 16);
    }
  };
  if (row < m) load_row(row);
  // One wave per row: the wave's own row decides; shared rows: the
  // workgroup's first row, so that every wave meets every barrier.
  for (int it = 0; WPR == 1 ? row < m : blockIdx.x * RPB + it * nr < m; ++it, row += nr) {
    const bool live = row < m;
    // t[c][i] = element li of chunk c*64 + 16*grp + i, after the transpose
    float t[CPL][16];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float v[16];
      if constexpr (kLines)
        raw[c].unpack(v, &tbuf[wv][0], lane);  // (in order with the transpose's LDS use)
      else
        raw[c].unpack(v);
#pragma unroll
      for (int a = 0; a < 4; ++a) h4_reg_pq(v[4 * a], v[4 * a + 1], v[4 * a + 2], v[4 * a + 3]);
#pragma unroll
      for (int a = 0; a < 4; ++a) h4_reg_pq(v[a], v[a + 4], v[a + 8], v[a + 12]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<f32x4*>(tw + li * kTRow + 4 * i) =
            f32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
#pragma unroll
      for (int i = 0; i < 16; ++i) t[c][i] = tw[i * kTRow + li];
    }
    const int nrow = row + nr;
    if (nrow < m) load_row(nrow);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
#pragma unroll
      for (int a = 0; a < 4; ++a) h4_reg_pq(t[c][4 * a], t[c][4 * a + 1], t[c][4 * a + 2], t[c][4 * a + 3]);
      if (log4g >= 4) {
#pragma unroll
        for (int a = 0; a < 4; ++a) h4_reg_pq(t[c][a], t[c][a + 4], t[c][a + 8], t[c][a + 12]);
      }
    }
    float mx = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(t[c][e]));
    mx = wave_max_nonneg(mx);
    if constexpr (WPR > 1) {
      if (lane == 0) red[it & 1][wv] = mx;
      __syncthreads();  // red[it & 1] is rewritten two rows later, after another barrier
#pragma unroll
      for (int w2 = 0; w2 < WPR; ++w2) mx = fmaxf(mx, red[it & 1][(wv / WPR) * WPR + w2]);
    }
    if (!live) continue;
    int mode;
    float r;
    const float s = row_scale(mx, log4g, r, mode);
    if (lane == 0 && part == 0) scale[row] = s;
    // The codes go back to the natural layout through LDS as bytes (lane li
    // writes byte li of each of its 16 chunks; lane li then reads chunk li
    // whole), so each chunk leaves as one 16-byte store.  The float
    // transpose above used the same buffer; a wave's LDS accesses run in
    // order, so its reads are done before these writes land.
    int8_t* tb = reinterpret_cast<int8_t*>(tw);
    int8_t* qr = q + (int64_t)row * k + col0 + (16 * grp + li) * 16;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      if (mode == kCodeNearestEven) {
#pragma unroll
        for (int i = 0; i < 16; ++i) tb[i * 16 + li] = (int8_t)code_bits_rne(t[c][i], r);
      } else if (mode == kCodeHalfAway) {
#pragma unroll
        for (int i = 0; i < 16; ++i) tb[i * 16 + li] = (int8_t)code_of(t[c][i], r);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          tb[i * 16 + li] = (int8_t)code_of_clamped(t[c][i] * kTinyRowScale, r);
      }
      *reinterpret_cast<u32x4*>(qr + c * 64 * 16) = *reinterpret_cast<const u32x4*>(tb + li * 16);
    }
  }
}

template <typename InT, int CPL, int WPR>
hipError_t launch_rows_t(const void* x, int64_t ldx, int m, int k, int log4g, int8_t* q,
                         float* scale, hipStream_t stream) {
  // One row per WPR waves, up to as many waves as the chip holds at once (the
  // kernel's register use decides how many fit per CU); beyond that each
  // wave walks several rows, loading the next while it transforms the
  // current one.  Only G = 64 and 256 split a row over several waves.
  const bool lds = (log4g == 3 || log4g == 4);
  if (WPR > 1 && !lds) return hipErrorInvalidValue;
  const void* fn = lds ? reinterpret_cast<const void*>(&pack_rows_lds_kernel<InT, CPL, WPR>)
                       : reinterpret_cast<const void*>(&pack_rows_kernel<InT, CPL>);
  static std::atomic<int> blocks_per_cu[2];
  int per_cu = blocks_per_cu[lds].load(std::memory_order_relaxed);
  if (per_cu == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess ||
        per_cu <= 0)
      per_cu = 2;
    blocks_per_cu[lds].store(per_cu, std::memory_order_relaxed);
  }
  const int64_t cap = int64_t(device_cu_count()) * per_cu * 4;
  const int64_t want = int64_t(m) * WPR;
  const int waves = int(want < cap ? want : cap);
  const int grid = (waves + 3) / 4;
  if (lds)
    hipLaunchKernelGGL((pack_rows_lds_kernel<InT, CPL, WPR>), dim3(grid), dim3(256), 0, stream,
                       static_cast<const InT*>(x), ldx, m, k, log4g, q, scale);
  else
    hipLaunchKernelGGL((pack_rows_kernel<InT, CPL>), dim3(grid), dim3(256), 0, stream,
                       static_cast<const InT*>(x), ldx, m, k, log4g, q, scale);
  return hipGetLastError();
}

// Rows of k = n * 1024 features: one wave per row for n <= 8; for G = 64
// and 256 also n = 10, 14 (two waves per row) and n = 12, 16, ..., 32 (four).
bool rows_supported(int64_t k, int log4g) {
  if (k % 1024 != 0) return false;
  const int64_t n = k / 1024;
  if (n >= 1 && n <= 8) return log4g <= 5;
  if (log4g != 3 && log4g != 4) return false;
  return n == 10 || n == 14 || (n % 4 == 0 && n <= 32);
}

template <typename InT>
hipError_t launch_rows(const void* x, int64_t ldx, int m, int k, int log4g, int8_t* q,
                       float* scale, hipStream_t stream) {
  switch (k / 1024) {
    case 1: return launch_rows_t<InT, 1, 1>(x, ldx, m, k, log4g, q, scale, stream);
    case 2: return launch_rows_t<InT, 2, 1>(x, ldx, m, k, log4g, q, scale, stream);
    case 3: return launch_rows_t<InT, 3, 1>(x, ldx, m, k, log4g, q, scale, stream);
    case 4: return launch_rows_t<InT, 4, 1>(x, ldx, m, k, log4g, q, scale, stream);
    case 5: return launch_rows_t<InT, 5, 1>(x, ldx, m, k, log4g, q, scale, stream);
    case 6: return launch_rows_t<InT, 6, 1>(x, ldx, m, k, log4g, q, scale, stream);
    case 7: return launch_rows_t<InT, 7, 1>(x, ldx, m, k, log4g, q, scale, stream);
    case 8: return launch_rows_t<InT, 8, 1>(x, ldx, m, k, log4g, q, scale, stream);
    case 10: return launch_rows_t<InT, 5, 2>(x, ldx, m, k, log4g, q, scale, stream);
    case 14: return launch_rows_t<InT, 7, 2>(x, ldx, m, k, log4g, q, scale, stream);
    case 12: return launch_rows_t<InT, 3, 4>(x, ldx, m, k, log4g, q, scale, stream);
    case 16: return launch_rows_t<InT, 4, 4>(x, ldx, m, k, log4g, q, scale, stream);
    case 20: return launch_rows_t<InT, 5, 4>(x, ldx, m, k, log4g, q, scale, stream);
    case 24: return launch_rows_t<InT, 6, 4>(x, ldx, m, k, log4g, q, scale, stream);
    case 28: return launch_rows_t<InT, 7, 4>(x, ldx, m, k, log4g, q, scale, stream);
    case 32: return launch_rows_t<InT, 8, 4>(x, ldx, m, k, log4g, q, scale, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename InT, int CPT>
hipError_t launch_pack_t(const void* x, int64_t ldx, int m, int k, int log4g, int threads,
                         int nseg, int8_t* q, float* scale, hipStream_t stream) {
  const int grid = m < (1 << 20) ? m : (1 << 20);
  const size_t lds = (log4g >= 6) ? size_t(threads) * 16 * sizeof(float) : 0;
  hipLaunchKernelGGL((pack_kernel<InT, CPT>), dim3(grid), dim3(threads), lds, stream,
                     static_cast<const InT*>(x), ldx, m, k, log4g, nseg, q, scale);
  return hipGetLastError();
}

}  // namespace

PackPlan plan_pack(int64_t k) {
  PackPlan p;
  const int64_t nch = k / 16;
  int64_t waves = (nch + 63) / 64;
  if (waves > 16) waves = 16;
  p.threads = int(waves * 64);
  const int64_t per_thread = (nch + p.threads - 1) / p.threads;
  // At most two chunks per thread: a 1024-thread workgroup leaves each wave
  // 128 registers, which four chunks would exceed (the compiler would spill
  // to scratch memory).  Longer rows are taken in segments and read twice.
  if (per_thread <= 1) {
    p.chunks_per_thread = 1;
    p.segments = 1;
  } else {
    p.chunks_per_thread = 2;
    p.segments = int((per_thread + 1) / 2);
  }
  return p;
}

hipError_t launch_pack(const void* x, bool bf16, int64_t ldx, int64_t m, int64_t k, int log4g,
                       int8_t* q, float* scale, hipStream_t stream) {
  const int mi = int(m), ki = int(k);
  if (rows_supported(k, log4g)) {
    return bf16 ? launch_rows<uint16_t>(x, ldx, mi, ki, log4g, q, scale, stream)
                : launch_rows<float>(x, ldx, mi, ki, log4g, q, scale, stream);
  }
  const PackPlan p = plan_pack(k);
  switch (p.chunks_per_thread * 2 + (bf16 ? 1 : 0)) {
    case 2: return launch_pack_t<float, 1>(x, ldx, mi, ki, log4g, p.threads, p.segments, q, scale, stream);
    case 3: return launch_pack_t<uint16_t, 1>(x, ldx, mi, ki, log4g, p.threads, p.segments, q, scale, stream);
    case 4: return launch_pack_t<float, 2>(x, ldx, mi, ki, log4g, p.threads, p.segments, q, scale, stream);
    case 5: return launch_pack_t<uint16_t, 2>(x, ldx, mi, ki, log4g, p.threads, p.segments, q, scale, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace convrot
