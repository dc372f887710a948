// Shared device helpers for the convrot kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#define CR_DEVICE __device__ __forceinline__

namespace convrot {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kNumXcd = 8;     // accelerator complex dies; workgroups are dealt to them round robin
constexpr int kVmMax = 63;     // largest vmcnt a wait can name
// Word 3 of a raw buffer resource on gfx9-family GPUs (32-bit data format).
constexpr int kBufferWord3 = 0x00020000;
constexpr unsigned kOutOfRange = 0x80000000u;  // an offset past every resource
constexpr int kNonTemporal = 2;  // cache-policy bits of a buffer access: nt (streaming)

// A raw buffer resource over [base, base + bytes): loads at offsets past the
// end return zero (the hardware range check).
CR_DEVICE __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes,
                                           kBufferWord3);
}

// Position of workgroup b in a grid of n: workgroups go to the XCDs round
// robin (b % 8), and each XCD takes a contiguous run of positions, so
// neighbouring positions share that XCD's L2.
CR_DEVICE int xcd_slot(int b, int n) {
  const int xcd = b % kNumXcd, idx = b / kNumXcd;
  const int q = n / kNumXcd, rem = n % kNumXcd;
  return (xcd < rem) ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
}

// s_waitcnt vmcnt(N), other counters unchanged.  gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14].
template <int N>
CR_DEVICE void waitvm() {
  static_assert(N >= 0 && N <= kVmMax, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
CR_DEVICE void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// A bare s_barrier: the waits are issued explicitly (a __syncthreads fence
// would also drain loads still in flight for later stages), and the memory
// clobber keeps the compiler from moving LDS accesses across it.
CR_DEVICE void barrier() { asm volatile("s_barrier" ::: "memory"); }

// f(integral_constant<int, I>) for every I of the sequence, in order.
template <int... I, typename F>
CR_DEVICE void for_each_index(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}

// DPP controls (GCN "data parallel primitives" operand modifiers).
constexpr int kDppQuadSwap1 = 0xB1;    // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;    // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppQuadRev = 0x1B;      // quad_perm [3,2,1,0]: lane ^ 3
constexpr int kDppRowRor4 = 0x124;     // rotate by 4 lanes inside a row of 16
constexpr int kDppRowRor8 = 0x128;     // rotate by 8 lanes inside a row of 16 (= lane ^ 8)

template <int kCtrl>
CR_DEVICE float dpp_f32(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// bf16 bits -> float32 (exact).
CR_DEVICE float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
CR_DEVICE float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Activation code of a rotated value x, given r = RN(1/s) for the row scale s:
// round half away from zero of x r, as trunc(RN(x r + copysign(0.5 - 2^-25, x)))
// -- one fused multiply-add; the float->int conversion truncates toward zero.
// With r = 1 this is exactly round-half-away of x for every float32 |x| <= 128
// (checked exhaustively on the host).  For other scales x r differs from the
// correctly rounded x / s by at most about one unit in the last place, so a
// code can differ from round(x / s) only where x / s lies within a few ulp of a
// half-integer.  r = 0 (a zero row) gives 0.
CR_DEVICE int code_of(float x, float r) {
  return (int)__builtin_fmaf(x, r, __builtin_copysignf(0.49999997f, x));
}

// The same, clamped to [-127, 127]: for rows whose scale is subnormal, where
// the scale's own rounding can put |x r| above 127.5.
CR_DEVICE int code_of_clamped(float x, float r) {
  const float f = __builtin_fmaf(x, r, __builtin_copysignf(0.49999997f, x));
  return (int)__builtin_amdgcn_fmed3f(f, -127.0f, 127.0f);
}

// The code decision for a row whose multiplier r has at least 9 significant
// bits (no_exact_ties(r)): x r is then never exactly a half-integer for
// |x r| <= 127.5 (that needs odd(x) odd(r) = |2k + 1| <= 255, and the odd
// part of r's significand is at least 256), so rounding the exact product to
// nearest even is rounding it half away from zero, for every x.  The fused
// multiply-add RN(x r + 1.5 2^23) does that rounding and leaves the integer
// in the low mantissa bits in two's complement: the low byte of the result
// is the int8 code (callers use that byte only).  One operation per code.
CR_DEVICE int code_bits_rne(float x, float r) {
  return __float_as_int(__builtin_fmaf(x, r, 0x1.8p23f));
}
CR_DEVICE bool no_exact_ties(float r) { return (__float_as_uint(r) & 0xFFFFu) != 0u; }

// Rows whose absmax is below kTinyRowMax take the pre-scaled path: x and the
// scale are both multiplied by 2^64 (exact), so 1/s cannot overflow float32
// (it would for s below 2^-128), and the codes are clamped.
constexpr float kTinyRowMax = 0x1p-100f;
constexpr float kTinyRowScale = 0x1p64f;

CR_DEVICE int clamp127(int q) { return max(-127, min(127, q)); }

// GELU in its erf form, y Phi(y), with Phi the standard normal CDF.  For
// either sign of y, y Phi(y) = max(y, 0) - |y| h with h = Phi(-|y|).  h is
// 2^P(t), t = min(|y|, 6) / 6, with P the degree-5 polynomial that
// gelu_fit.py fits to log2 Phi(-a) on [0, 6], weighted by how much an error
// of P moves the GELU value (|y| h ln2 per unit, relative to max(1, |y|)):
// the float32 result stays within 3.3e-7 max(1, |y|) of y Phi(y), and
// Phi(-6) < 1e-9 bounds what the clamp at 6 leaves out.  Nine full-rate
// vector operations and one base-2 exponential per value (t is a single
// multiply whose output clamp bit does the min); the GEMM epilogue evaluates
// it for every output, and each vector instruction costs matrix-core time.
CR_DEVICE float gelu_erf(float y) {
  const float t = fminf(fmaxf(fabsf(y) * 0.16666667f, 0.0f), 1.0f);
  float p = -3.9505641f;
  p = __builtin_fmaf(p, t, 9.483913f);
  p = __builtin_fmaf(p, t, -11.315078f);
  p = __builtin_fmaf(p, t, -16.538921f);
  p = __builtin_fmaf(p, t, -6.9062366f);
  p = __builtin_fmaf(p, t, -1.0000027f);
  const float h = __builtin_amdgcn_exp2f(p);
  return __builtin_fmaf(-fabsf(y), h, fmaxf(y, 0.0f));
}

}  // namespace convrot
