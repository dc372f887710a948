// Shared device helpers for the convrot kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define CR_DEVICE __device__ __forceinline__

namespace convrot {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

// Round half away from zero, then to int32, for |v| <= 128.
// trunc(v + copysign(0.5 - 2^-25, v)) equals round-half-away for every float32
// of magnitude at most 128 (checked exhaustively on the host); the float->int
// conversion truncates toward zero.
CR_DEVICE int round_half_away_small(float v) {
  return (int)(v + __builtin_copysignf(0.49999997f, v));
}

// Correctly rounded float32 quotient x / b from r = RN(1/b): one product, one
// residual and one correction (Markstein's theorem for round-to-nearest).
CR_DEVICE float div_by_recip(float x, float b, float r) {
  float q = x * r;
  float e = __builtin_fmaf(-q, b, x);
  return __builtin_fmaf(e, r, q);
}

CR_DEVICE int clamp127(int q) { return max(-127, min(127, q)); }

}  // namespace convrot
