/* Host emulation of the activation pack's float32 code arithmetic (tests only).
 *
 * The pack kernels decide each int8 code of a row from its rotated values held
 * unnormalised, x_un = 2^n X_rot (n = log4 G; the butterfly's factor 2 per
 * stage is exact), and the row maximum mx = max |x_un|:
 *   m = mx 2^-n, s = RN(m / 127) (stored), s_un = s 2^n, r = RN(1 / s_un);
 *   if r is neither 0 nor a power of two, r_up = r when r > 1 / s_un, else r
 *   raised by one unit in its last place (the sign of the exact residual
 *   fma(-s_un, r, 1) decides; r_up > 1 / s_un strictly), and if the low 16
 *   bits of r_up's encoding are not all zero (r_up has at least 9
 *   significant bits):
 *   code = low byte of RN(x_un r_up + 1.5 2^23), i.e. the exact product
 *   x_un r_up rounded to nearest, ties to even (there are none);
 *   otherwise code = trunc(RN(x_un r + copysign(0.5 - 2^-25, x_un)));
 * rows with m < 2^-100 ("tiny") use s_un 2^64 and x_un 2^64 instead (both
 * exact) and clamp the code to [-127, 127].  This file restates those steps
 * in C with the host's correctly rounded float32 operations (fmaf), so that
 * tests can check them against the oracle on inputs the GPU never sees.  It
 * shares nothing with the kernels or the oracle.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float float_of_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* The rounding step alone, at unit scale (r = 1): the number of float32 v
 * with bit patterns lo..hi (non-negative floats), each taken with both signs,
 * for which trunc(RN(v * 1 + copysign(half, v))) differs from round(v), C's
 * round half away from zero.  The kernels use half = 0.5 - 2^-25; lo = 0,
 * hi = bits of 128.0f covers every |v| <= 128. */
long long round_step_mismatches(float half, uint32_t lo, uint32_t hi) {
  long long bad = 0;
  for (uint32_t u = lo; u <= hi; ++u) {
    const float v = float_of_bits(u);
    const int p = (int)fmaf(v, 1.0f, half);
    const int q = (int)fmaf(-v, 1.0f, -half);
    bad += (p != (int)roundf(v)) + (q != (int)roundf(-v));
  }
  return bad;
}

/* splitmix64: a seeded stream of 64-bit values for the random checks below. */
static uint64_t next_u64(uint64_t* state) {
  uint64_t z = (*state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* The low byte of RN(x r + 1.5 2^23) as a signed code. */
static int rne_code(float x, float r) {
  const float f = fmaf(x, r, 0x1.8p23f);
  uint32_t b;
  memcpy(&b, &f, sizeof b);
  return (int)(int8_t)(b & 0xFFu);
}

/* Round half away from zero of the exact product x r (24 x 24 bits: exact in
 * a double, and so is |p| + 0.5 for |p| < 128). */
static int half_away_code(float x, float r) {
  const double p = (double)x * (double)r;
  return p >= 0.0 ? (int)floor(p + 0.5) : -(int)floor(-p + 0.5);
}

/* The nearest-even step against round half away from zero of the exact
 * product, for each of the nr multipliers rs[i]: every x = RN((k + 1/2) / r)
 * for k = -128 .. 127 together with its four float32 neighbours on each
 * side (the values nearest each tie), plus xs_per_r random x with
 * |x r| < 127.5.  Returns the number of (x, r) pairs whose codes differ. */
long long rne_step_mismatches(const float* rs, long nr, long xs_per_r, uint64_t seed) {
  long long bad = 0;
  uint64_t st = seed;
  for (long i = 0; i < nr; ++i) {
    const float r = rs[i];
    for (int k = -128; k < 128; ++k) {
      float x = (float)(((double)k + 0.5) / (double)r);
      for (int j = 0; j < 4; ++j) x = nextafterf(x, -INFINITY);
      for (int j = 0; j < 9; ++j, x = nextafterf(x, INFINITY)) {
        if (fabs((double)x * (double)r) >= 127.5) continue;
        bad += rne_code(x, r) != half_away_code(x, r);
      }
    }
    for (long j = 0; j < xs_per_r; ++j) {
      const double u = (double)(next_u64(&st) >> 11) * 0x1p-53 * 255.0 - 127.5;  /* [-127.5, 127.5) */
      const float x = (float)(u / (double)r);
      if (fabs((double)x * (double)r) >= 127.5) continue;
      bad += rne_code(x, r) != half_away_code(x, r);
    }
  }
  return bad;
}

/* One row as the kernels quantise it.  x_un: k values 2^n X_rot as float32;
 * writes the k codes and the stored scale. */
void emulate_row(const float* x_un, long k, int n, int8_t* q, float* scale) {
  float mx = 0.0f;
  for (long i = 0; i < k; ++i) mx = fmaxf(mx, fabsf(x_un[i]));
  const float m = ldexpf(mx, -n);
  const float s = m / 127.0f;
  const int tiny = m < 0x1p-100f;
  float s_un = ldexpf(s, n);
  if (tiny) s_un *= 0x1p64f;
  const float r = (s_un != 0.0f) ? 1.0f / s_un : 0.0f;
  const float half = 0x1.fffffep-2f;
  uint32_t rb;
  memcpy(&rb, &r, sizeof rb);
  const uint32_t ub = rb + (fmaf(-s_un, r, 1.0f) > 0.0f ? 1u : 0u);
  float r_up;
  memcpy(&r_up, &ub, sizeof r_up);
  const int rne = !tiny && (rb & 0x7FFFFFu) != 0 && (ub & 0xFFFFu) != 0;
  for (long i = 0; i < k; ++i) {
    if (rne) {
      q[i] = (int8_t)rne_code(x_un[i], r_up);
    } else if (!tiny) {
      q[i] = (int8_t)(int)fmaf(x_un[i], r, copysignf(half, x_un[i]));
    } else {
      const float x = x_un[i] * 0x1p64f;
      float f = fmaf(x, r, copysignf(half, x));
      f = fminf(fmaxf(f, -127.0f), 127.0f);
      q[i] = (int8_t)(int)f;
    }
  }
  *scale = s;
}
