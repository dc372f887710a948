/* Host emulation of the activation pack's float32 code arithmetic (tests only).
 *
 * The pack kernels decide each int8 code of a row from its rotated values held
 * unnormalised, x_un = 2^n X_rot (n = log4 G; the butterfly's factor 2 per
 * stage is exact), and the row maximum mx = max |x_un|:
 *   m = mx 2^-n, s = RN(m / 127) (stored), s_un = s 2^n, r = RN(1 / s_un);
 *   code = trunc(RN(x_un r + copysign(0.5 - 2^-25, x_un)));
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
  for (long i = 0; i < k; ++i) {
    if (!tiny) {
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
