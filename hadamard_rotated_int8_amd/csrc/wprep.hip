// Offline weight preparation in float64: W_rot = W R, per-row absmax, int8 codes.
//
// Implements the stable-diffusion.cpp page "INT8 Convrot Safetensors",
// sections "How INT8 convrot works" (W_rot = W R with the block-diagonal R)
// and "Weight quantization":
//   s_w[o] = max_i |W_rot[o, i]| / 127,  Q_w[o, i] = clamp(round(W_rot[o, i] / s_w[o]), -127, 127).
// The rotation, absmax, division and rounding run in float64; the float64
// quotient max/127 is rounded once to the stored float32 scale and the codes
// divide by that stored value.  This is not on the hot path (it runs once per
// checkpoint), so it favours a simple, general structure: one workgroup per
// weight row, the row taken in segments of whole groups staged in LDS, radix-4
// butterflies over LDS, and two passes (absmax, then codes) that re-read W.
#include "common.h"
#include "kernels.h"

namespace convrot {
namespace {

constexpr int kWprepThreads = 256;

// Rotate `len` doubles in LDS (len is a multiple of 4^log4g) in place.
CR_DEVICE void rotate_lds(double* seg, int len, int log4g, int t) {
  int stride = 1;
  for (int dg = 0; dg < log4g; ++dg) {
    __syncthreads();
    const int nbf = len >> 2;
    for (int b = t; b < nbf; b += kWprepThreads) {
      const int lo = b % stride;
      const int hi = b / stride;
      double* p = seg + hi * 4 * stride + lo;
      const double x0 = p[0], x1 = p[stride], x2 = p[2 * stride], x3 = p[3 * stride];
      const double s = (x0 + x1) + (x2 + x3);
      // (H4 x)_d = sum/2 - x_{3-d}
      p[0] = __builtin_fma(0.5, s, -x3);
      p[stride] = __builtin_fma(0.5, s, -x2);
      p[2 * stride] = __builtin_fma(0.5, s, -x1);
      p[3 * stride] = __builtin_fma(0.5, s, -x0);
    }
    stride *= 4;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kWprepThreads) void wprep_kernel(const float* __restrict__ w,
                                                              int64_t ldw, int n, int k,
                                                              int log4g, int seg_len,
                                                              int8_t* __restrict__ q,
                                                              float* __restrict__ scale) {
  extern __shared__ double seg[];
  __shared__ double red[kWprepThreads / 64];
  const int t = threadIdx.x;
  for (int row = blockIdx.x; row < n; row += gridDim.x) {
    const float* wr = w + (int64_t)row * ldw;
    int8_t* qr = q + (int64_t)row * k;
    double sd = 0.0;
    for (int pass = 0; pass < 2; ++pass) {
      double mx = 0.0;
      for (int s0 = 0; s0 < k; s0 += seg_len) {
        const int len = (k - s0 < seg_len) ? (k - s0) : seg_len;
        __syncthreads();
        for (int i = t; i < len; i += kWprepThreads) seg[i] = (double)wr[s0 + i];
        rotate_lds(seg, len, log4g, t);
        if (pass == 0) {
          for (int i = t; i < len; i += kWprepThreads) mx = fmax(mx, fabs(seg[i]));
        } else {
          for (int i = t; i < len; i += kWprepThreads) {
            int code = 0;
            if (sd != 0.0) {
              const double v = seg[i] / sd;  // IEEE float64 division
              code = clamp127((int)round(v));  // round(): half away from zero
            }
            qr[s0 + i] = (int8_t)code;
          }
        }
      }
      if (pass == 0) {
        for (int off = 32; off >= 1; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off));
        if ((t & 63) == 0) red[t >> 6] = mx;
        __syncthreads();
        mx = red[0];
        for (int i = 1; i < kWprepThreads / 64; ++i) mx = fmax(mx, red[i]);
        const float s = (float)(mx / 127.0);  // float64 quotient rounded once to float32
        sd = (double)s;
        if (t == 0) scale[row] = s;
        __syncthreads();
      }
    }
  }
}

}  // namespace

hipError_t launch_wprep(const float* w, int64_t n, int64_t k, int64_t ldw, int log4g, int8_t* q,
                        float* scale, hipStream_t stream) {
  const int g = 1 << (2 * log4g);
  int seg_len = g > 4096 ? g : 4096;
  if (seg_len > k) seg_len = int(k);  // k is a multiple of g
  const size_t lds = size_t(seg_len) * sizeof(double);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&wprep_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  const int grid = n < 65536 ? int(n) : 65536;
  hipLaunchKernelGGL(wprep_kernel, dim3(grid), dim3(kWprepThreads), lds, stream, w, ldw, int(n),
                     int(k), log4g, seg_len, q, scale);
  return hipGetLastError();
}

}  // namespace convrot
