// Deterministic position gradients.
//
// The position streams add each edge's share to its sender (and each node's
// own share) with atomic additions, whose fp32 rounding depends on their
// order.  In the deterministic mode the streams run twice: the first fp32
// pass gives the magnitude of the result, from which a fixed-point shift F is
// chosen; the second adds every share as a 64-bit integer v * 2^F (modulo
// 2^64, exact, so the order does not matter), and the integers are turned
// back into fp32.  With five bits of headroom above max|g| (the fp32 pass may
// be off by its rounding where shares cancel) the sums cannot
// wrap, and the absolute resolution 2^-F is about 2^-57 max|g|.
#include <cmath>

#include "kernels.h"
#include "timing.h"

namespace tpconv {

namespace {

__global__ void fixed_max_kernel(const float* g, int64_t n, uint32_t* maxbits) {
  __shared__ uint32_t red[256];
  uint32_t m = 0u;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float v = fabsf(g[i]);
    const uint32_t b = __float_as_uint(v);
    m = (v == v && b > m) ? b : m;  // the bits of a non-negative float order as the float does
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicMax(maxbits, red[0]);
}

__global__ void fixed_shift_kernel(const uint32_t* maxbits, int32_t* shift) {
  const float G = __uint_as_float(*maxbits);
  int F = 0;
  if (G > 0.f && isfinite(G)) {
    int ex = 0;
    frexpf(G, &ex);  // G < 2^ex
    F = 58 - ex;     // |sum| * 2^F < 2^58: five bits below the sign
  }
  *shift = max(-60, min(F, 140));
}

__global__ void fixed_to_float_kernel(const unsigned long long* acc, const int32_t* shift, float* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = (float)ldexp((double)(long long)acc[i], -*shift);
}

}  // namespace

hipError_t launch_fixed_shift(const float* g, int64_t n, uint32_t* maxbits, int32_t* shift, hipStream_t s) {
  if (n < 0 || !maxbits || !shift || (n > 0 && !g)) return hipErrorInvalidValue;
  TimingScope ts(kcFill, s);
  hipLaunchKernelGGL(fixed_max_kernel, dim3(1024), dim3(256), 0, s, g, n, maxbits);
  hipLaunchKernelGGL(fixed_shift_kernel, dim3(1), dim3(1), 0, s, maxbits, shift);
  return hipGetLastError();
}

hipError_t launch_fixed_to_float(const unsigned long long* acc, const int32_t* shift, float* out, int64_t n,
                                 hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (!acc || !shift || !out || (n + 255) / 256 > INT32_MAX) return hipErrorInvalidValue;
  TimingScope ts(kcFill, s);
  hipLaunchKernelGGL(fixed_to_float_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, acc, shift, out, n);
  return hipGetLastError();
}

}  // namespace tpconv
