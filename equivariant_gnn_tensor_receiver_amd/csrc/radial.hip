// Weight gradient of the radial MLP in front of the streams.
//
// With R_k = silu(sum_j A[k, j] B_j(d)) the loss depends on A only through
// the radial functions, and the receiver state is linear in them:
// S_v[k] = sum_e R_e[k] U_e.  So dL/dA[k, j] = <gS[k], S^(j)[k]>, where gS is
// the state cotangent and S^(j) the state streamed with R_e[k] replaced by
// dR_e[k]/dA[k, j] = silu'(z_ek) B_j(d_e) (the streams' mlp_col = j mode);
// for the force loss the tangent state takes the place of S ("Sobek" page,
// abstract: the streaming form covers the backward and double backward with
// node-sized state only).  The receiver stream forms S^(j) tile by tile in
// registers and writes only each tile's dot with gS per k (dot_state mode);
// this kernel adds those per-item sums in a fixed order.
#include "kernels.h"
#include "timing.h"

namespace tpconv {

namespace {

constexpr int kDotThreads = 256;

__global__ __launch_bounds__(kDotThreads) void dot_reduce_kernel(const float* part, int64_t nblocks, int K,
                                                                 float* out, int col, int stride) {
  __shared__ float red[kDotThreads];
  const int k = blockIdx.x;
  float acc = 0.f;
  for (int64_t b = threadIdx.x; b < nblocks; b += kDotThreads) acc += part[b * K + k];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kDotThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[(int64_t)k * stride + col] = red[0];
}

}  // namespace

hipError_t launch_dot_reduce(const float* part, int64_t nblocks, int K, float* out, int col, int stride,
                             hipStream_t s) {
  if (K <= 0 || nblocks < 0 || col < 0 || col >= stride || !out || (nblocks > 0 && !part)) return hipErrorInvalidValue;
  TimingScope ts(kcStateDot, s);
  hipLaunchKernelGGL(dot_reduce_kernel, dim3((unsigned)K), dim3(kDotThreads), 0, s, part, nblocks, K, out, col,
                     stride);
  return hipGetLastError();
}

}  // namespace tpconv
