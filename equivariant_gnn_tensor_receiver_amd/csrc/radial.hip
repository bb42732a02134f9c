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
// registers and writes only each tile's dot with gS per k (dot_state mode),
// column j into its own slab; this kernel adds the per-item sums of all
// columns in one launch, in a fixed order.
#include "kernels.h"
#include "timing.h"

namespace tpconv {

namespace {

constexpr int kDotThreads = 1024;

// One block per column j reads that column's slab [nitems][K] front to back
// (coalesced).  Thread t < R*K (R a power of two) owns k = t % K and adds the
// slab entries t, t + R*K, t + 2*R*K, ... in that order; the R partial sums
// of each k are then added by a fixed tree.  The result depends on nothing
// but the inputs.
__global__ __launch_bounds__(kDotThreads) void dot_reduce_kernel(const float* part, int64_t nitems, int K, int R,
                                                                 float* out, int stride) {
  __shared__ float red[kDotThreads];
  const int j = blockIdx.x, t = threadIdx.x, T = R * K;
  const int64_t n = nitems * K;
  const float* slab = part + (int64_t)j * n;
  float acc = 0.f;
  if (t < T) {
#pragma unroll 4
    for (int64_t i = t; i < n; i += T) acc += slab[i];
  }
  red[t] = acc;
  __syncthreads();
  for (int w = R / 2; w > 0; w >>= 1) {
    if (t < w * K) red[t] += red[t + w * K];
    __syncthreads();
  }
  if (t < K) out[(int64_t)t * stride + j] = red[t];
}

}  // namespace

hipError_t launch_dot_reduce(const float* part, int64_t nitems, int K, int ncols, float* out, int stride,
                             hipStream_t s) {
  if (K <= 0 || K > kDotThreads || nitems < 0 || ncols <= 0 || ncols > stride || !out || (nitems > 0 && !part))
    return hipErrorInvalidValue;
  int R = 1;
  while (2 * R * K <= kDotThreads) R *= 2;
  TimingScope ts(kcStateDot, s);
  hipLaunchKernelGGL(dot_reduce_kernel, dim3((unsigned)ncols), dim3(kDotThreads), 0, s, part, nitems, K, R, out,
                     stride);
  return hipGetLastError();
}

}  // namespace tpconv
