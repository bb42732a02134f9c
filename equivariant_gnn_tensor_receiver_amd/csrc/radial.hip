// Weight gradient of the radial MLP in front of the streams.
//
// With R_k = silu(sum_j A[k, j] B_j(d)) the loss depends on A only through
// the radial functions, and the receiver state is linear in them:
// S_v[k] = sum_e R_e[k] U_e.  So dL/dA[k, j] = <gS[k], S^(j)[k]>, where gS is
// the state cotangent and S^(j) the state streamed with R_e[k] replaced by
// dR_e[k]/dA[k, j] = silu'(z_ek) B_j(d_e) (the streams' mlp_col = j mode);
// for the force loss the tangent state takes the place of S ("Sobek" page,
// abstract: the streaming form covers the backward and double backward with
// node-sized state only).  These kernels form the per-k dot products of two
// states, deterministically: K sums per chunk of rows, then one block per k
// adds them in block order.
#include "kernels.h"
#include "timing.h"

namespace tpconv {

namespace {

constexpr int kDotThreads = 256;
constexpr int kDotMaxK = 16;

// Sum of one value per thread over the block in a fixed order (tree in LDS).
__device__ __forceinline__ float block_sum(float v, float* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int w = kDotThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();  // red is reused by the next call
  return r;
}

// Block b: rows [r0, r1) of its group; for each k, thread t takes the columns
// k * cpk + c, c = t, t + 256, .. (consecutive threads, consecutive columns of
// a row) over all rows, then the block sums the threads' values.
__global__ __launch_bounds__(kDotThreads) void state_dot_rows_kernel(const StateDotArgs a) {
  __shared__ float red[kDotThreads];
  const int b = blockIdx.x;
  int g = 0;
  while (g + 1 < a.ngroups && b >= a.chunk_begin[g + 1]) ++g;
  const int chunk = b - a.chunk_begin[g];
  const int64_t r0 = (int64_t)chunk * a.rows_per_chunk;
  const int64_t r1 = min(a.rows[g], r0 + a.rows_per_chunk);
  const int cols = a.cols[g], cpk = a.cpk[g];
  const float* pa = a.a + a.base[g];
  const float* pb = a.b + a.base[g];
  for (int k = 0; k < a.K; ++k) {
    float acc = 0.f;
    for (int c = threadIdx.x; c < cpk; c += kDotThreads) {
      const int col = k * cpk + c;
      for (int64_t r = r0; r < r1; ++r) acc = __builtin_fmaf(pa[r * cols + col], pb[r * cols + col], acc);
    }
    const float t = block_sum(acc, red);
    if (threadIdx.x == 0) a.part[(int64_t)b * a.K + k] = t;
  }
}

__global__ __launch_bounds__(kDotThreads) void state_dot_reduce_kernel(const StateDotArgs a) {
  __shared__ float red[kDotThreads];
  const int k = blockIdx.x;
  float acc = 0.f;
  for (int b = threadIdx.x; b < a.nblocks; b += kDotThreads) acc += a.part[(int64_t)b * a.K + k];
  const float t = block_sum(acc, red);
  if (threadIdx.x == 0) a.out[(int64_t)k * a.out_stride + a.out_col] = t;
}

}  // namespace

hipError_t launch_state_dot(const StateDotArgs& a, hipStream_t s) {
  if (a.ngroups <= 0 || a.ngroups > kMaxGroups || a.K <= 0 || a.K > kDotMaxK || a.rows_per_chunk <= 0)
    return hipErrorInvalidValue;
  int64_t blocks = 0;
  for (int g = 0; g < a.ngroups; ++g) {
    if (a.chunk_begin[g] != blocks || a.cols[g] != a.K * a.cpk[g]) return hipErrorInvalidValue;
    blocks += a.nchunks[g];
  }
  if (blocks != a.nblocks || blocks <= 0) return hipErrorInvalidValue;
  TimingScope ts(kcStateDot, s);
  hipLaunchKernelGGL(state_dot_rows_kernel, dim3((unsigned)blocks), dim3(kDotThreads), 0, s, a);
  hipLaunchKernelGGL(state_dot_reduce_kernel, dim3((unsigned)a.K), dim3(kDotThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace tpconv
