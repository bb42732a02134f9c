// Ragged multiplicities ("Sobek" page, abstract: varied feature structures):
// conversions between the caller's ragged layout and the padded layout the
// kernels use, where every irrep of a side has the side's largest
// multiplicity and the extra channels are zero.  Zero input channels and zero
// weight rows / columns add nothing to any output or gradient, so padding,
// running the uniform operator and dropping the padded channels gives the
// ragged operator exactly.
#include "kernels.h"
#include "timing.h"

namespace tpconv {

namespace {

// Node tensors: padded [N][D][C] <-> ragged [N][F]; row r of a node holds the
// caller's features off[r] .. off[r] + mul[r] - 1.
template <typename T, bool PACK>
__global__ void nodes_kernel(const RaggedNodeMap m, const T* src, T* dst, int64_t N) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)m.D * m.C;
  if (i >= N * per) return;
  const int64_t n = i / per;
  const int rc = (int)(i - n * per);
  const int r = rc / m.C, c = rc - r * m.C;
  const bool inside = c < m.mul[r];
  const int64_t f = n * m.F + m.off[r] + c;
  if constexpr (PACK)
    dst[i] = inside ? src[f] : T(0);
  else if (inside)
    dst[f] = src[i];
}

// Weights: padded [K][P][Ci][Co] (channel-wise [K][P][C]) <-> ragged
// [K][W_per_k] with path p's block [c1][c3] (channel-wise [c1]) at woff[p].
template <typename T, bool PACK>
__global__ void weights_kernel(const RaggedWeightMap m, const T* src, T* dst, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t per_p = m.cw ? m.Ci : (int64_t)m.Ci * m.Co;
  const int64_t kp = i / per_p;
  const int rem = (int)(i - kp * per_p);
  const int k = (int)(kp / m.P), p = (int)(kp - (int64_t)k * m.P);
  const int ci = m.cw ? rem : rem / m.Co, co = m.cw ? 0 : rem - ci * m.Co;
  const bool inside = ci < m.c1[p] && (m.cw || co < m.c3[p]);
  const int64_t f = (int64_t)k * m.W_per_k + m.woff[p] + (m.cw ? ci : (int64_t)ci * m.c3[p] + co);
  if constexpr (PACK)
    dst[i] = inside ? src[f] : T(0);
  else if (inside)
    dst[f] = src[i];
}

inline unsigned blocks_of(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_ragged_nodes(const RaggedNodeMap& m, const void* src, void* dst, int64_t N, int elem_bytes,
                               bool pack, hipStream_t s) {
  const int64_t n = N * m.D * (int64_t)m.C;
  if (n <= 0) return hipSuccess;
  if ((n + 255) / 256 > INT32_MAX) return hipErrorInvalidValue;
  TimingScope ts(kcFill, s);
  if (elem_bytes == 2) {
    const auto* a = static_cast<const uint16_t*>(src);
    auto* b = static_cast<uint16_t*>(dst);
    if (pack)
      hipLaunchKernelGGL((nodes_kernel<uint16_t, true>), dim3(blocks_of(n)), dim3(256), 0, s, m, a, b, N);
    else
      hipLaunchKernelGGL((nodes_kernel<uint16_t, false>), dim3(blocks_of(n)), dim3(256), 0, s, m, a, b, N);
  } else {
    const auto* a = static_cast<const float*>(src);
    auto* b = static_cast<float*>(dst);
    if (pack)
      hipLaunchKernelGGL((nodes_kernel<float, true>), dim3(blocks_of(n)), dim3(256), 0, s, m, a, b, N);
    else
      hipLaunchKernelGGL((nodes_kernel<float, false>), dim3(blocks_of(n)), dim3(256), 0, s, m, a, b, N);
  }
  return hipGetLastError();
}

hipError_t launch_ragged_weights(const RaggedWeightMap& m, const void* src, void* dst, int elem_bytes, bool pack,
                                 hipStream_t s) {
  const int64_t total = (int64_t)m.K * m.P * m.Ci * (m.cw ? 1 : m.Co);
  if (total <= 0) return hipSuccess;
  TimingScope ts(kcFill, s);
  if (elem_bytes == 2) {
    const auto* a = static_cast<const uint16_t*>(src);
    auto* b = static_cast<uint16_t*>(dst);
    if (pack)
      hipLaunchKernelGGL((weights_kernel<uint16_t, true>), dim3(blocks_of(total)), dim3(256), 0, s, m, a, b, total);
    else
      hipLaunchKernelGGL((weights_kernel<uint16_t, false>), dim3(blocks_of(total)), dim3(256), 0, s, m, a, b, total);
  } else {
    const auto* a = static_cast<const float*>(src);
    auto* b = static_cast<float*>(dst);
    if (pack)
      hipLaunchKernelGGL((weights_kernel<float, true>), dim3(blocks_of(total)), dim3(256), 0, s, m, a, b, total);
    else
      hipLaunchKernelGGL((weights_kernel<float, false>), dim3(blocks_of(total)), dim3(256), 0, s, m, a, b, total);
  }
  return hipGetLastError();
}

}  // namespace tpconv
