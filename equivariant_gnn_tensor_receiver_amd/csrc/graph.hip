// Graph preparation: CSR validation, the sender-sorted view used by the
// sender-side streams of the backward passes, and a spatial visiting order of
// the nodes.
//
// The view stores, for every sender, the receivers of its out-edges in
// increasing order (a stable sort by sender of the receiver-sorted edges).
// Built as: histogram of senders -> exclusive scan (colptr) -> scatter with
// per-sender cursors -> sort inside each segment.  Because a segment holds
// only receiver ids, the sorted segment is unique and the result is
// deterministic even though the scatter order is not.
#include "kernels.h"
#include "timing.h"

namespace tpconv {

namespace {

__global__ void fill_i32(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void validate_kernel(const int32_t* rowptr, const int32_t* senders, int64_t N, int64_t E,
                                int32_t* flag) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int bad = 0;
  if (i <= N) {
    const int32_t a = rowptr[i];
    if (a < 0 || a > E) bad = 1;
    if (i == 0 && a != 0) bad = 1;
    if (i == N && a != E) bad = 1;
    if (i < N && rowptr[i + 1] < a) bad = 1;
  }
  if (i < E) {
    const int32_t s = senders[i];
    if (s < 0 || s >= N) bad = 1;
  }
  if (bad) atomicOr(flag, 1);
}

__global__ void histogram_kernel(const int32_t* senders, int64_t E, int32_t* count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < E) atomicAdd(&count[senders[i]], 1);
}

// Exclusive scan of n = N+1 counts in place (count[N] = 0 on entry), one block.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* data, int64_t n) {
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  const int64_t per = (n + 1023) / 1024;
  const int64_t b = t * per, e = b + per < n ? b + per : n;
  int32_t s = 0;
  for (int64_t i = b; i < e; ++i) s += data[i];
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int32_t run = t ? part[t - 1] : 0;
  for (int64_t i = b; i < e; ++i) {
    const int32_t c = data[i];
    data[i] = run;
    run += c;
  }
}

__global__ void scatter_kernel(const int32_t* rowptr, const int32_t* senders, int64_t N, int32_t* cursor,
                               int32_t* receivers_out) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= N) return;
  for (int32_t e = rowptr[v]; e < rowptr[v + 1]; ++e) {
    const int32_t at = atomicAdd(&cursor[senders[e]], 1);
    receivers_out[at] = (int32_t)v;
  }
}

// Shell sort of each sender segment (gaps 701, 301, 132, 57, 23, 10, 4, 1).
__global__ void segment_sort_kernel(const int32_t* colptr, int64_t N, int32_t* vals) {
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= N) return;
  int32_t* a = vals + colptr[s];
  const int n = colptr[s + 1] - colptr[s];
  const int gaps[8] = {701, 301, 132, 57, 23, 10, 4, 1};
  for (int gi = 0; gi < 8; ++gi) {
    const int g = gaps[gi];
    for (int i = g; i < n; ++i) {
      const int32_t x = a[i];
      int j = i;
      while (j >= g && a[j - g] > x) {
        a[j] = a[j - g];
        j -= g;
      }
      a[j] = x;
    }
  }
}

inline unsigned blocks(int64_t n, int b) { return (unsigned)((n + b - 1) / b); }

// Bounding box of the node positions (one block): box = {min x, y, z, max x, y, z}.
__global__ __launch_bounds__(1024) void bbox_kernel(const float* pos, int64_t N, float* box) {
  __shared__ float part[6][1024];
  const int t = threadIdx.x;
  float lo[3] = {INFINITY, INFINITY, INFINITY}, hi[3] = {-INFINITY, -INFINITY, -INFINITY};
  for (int64_t i = t; i < N; i += 1024)
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      const float v = pos[3 * i + c];
      lo[c] = fminf(lo[c], v);
      hi[c] = fmaxf(hi[c], v);
    }
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    part[c][t] = lo[c];
    part[3 + c][t] = hi[c];
  }
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (t < off)
#pragma unroll
      for (int c = 0; c < 3; ++c) {
        part[c][t] = fminf(part[c][t], part[c][t + off]);
        part[3 + c][t] = fmaxf(part[3 + c][t], part[3 + c][t + off]);
      }
    __syncthreads();
  }
  if (t < 6) box[t] = part[t][0];
}

// Ten bits spread to every third position.
__device__ __forceinline__ uint32_t spread3(uint32_t v) {
  v &= 0x3ffu;
  v = (v | (v << 16)) & 0x030000ffu;
  v = (v | (v << 8)) & 0x0300f00fu;
  v = (v | (v << 4)) & 0x030c30c3u;
  v = (v | (v << 2)) & 0x09249249u;
  return v;
}

// key = (30-bit Morton code of the position in the box's cube) << 32 | node;
// keys past N sort last.  Every key is unique, so the sorted order is too.
__global__ void morton_keys_kernel(const float* pos, int64_t N, int64_t M, const float* box, uint64_t* keys) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M) return;
  if (i >= N) {
    keys[i] = ~0ull;
    return;
  }
  const float ext = fmaxf(fmaxf(box[3] - box[0], box[4] - box[1]), fmaxf(box[5] - box[2], 1e-30f));
  const float scale = 1024.f / ext;
  uint32_t q[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    const float f = (pos[3 * i + c] - box[c]) * scale;
    q[c] = (uint32_t)fminf(fmaxf(f, 0.f), 1023.f);
  }
  const uint32_t code = spread3(q[0]) | (spread3(q[1]) << 1) | (spread3(q[2]) << 2);
  keys[i] = ((uint64_t)code << 32) | (uint64_t)(uint32_t)i;
}

// One compare-exchange stage (k, j) of a bitonic sort of M = 2^n keys, ascending.
__global__ void bitonic_stage_kernel(uint64_t* keys, int64_t M, int64_t k, int64_t j) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= M) return;
  const int64_t p = i ^ j;
  if (p <= i) return;
  const uint64_t a = keys[i], b = keys[p];
  const bool ascending = (i & k) == 0;
  if ((a > b) == ascending) {
    keys[i] = b;
    keys[p] = a;
  }
}

__global__ void order_from_keys_kernel(const uint64_t* keys, int64_t N, int32_t* order) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < N) order[i] = (int32_t)(uint32_t)(keys[i] & 0xffffffffu);
}

int64_t pow2_at_least(int64_t n) {
  int64_t m = 1;
  while (m < n) m <<= 1;
  return m;
}

}  // namespace

size_t graph_order_workspace(int64_t N) { return (size_t)(8 * pow2_at_least(N > 0 ? N : 1) + 256); }

hipError_t graph_order(const float* pos, int64_t N, int32_t* order, void* ws, size_t ws_bytes, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  if (ws_bytes < graph_order_workspace(N)) return hipErrorInvalidValue;
  TimingScope ts(kcGraph, s);
  const int64_t M = pow2_at_least(N);
  uint64_t* keys = static_cast<uint64_t*>(ws);
  float* box = reinterpret_cast<float*>(static_cast<char*>(ws) + 8 * M);
  hipLaunchKernelGGL(bbox_kernel, dim3(1), dim3(1024), 0, s, pos, N, box);
  hipLaunchKernelGGL(morton_keys_kernel, dim3(blocks(M, 256)), dim3(256), 0, s, pos, N, M, box, keys);
  for (int64_t k = 2; k <= M; k <<= 1)
    for (int64_t j = k >> 1; j > 0; j >>= 1)
      hipLaunchKernelGGL(bitonic_stage_kernel, dim3(blocks(M, 256)), dim3(256), 0, s, keys, M, k, j);
  hipLaunchKernelGGL(order_from_keys_kernel, dim3(blocks(N, 256)), dim3(256), 0, s, keys, N, order);
  return hipGetLastError();
}

size_t graph_csc_workspace(int64_t N, int64_t E) {
  (void)E;
  return (size_t)((N + 1) * sizeof(int32_t) + 255) / 256 * 256;
}

hipError_t launch_graph_validate(const int32_t* rowptr, const int32_t* senders, int64_t N, int64_t E,
                                 int32_t* flag, hipStream_t s) {
  hipLaunchKernelGGL(fill_i32, dim3(1), dim3(64), 0, s, flag, (int64_t)1, 0);
  const int64_t n = (N + 1 > E ? N + 1 : E);
  hipLaunchKernelGGL(validate_kernel, dim3(blocks(n, 256)), dim3(256), 0, s, rowptr, senders, N, E, flag);
  return hipGetLastError();
}

hipError_t graph_csc(const int32_t* rowptr, const int32_t* senders, int64_t N, int64_t E, int32_t* colptr,
                     int32_t* receivers_out, void* ws, size_t ws_bytes, hipStream_t s) {
  if (ws_bytes < graph_csc_workspace(N, E)) return hipErrorInvalidValue;
  TimingScope ts(kcGraph, s);
  int32_t* cursor = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(fill_i32, dim3(blocks(N + 1, 256)), dim3(256), 0, s, colptr, N + 1, 0);
  if (E > 0) hipLaunchKernelGGL(histogram_kernel, dim3(blocks(E, 256)), dim3(256), 0, s, senders, E, colptr);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, colptr, N + 1);
  if (E > 0 && N > 0) {
    hipMemcpyAsync(cursor, colptr, (size_t)(N + 1) * sizeof(int32_t), hipMemcpyDeviceToDevice, s);
    hipLaunchKernelGGL(scatter_kernel, dim3(blocks(N, 128)), dim3(128), 0, s, rowptr, senders, N, cursor,
                       receivers_out);
    hipLaunchKernelGGL(segment_sort_kernel, dim3(blocks(N, 128)), dim3(128), 0, s, colptr, N, receivers_out);
  }
  return hipGetLastError();
}

}  // namespace tpconv
