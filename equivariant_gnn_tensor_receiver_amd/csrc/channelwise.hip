// Contractions of the channel-wise ("uvu") connection, W[k, p, c].
//
// With one weight per (radial function, path, channel) the dense products of
// the fully connected operator become diagonal in the channel (Sobek page,
// abstract: the second operator family; the reassociated state S is the same):
//   out[v][l3, c, m3] = sum_{p -> l3} sum_k W[k, p, c] S_v[k, p, c, m3]
//   g_x[s][l1, c, m1] = sum_{p <- l1} sum_k W[k, p, c] T_s[k, p, c, m1]
//   gW[k, p, c]       = sum_{v, m3} S_v[k, p, c, m3] g_out[v][l3, c, m3]
// Each state element is read once and used once, so these are streaming
// kernels bound by HBM bandwidth: lanes run along the channel, which is the
// contiguous index of the state rows, the feature rows and W.  The weight
// gradient is split over row ranges into partials that a second kernel sums
// in a fixed order, so every result is deterministic.
#include "device_common.h"
#include "kernels.h"
#include "timing.h"

namespace tpconv {

namespace {

__device__ __forceinline__ float w_at(const void* W, int64_t i, bool bf16) {
  return bf16 ? load_feat(static_cast<const uint16_t*>(W), i) : static_cast<const float*>(W)[i];
}

// Sum over the 64 lanes of a wave (fixed order: butterfly over DPP quads and
// mirrors, then the permlane row and half swaps).
template <int CTRL>
__device__ __forceinline__ float dpp_sum_step(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_sum_step<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_sum_step<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_sum_step<0x141>(v);  // row_half_mirror
  v = dpp_sum_step<0x140>(v);  // row_mirror
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int find_group(const CwArgs& a, int64_t i) {
  int gi = 0;
  while (gi + 1 < a.ngroups && i >= a.g[gi + 1].first) ++gi;
  return gi;
}

// One thread per destination element (node, m, c) of every group; K and the
// weight type are compile-time so that all K * npg state loads of a thread
// are issued before the first multiply.
template <int K, bool WBF16>
__global__ __launch_bounds__(256) void cw_contract_kernel(const CwArgs /*args*/) {
  const CwArgs& a = *(const CwArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.total) return;
  const CwGroup& G = a.g[find_group(a, i)];
  const int64_t li = i - G.first;
  const int c = (int)(li % a.C);
  const int64_t row = li / a.C;  // node * n + m
  const int64_t node = row / G.n;
  const int m = (int)(row - node * G.n);
  const int cpk = G.npg * a.C;
  const float* srow = a.state + G.state_off + row * ((int64_t)K * cpk) + c;
  float acc = 0.f;
  for (int q = 0; q < G.npg; ++q) {
    const int64_t wp = (int64_t)a.path_list[G.plist + q] * a.C + c;
    float sv[K], wv[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      sv[k] = srow[(int64_t)k * cpk + q * a.C];
      wv[k] = w_at(a.W, (int64_t)k * a.P * a.C + wp, WBF16);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) acc = __builtin_fmaf(wv[k], sv[k], acc);
  }
  a.dst[(node * a.D_feat + G.row_off + m) * a.C + c] = acc;
}

// One thread per (group element (k, q, c), split): a run of rows (v, m),
// eight rows in flight at a time.
__global__ __launch_bounds__(256) void cw_gw_kernel(const CwArgs /*args*/) {
  const CwArgs& a = *(const CwArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= a.elems) return;
  int gi = 0;
  while (gi + 1 < a.ngroups && e >= a.g[gi + 1].elem_off) ++gi;
  const CwGroup& G = a.g[gi];
  const int64_t le = e - G.elem_off;  // (k * npg + q) * C + c
  const int c = (int)(le % a.C);
  const int64_t kq = le / a.C;
  const int k = (int)(kq / G.npg), q = (int)(kq - (int64_t)k * G.npg);
  const int cpk = G.npg * a.C;
  const int64_t rows = a.N * G.n;
  const int64_t per = (rows + a.splits - 1) / a.splits;
  const int64_t r0 = min(rows, (int64_t)blockIdx.y * per), r1 = min(rows, r0 + per);
  const int64_t stride = (int64_t)a.K * cpk;
  const float* sp = a.state + G.state_off + (int64_t)k * cpk + q * a.C + c + r0 * stride;
  const float* gp = a.gout + (int64_t)G.row_off * a.C + c;
  // row r = (node, mm) of the group, stepped without division
  int64_t node = r0 / G.n;
  int mm = (int)(r0 - node * G.n);
  auto g_at = [&]() { return gp[(node * a.D_feat + mm) * a.C]; };
  auto advance = [&]() {
    const int m2 = mm + 1;
    const bool wrap = m2 == G.n;
    mm = wrap ? 0 : m2;
    node += wrap ? 1 : 0;
  };
  float acc = 0.f;
  constexpr int U = 8;
  int64_t r = r0;
  for (; r + U <= r1; r += U) {
    float sv[U], gv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      sv[u] = sp[u * stride];
      gv[u] = g_at();
      advance();
    }
    sp += U * stride;
#pragma unroll
    for (int u = 0; u < U; ++u) acc = __builtin_fmaf(sv[u], gv[u], acc);
  }
  for (; r < r1; ++r) {
    acc = __builtin_fmaf(*sp, g_at(), acc);
    sp += stride;
    advance();
  }
  a.dst[(int64_t)blockIdx.y * a.elems + e] = acc;
}

// One wave per element: lanes take splits lane, lane + 64, ... and the wave
// sums them with a fixed DPP / permlane tree, so the order never changes.
__global__ __launch_bounds__(256) void cw_reduce_kernel(const CwArgs /*args*/) {
  const CwArgs& a = *(const CwArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const int64_t e = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (e >= a.elems) return;  // uniform over the wave
  const int lane = threadIdx.x & 63;
  float s = 0.f;
  for (int sp = lane; sp < a.splits; sp += 64) s += a.part[(int64_t)sp * a.elems + e];
  s = wave_sum(s);
  if (lane != 0) return;
  int gi = 0;
  while (gi + 1 < a.ngroups && e >= a.g[gi + 1].elem_off) ++gi;
  const CwGroup& G = a.g[gi];
  const int64_t le = e - G.elem_off;
  const int c = (int)(le % a.C);
  const int64_t kq = le / a.C;
  const int k = (int)(kq / G.npg), q = (int)(kq - (int64_t)k * G.npg);
  a.dst[((int64_t)k * a.P + a.path_list[G.plist + q]) * a.C + c] = s;
}

dim3 grid_for(int64_t n) { return dim3((unsigned)((n + 255) / 256)); }

}  // namespace

hipError_t launch_cw_contract(const CwArgs& a, hipStream_t s) {
  if (a.total <= 0) return hipSuccess;
  TimingScope ts(kcCwContract, s);
  const dim3 g = grid_for(a.total), b(256);
  if (a.K == 8 && a.w_bf16)
    hipLaunchKernelGGL((cw_contract_kernel<8, true>), g, b, 0, s, a);
  else if (a.K == 8)
    hipLaunchKernelGGL((cw_contract_kernel<8, false>), g, b, 0, s, a);
  else if (a.K == 16 && a.w_bf16)
    hipLaunchKernelGGL((cw_contract_kernel<16, true>), g, b, 0, s, a);
  else if (a.K == 16)
    hipLaunchKernelGGL((cw_contract_kernel<16, false>), g, b, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_cw_gw(const CwArgs& a, hipStream_t s) {
  if (a.elems <= 0) return hipSuccess;
  TimingScope ts(kcCwGw, s);
  dim3 g = grid_for(a.elems);
  g.y = (unsigned)a.splits;
  hipLaunchKernelGGL(cw_gw_kernel, g, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_cw_reduce(const CwArgs& a, hipStream_t s) {
  if (a.elems <= 0) return hipSuccess;
  TimingScope ts(kcCwReduce, s);
  hipLaunchKernelGGL(cw_reduce_kernel, dim3((unsigned)((a.elems + 3) / 4)), dim3(256), 0, s, a);  // 4 waves/block
  return hipGetLastError();
}

}  // namespace tpconv
