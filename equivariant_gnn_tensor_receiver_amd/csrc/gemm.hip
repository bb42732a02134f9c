// Dense contractions with the shared weights W on the fp32 matrix cores.
//
// After the edge stream, the remaining work of every pass is one dense
// contraction per irrep group ("Sobek" page, abstract: the formulation keeps
// fully connected multiplicity mixing; here W[k,p,ci,co] is applied once per
// node instead of once per edge):
//   out  = S_g . W        rows (v, m3), reduction (k, q, ci), columns co
//   gS_g = g_out . W^T    rows (v, m3), reduction co, columns (k, q, ci)
//   g_x  = T_g . W^T      rows (s, m1), reduction (k, q, co), columns ci
//   gW   = S_g^T . g_out  rows (k, q, ci), reduction (v, m3), columns co (split, then summed in order)
// One kernel covers the four kinds through accessor functions; tiles are
// staged through LDS and multiplied with v_mfma_f32_16x16x4f32 (fp32 in,
// fp32 accumulate).  Each block computes a BM x BN tile with 4 waves of
// 32 x 32 (2 x 2 MFMA tiles each).
#include "kernels.h"
#include "device_common.h"

namespace tpconv {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int BK = 16;

template <bool WBF16>
__device__ __forceinline__ float load_w(const void* W, int64_t i) {
  if constexpr (WBF16)
    return load_feat(static_cast<const uint16_t*>(W), i);
  else
    return static_cast<const float*>(W)[i];
}

// Which operand dimension is contiguous in memory (drives the tile loader).
template <int KIND> struct KindTraits;
template <> struct KindTraits<kGemmOut> { static constexpr bool a_k = true, b_n = true; };
template <> struct KindTraits<kGemmGs> { static constexpr bool a_k = true, b_n = false; };
template <> struct KindTraits<kGemmGx> { static constexpr bool a_k = true, b_n = false; };
template <> struct KindTraits<kGemmGw> { static constexpr bool a_k = false, b_n = true; };

template <int KIND, bool WBF16>
__device__ __forceinline__ float load_a(const GemmArgs& a, const GemmGroup& G, int m, int r) {
  if constexpr (KIND == kGemmOut || KIND == kGemmGx) {
    return a.state[G.state_off + (int64_t)m * G.Kr + r];
  } else if constexpr (KIND == kGemmGs) {
    const int v = m / G.n, mm = m - v * G.n;
    return a.feat[((int64_t)v * a.D_feat + G.row_off + mm) * a.C_out + r];
  } else {  // Gw: A(j, r) = S_g[r][j]
    return a.state[G.state_off + (int64_t)r * G.M + m];
  }
}

template <int KIND, bool WBF16>
__device__ __forceinline__ float load_b(const GemmArgs& a, const GemmGroup& G, int r, int n) {
  if constexpr (KIND == kGemmOut) {  // W[(k,q,ci) = r][co = n]
    const int cpk = G.npg * a.C_in;
    const int k = r / cpk, rem = r - k * cpk, q = rem / a.C_in, ci = rem - q * a.C_in;
    const int path = a.path_list[G.plist + q];
    return load_w<WBF16>(a.W, (((int64_t)k * a.P + path) * a.C_in + ci) * a.C_out + n);
  } else if constexpr (KIND == kGemmGs) {  // W[(k,q,ci) = n][co = r]
    const int cpk = G.npg * a.C_in;
    const int k = n / cpk, rem = n - k * cpk, q = rem / a.C_in, ci = rem - q * a.C_in;
    const int path = a.path_list[G.plist + q];
    return load_w<WBF16>(a.W, (((int64_t)k * a.P + path) * a.C_in + ci) * a.C_out + r);
  } else if constexpr (KIND == kGemmGx) {  // W[(k,q,co) = r][ci = n]
    const int cpk = G.npg * a.C_out;
    const int k = r / cpk, rem = r - k * cpk, q = rem / a.C_out, co = rem - q * a.C_out;
    const int path = a.path_list[G.plist + q];
    return load_w<WBF16>(a.W, (((int64_t)k * a.P + path) * a.C_in + n) * a.C_out + co);
  } else {  // Gw: g_out[(v, m3) = r][co = n]
    const int v = r / G.n, mm = r - v * G.n;
    return a.feat[((int64_t)v * a.D_feat + G.row_off + mm) * a.C_out + n];
  }
}

template <int KIND>
__device__ __forceinline__ void store_c(const GemmArgs& a, const GemmGroup& G, int m, int n, float v) {
  if constexpr (KIND == kGemmOut) {
    const int node = m / G.n, mm = m - node * G.n;
    a.out[((int64_t)node * a.D_feat + G.row_off + mm) * a.C_out + n] = v;
  } else if constexpr (KIND == kGemmGs) {
    a.out[G.state_off + (int64_t)m * G.N + n] = v;
  } else if constexpr (KIND == kGemmGx) {
    const int node = m / G.n, mm = m - node * G.n;
    a.out[((int64_t)node * a.D_feat + G.row_off + mm) * a.C_in + n] = v;
  } else {
    a.out[G.part_off + ((int64_t)blockIdx.y * G.M + m) * G.N + n] = v;
  }
}

template <int KIND, int BM, int BN, bool WBF16>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs a) {
  constexpr int WN = BN / 32;
  static_assert((BM / 32) * WN == 4, "4 waves of 32x32");
  const int gi = blockIdx.z;
  if (gi >= a.ngroups) return;
  const GemmGroup& G = a.g[gi];
  const int tile = blockIdx.x;
  if (tile >= G.tiles) return;
  const int tm = tile / G.tiles_n, tn = tile - tm * G.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  int r_begin = 0, r_end = G.Kr;
  if constexpr (KIND == kGemmGw) {
    const int per = ((G.Kr + a.splits - 1) / a.splits + BK - 1) / BK * BK;
    r_begin = blockIdx.y * per;
    r_end = min(G.Kr, r_begin + per);
  } else {
    if (blockIdx.y != 0) return;
  }
  __shared__ float As[BK][BM + 1];
  __shared__ float Bs[BK][BN + 1];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w / WN, wn = w - wm * WN;
  floatx4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = r_begin; k0 < r_end; k0 += BK) {
#pragma unroll 4
    for (int idx = t; idx < BM * BK; idx += 256) {
      int m, k;
      if constexpr (KindTraits<KIND>::a_k) {
        m = idx / BK;
        k = idx - m * BK;
      } else {
        k = idx / BM;
        m = idx - k * BM;
      }
      const int gm = m0 + m, gk = k0 + k;
      As[k][m] = (gm < G.M && gk < r_end) ? load_a<KIND, WBF16>(a, G, gm, gk) : 0.f;
    }
#pragma unroll 4
    for (int idx = t; idx < BN * BK; idx += 256) {
      int n, k;
      if constexpr (KindTraits<KIND>::b_n) {
        k = idx / BN;
        n = idx - k * BN;
      } else {
        n = idx / BK;
        k = idx - n * BK;
      }
      const int gn = n0 + n, gk = k0 + k;
      Bs[k][n] = (gn < G.N && gk < r_end) ? load_b<KIND, WBF16>(a, G, gk, gn) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 4) {
      float av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) av[i] = As[kk + (lane >> 4)][wm * 32 + i * 16 + (lane & 15)];
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[j] = Bs[kk + (lane >> 4)][wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gm = m0 + wm * 32 + i * 16 + 4 * (lane >> 4) + r;
        const int gn = n0 + wn * 32 + j * 16 + (lane & 15);
        if (gm < G.M && gn < G.N) store_c<KIND>(a, G, gm, gn, acc[i][j][r]);
      }
}

__global__ void gw_reduce_kernel(const ReduceArgs a, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  // locate group
  int64_t rem = i;
  int gi = 0;
  for (; gi < a.ngroups; ++gi) {
    const int64_t sz = (int64_t)a.g[gi].M * a.g[gi].N;
    if (rem < sz) break;
    rem -= sz;
  }
  if (gi >= a.ngroups) return;
  const GemmGroup& G = a.g[gi];
  const int j = (int)(rem / G.N), co = (int)(rem - (int64_t)j * G.N);
  float s = 0.f;
  for (int sp = 0; sp < a.splits; ++sp) s += a.part[G.part_off + ((int64_t)sp * G.M + j) * G.N + co];
  const int cpk = G.npg * a.C_in;
  const int k = j / cpk, r2 = j - k * cpk, q = r2 / a.C_in, ci = r2 - q * a.C_in;
  const int path = a.path_list[G.plist + q];
  a.gw[(((int64_t)k * a.P + path) * a.C_in + ci) * a.C_out + co] = s;
}

__global__ void fill_kernel(float* p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

template <int KIND, bool WBF16>
hipError_t launch_kind(const GemmArgs& a, int max_tiles, int bn, hipStream_t s) {
  const dim3 grid((unsigned)max_tiles, (unsigned)(KIND == kGemmGw ? a.splits : 1), (unsigned)a.ngroups);
  if (bn == 64)
    hipLaunchKernelGGL((gemm_kernel<KIND, 64, 64, WBF16>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel<KIND, 128, 32, WBF16>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// Column tile width used by the host when it sizes the tile grid.
int gemm_bn(int kind, const GemmArgs& a) {
  int ncols = 0;
  for (int g = 0; g < a.ngroups; ++g) ncols = a.g[g].N > ncols ? a.g[g].N : ncols;
  (void)kind;
  return ncols >= 64 ? 64 : 32;
}

hipError_t launch_gemm(int kind, const GemmArgs& a, int max_tiles, hipStream_t s) {
  if (max_tiles <= 0 || a.ngroups <= 0) return hipSuccess;
  const int bn = gemm_bn(kind, a);
  const bool wb = a.w_bf16 != 0;
  switch (kind) {
    case kGemmOut: return wb ? launch_kind<kGemmOut, true>(a, max_tiles, bn, s) : launch_kind<kGemmOut, false>(a, max_tiles, bn, s);
    case kGemmGs: return wb ? launch_kind<kGemmGs, true>(a, max_tiles, bn, s) : launch_kind<kGemmGs, false>(a, max_tiles, bn, s);
    case kGemmGx: return wb ? launch_kind<kGemmGx, true>(a, max_tiles, bn, s) : launch_kind<kGemmGx, false>(a, max_tiles, bn, s);
    case kGemmGw: return launch_kind<kGemmGw, false>(a, max_tiles, bn, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gw_reduce(const ReduceArgs& a, int64_t total, hipStream_t s) {
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(gw_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a, total);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace tpconv
