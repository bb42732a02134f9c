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
// One kernel template covers the four kinds through accessor functions.  A
// block of 2 waves computes a 64 x BN tile; each wave owns 32 rows and BN/32
// v_mfma_f32_32x32x2f32 accumulators (fp32 in, fp32 accumulate).  Tiles of 16
// reduction steps are double-buffered in LDS (k-major, so each MFMA operand
// read is 32 consecutive floats) and the next tile's global loads are issued
// before the current tile is multiplied.  Global loads are float4 along each
// operand's contiguous dimension when channel counts are multiples of 16.
#include "device_common.h"
#include "kernels.h"
#include "timing.h"

namespace tpconv {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int BK = 16;
constexpr int BM = 64;
constexpr int kThreads = 128;

template <bool WBF16>
__device__ __forceinline__ float load_w(const void* W, int64_t i) {
  if constexpr (WBF16)
    return load_feat(static_cast<const uint16_t*>(W), i);
  else
    return static_cast<const float*>(W)[i];
}

template <bool WBF16>
__device__ __forceinline__ floatx4 load_w4(const void* W, int64_t i) {
  if constexpr (WBF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(W) + i);
    return floatx4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                   __uint_as_float(u.y & 0xffff0000u)};
  } else {
    return *reinterpret_cast<const floatx4*>(static_cast<const float*>(W) + i);
  }
}

// Contiguous dimension of each operand: A along k (reduction) or m; B along n or k.
template <int KIND> struct KindTraits;
template <> struct KindTraits<kGemmOut> { static constexpr bool a_k = true, b_n = true; };
template <> struct KindTraits<kGemmGs> { static constexpr bool a_k = true, b_n = false; };
template <> struct KindTraits<kGemmGx> { static constexpr bool a_k = true, b_n = false; };
template <> struct KindTraits<kGemmGw> { static constexpr bool a_k = false, b_n = true; };

// Element offset of A(m, r) and B(r, n) in their tensors.
template <int KIND>
__device__ __forceinline__ int64_t a_index(const GemmArgs& a, const GemmGroup& G, int m, int r) {
  if constexpr (KIND == kGemmOut || KIND == kGemmGx) {
    return G.state_off + (int64_t)m * G.Kr + r;
  } else if constexpr (KIND == kGemmGs) {
    const int v = m / G.n, mm = m - v * G.n;
    return ((int64_t)v * a.D_feat + G.row_off + mm) * a.C_out + r;
  } else {  // Gw: A(j, r) = S_g[r][j]
    return G.state_off + (int64_t)r * G.M + m;
  }
}

template <int KIND>
__device__ __forceinline__ int64_t b_index(const GemmArgs& a, const GemmGroup& G, int r, int n) {
  if constexpr (KIND == kGemmOut) {  // W[(k,q,ci) = r][co = n]
    const int cpk = G.npg * a.C_in;
    const int k = r / cpk, rem = r - k * cpk, q = rem / a.C_in, ci = rem - q * a.C_in;
    return (((int64_t)k * a.P + a.path_list[G.plist + q]) * a.C_in + ci) * a.C_out + n;
  } else if constexpr (KIND == kGemmGs) {  // W[(k,q,ci) = n][co = r]
    const int cpk = G.npg * a.C_in;
    const int k = n / cpk, rem = n - k * cpk, q = rem / a.C_in, ci = rem - q * a.C_in;
    return (((int64_t)k * a.P + a.path_list[G.plist + q]) * a.C_in + ci) * a.C_out + r;
  } else if constexpr (KIND == kGemmGx) {  // W[(k,q,co) = r][ci = n]
    const int cpk = G.npg * a.C_out;
    const int k = r / cpk, rem = r - k * cpk, q = rem / a.C_out, co = rem - q * a.C_out;
    return (((int64_t)k * a.P + a.path_list[G.plist + q]) * a.C_in + n) * a.C_out + co;
  } else {  // Gw: g_out[(v, m3) = r][co = n]
    const int v = r / G.n, mm = r - v * G.n;
    return ((int64_t)v * a.D_feat + G.row_off + mm) * a.C_out + n;
  }
}

template <int KIND, bool WBF16>
__device__ __forceinline__ float load_a1(const GemmArgs& a, const GemmGroup& G, int m, int r) {
  const int64_t i = a_index<KIND>(a, G, m, r);
  return (KIND == kGemmGs) ? a.feat[i] : a.state[i];
}

template <int KIND, bool WBF16>
__device__ __forceinline__ float load_b1(const GemmArgs& a, const GemmGroup& G, int r, int n) {
  const int64_t i = b_index<KIND>(a, G, r, n);
  if constexpr (KIND == kGemmGw) return a.feat[i];
  return load_w<WBF16>(a.W, i);
}

template <int KIND, bool WBF16>
__device__ __forceinline__ floatx4 load_a4(const GemmArgs& a, const GemmGroup& G, int m, int r) {
  const int64_t i = a_index<KIND>(a, G, m, r);
  return *reinterpret_cast<const floatx4*>(((KIND == kGemmGs) ? a.feat : a.state) + i);
}

template <int KIND, bool WBF16>
__device__ __forceinline__ floatx4 load_b4(const GemmArgs& a, const GemmGroup& G, int r, int n) {
  const int64_t i = b_index<KIND>(a, G, r, n);
  if constexpr (KIND == kGemmGw) return *reinterpret_cast<const floatx4*>(a.feat + i);
  return load_w4<WBF16>(a.W, i);
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

// Register staging of one BM x BK (A) and BK x BN (B) tile.
template <int BN>
struct Stage {
  static constexpr int NA = BM * BK / 4 / kThreads;  // float4 per thread
  static constexpr int NB = (BN * BK / 4 + kThreads - 1) / kThreads;
  floatx4 a[NA];
  floatx4 b[NB];
};

template <int KIND, int BN, bool WBF16>
__device__ __forceinline__ void load_tile(const GemmArgs& a, const GemmGroup& G, int m0, int n0, int k0, int r_end,
                                          bool vec, Stage<BN>& st) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Stage<BN>::NA; ++i) {
    const int idx = t + i * kThreads;  // float4 index in the tile
    int m, k;
    if constexpr (KindTraits<KIND>::a_k) {
      m = idx / (BK / 4);
      k = (idx % (BK / 4)) * 4;
    } else {
      k = idx / (BM / 4);
      m = (idx % (BM / 4)) * 4;
    }
    const int gm = m0 + m, gk = k0 + k;
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KindTraits<KIND>::a_k) {
      if (vec && gm < G.M && gk + 3 < r_end) {
        v = load_a4<KIND, WBF16>(a, G, gm, gk);
      } else if (gm < G.M) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (gk + e < r_end) v[e] = load_a1<KIND, WBF16>(a, G, gm, gk + e);
      }
    } else {
      if (vec && gm + 3 < G.M && gk < r_end) {
        v = load_a4<KIND, WBF16>(a, G, gm, gk);
      } else if (gk < r_end) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (gm + e < G.M) v[e] = load_a1<KIND, WBF16>(a, G, gm + e, gk);
      }
    }
    st.a[i] = v;
  }
#pragma unroll
  for (int i = 0; i < Stage<BN>::NB; ++i) {
    const int idx = t + i * kThreads;
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (idx < BN * BK / 4) {
      int n, k;
      if constexpr (KindTraits<KIND>::b_n) {
        k = idx / (BN / 4);
        n = (idx % (BN / 4)) * 4;
      } else {
        n = idx / (BK / 4);
        k = (idx % (BK / 4)) * 4;
      }
      const int gn = n0 + n, gk = k0 + k;
      if constexpr (KindTraits<KIND>::b_n) {
        if (vec && gn + 3 < G.N && gk < r_end) {
          v = load_b4<KIND, WBF16>(a, G, gk, gn);
        } else if (gk < r_end) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (gn + e < G.N) v[e] = load_b1<KIND, WBF16>(a, G, gk, gn + e);
        }
      } else {
        if (vec && gn < G.N && gk + 3 < r_end) {
          v = load_b4<KIND, WBF16>(a, G, gk, gn);
        } else if (gn < G.N) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (gk + e < r_end) v[e] = load_b1<KIND, WBF16>(a, G, gk + e, gn);
        }
      }
    }
    st.b[i] = v;
  }
}

template <int KIND, int BN>
__device__ __forceinline__ void store_tile(const Stage<BN>& st, float (*As)[BM + 4], float (*Bs)[BN + 4]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Stage<BN>::NA; ++i) {
    const int idx = t + i * kThreads;
    if constexpr (KindTraits<KIND>::a_k) {
      const int m = idx / (BK / 4), k = (idx % (BK / 4)) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) As[k + e][m] = st.a[i][e];
    } else {
      const int k = idx / (BM / 4), m = (idx % (BM / 4)) * 4;
      *reinterpret_cast<floatx4*>(&As[k][m]) = st.a[i];
    }
  }
#pragma unroll
  for (int i = 0; i < Stage<BN>::NB; ++i) {
    const int idx = t + i * kThreads;
    if (idx >= BN * BK / 4) continue;
    if constexpr (KindTraits<KIND>::b_n) {
      const int k = idx / (BN / 4), n = (idx % (BN / 4)) * 4;
      *reinterpret_cast<floatx4*>(&Bs[k][n]) = st.b[i];
    } else {
      const int n = idx / (BK / 4), k = (idx % (BK / 4)) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) Bs[k + e][n] = st.b[i][e];
    }
  }
}

template <int KIND, int BN, bool WBF16>
__global__ __launch_bounds__(kThreads) void gemm_kernel(const GemmArgs a) {
  constexpr int NT = BN / 32;  // 32x32 accumulators per wave
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
  __shared__ __attribute__((aligned(16))) float As[2][BK][BM + 4];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK][BN + 4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const bool vec = a.vec != 0;
  floatx16 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  const int nk = r_end > r_begin ? (r_end - r_begin + BK - 1) / BK : 0;
  Stage<BN> st;
  if (nk > 0) {
    load_tile<KIND, BN, WBF16>(a, G, m0, n0, r_begin, r_end, vec, st);
    store_tile<KIND, BN>(st, As[0], Bs[0]);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) load_tile<KIND, BN, WBF16>(a, G, m0, n0, r_begin + (kt + 1) * BK, r_end, vec, st);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 2) {
      const float av = As[buf][kk + (lane >> 5)][w * 32 + (lane & 31)];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float bv = Bs[buf][kk + (lane >> 5)][j * 32 + (lane & 31)];
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc[j], 0, 0, 0);
      }
    }
    if (more) store_tile<KIND, BN>(st, As[buf ^ 1], Bs[buf ^ 1]);
    __syncthreads();
  }
  // D layout of 32x32x2: register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int gm = m0 + w * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const int gn = n0 + j * 32 + (lane & 31);
      if (gm < G.M && gn < G.N) store_c<KIND>(a, G, gm, gn, acc[j][r]);
    }
}

__global__ void gw_reduce_kernel(const ReduceArgs a, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
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
  if (bn == 128)
    hipLaunchKernelGGL((gemm_kernel<KIND, 128, WBF16>), grid, dim3(kThreads), 0, s, a);
  else if (bn == 64)
    hipLaunchKernelGGL((gemm_kernel<KIND, 64, WBF16>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_kernel<KIND, 32, WBF16>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int gemm_bm() { return BM; }

int gemm_bn(int kind, const GemmArgs& a) {
  int ncols = 0;
  for (int g = 0; g < a.ngroups; ++g) ncols = a.g[g].N > ncols ? a.g[g].N : ncols;
  (void)kind;
  return ncols > 64 ? 128 : (ncols > 32 ? 64 : 32);
}

hipError_t launch_gemm(int kind, const GemmArgs& a, int max_tiles, hipStream_t s) {
  if (max_tiles <= 0 || a.ngroups <= 0) return hipSuccess;
  const int bn = gemm_bn(kind, a);
  const bool wb = a.w_bf16 != 0;
  TimingScope ts(kcGemmOut + kind, s);
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
  TimingScope ts(kcGwReduce, s);
  hipLaunchKernelGGL(gw_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a, total);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TimingScope ts(kcFill, s);
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace tpconv
