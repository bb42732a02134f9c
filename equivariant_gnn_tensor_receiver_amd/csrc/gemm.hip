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
//
// These products are skinny (32..128 columns) and stream a node-sized
// operand once, so the kernel is built for bytes in flight rather than for
// LDS reuse.  Every wave owns a (32*MT)-row x (32*NT)-column tile and loads its
// operands straight into registers: for v_mfma_f32_32x32x2f32 lane (i, h)
// (i = lane % 32, h = lane / 32) supplies A[i][kk = h] and B[kk = h][i], and
// the reduction order inside a chunk of 2*VH indices is permuted so that lane
// half h takes the VH consecutive indices r0 + VH*h + t (t = 0..VH-1), step t
// of the chunk summing r0 + t and r0 + VH + t.  An operand that is contiguous
// along the reduction is then read as 16-byte vectors per lane; one that is
// contiguous along its row or column index is read as 128-byte coalesced
// rows.  The next chunk is loaded while the current one is multiplied.  Small
// problems split the reduction over the 1, 2 or 4 waves of a block (interleaved
// chunks, so that the waves read neighbouring segments of a row); the waves'
// partial tiles are summed in a fixed order through LDS, so results do not
// depend on timing.
#include "device_common.h"
#include "kernels.h"
#include "timing.h"

namespace tpconv {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kTargetWaves = 4096;  // 4 waves per SIMD
constexpr int kMaxWaveSplit = 4;

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Raw 32-bit pattern of one weight: the fp32 bits, or the bf16 bits
// zero-extended (widened by a shift where the value is used).
template <bool WBF16>
__device__ __forceinline__ uint32_t raw_w(const void* W, int64_t i) {
  if constexpr (WBF16)
    return static_cast<const uint16_t*>(W)[i];
  else
    return __float_as_uint(static_cast<const float*>(W)[i]);
}


// VH consecutive floats p[0..VH) (16-byte loads when VEC).  Loads are never
// predicated and their values are not touched here: the caller clamps `p`
// into the tensor, and a reduction index past the end is zeroed in A just
// before the multiply (B may then hold any finite value).  A select right
// after a load would make the compiler wait for it, which defeats the
// one-chunk-ahead prefetch.
template <int VH, bool VEC>
__device__ __forceinline__ void load_run(const float* p, int valid, float (&v)[VH]) {
  if constexpr (VEC) {
#pragma unroll
    for (int j = 0; j < VH / 4; ++j) {
      const floatx4 x = *reinterpret_cast<const floatx4*>(p + 4 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * j + e] = x[e];
    }
  } else {
    const int last = valid > 0 ? valid - 1 : 0;
#pragma unroll
    for (int t = 0; t < VH; ++t) v[t] = p[t < last ? t : last];
  }
}

// x / d for 0 <= x < 2^22 and 0 < d < 2^22: the quotient through the fp32
// reciprocal is off by at most one, and the remainder test corrects it (the
// divisors are uniform, so the reciprocal is one scalar-side instruction).
__device__ __forceinline__ int div_small(int x, int d) {
  int q = (int)((float)x * __builtin_amdgcn_rcpf((float)d));
  const int r = x - q * d;
  q += r >= d ? 1 : 0;
  q -= r < 0 ? 1 : 0;
  return q;
}

// (k, q, c) of a reduction/column index k * npg * C + q * C + c of a group.
__device__ __forceinline__ int w_index(const GemmGroup& G, int kqc, int C, int& q, int& c) {
  const int cpk = G.npg * C;
  const int k = div_small(kqc, cpk), rem = kqc - k * cpk;
  q = div_small(rem, C);
  c = rem - q * C;
  return k;
}

// Row k * P + path of W and channel c for a reduction/column index (k, q, c)
// of a group.  `pl` holds, in lane i, the group's i-th path index (read once
// per kernel), so the lookup is a lane shuffle, not a memory load.
__device__ __forceinline__ int64_t w_row(const GemmArgs& a, const GemmGroup& G, int kqc, int C, int pl, int& c) {
  int q;
  const int k = w_index(G, kqc, C, q, c);
  return (int64_t)k * a.P + __shfl(pl, q);
}

// The same for an index that is uniform over each lane half (h = lane / 32,
// as the reduction indices of a chunk are): the path comes from two lane
// reads instead of a shuffle through LDS.
__device__ __forceinline__ int64_t w_row_halves(const GemmArgs& a, const GemmGroup& G, int kqc, int C, int pl,
                                                int h, int& c) {
  int q;
  const int k = w_index(G, kqc, C, q, c);
  const int q0 = __builtin_amdgcn_readfirstlane(q), q1 = __builtin_amdgcn_readlane(q, 32);
  const int p0 = __builtin_amdgcn_readlane(pl, q0), p1 = __builtin_amdgcn_readlane(pl, q1);
  return (int64_t)k * a.P + (h ? p1 : p0);
}

// A operand: values t = 0..VH-1 of row m at reductions rs + t; indices past
// the end of the reduction read inside the tensor (zeroed later).
template <int KIND, int VH, bool VEC>
__device__ __forceinline__ void load_a(const GemmArgs& a, const GemmGroup& G, int m, int rs, int r_end,
                                       float (&v)[VH]) {
  if constexpr (KIND == kGemmOut || KIND == kGemmGx || KIND == kGemmGs) {
    const float* row;
    if constexpr (KIND == kGemmGs) {
      const int node = m / G.n, mm = m - node * G.n;
      row = a.feat + ((int64_t)node * a.D_feat + G.row_off + mm) * a.C_out;
    } else {
      row = a.state + G.state_off + (int64_t)m * G.Kr;
    }
    // VEC: Kr is a multiple of 16 and rs of VH, so a whole run is in or out
    const int rc = VEC ? (rs < r_end ? rs : r_end - VH) : (rs < r_end ? rs : r_end - 1);
    load_run<VH, VEC>(row + (rc > 0 ? rc : 0), r_end - rs, v);
  } else {  // Gw: A(j, r) = S_g[r][j], contiguous along j across the lanes
    const float* p = a.state + G.state_off + m;
#pragma unroll
    for (int t = 0; t < VH; ++t) v[t] = p[(int64_t)min(rs + t, G.Kr - 1) * G.M];
  }
}

// B operand: values t = 0..VH-1 of column n at reductions rs + t, as raw bits
// (see Bits); indices past the end of the reduction read inside the tensor.
template <int KIND, int VH, bool WBF16, bool VEC>
struct Bits {
  // bf16 weights read 4 at a time (gS and g_x with 16-byte channel rows) stay
  // packed two per word; other bf16 weights take one word each
  static constexpr bool PACKED = WBF16 && VEC && (KIND == kGemmGs || KIND == kGemmGx);
  static constexpr int N = PACKED ? VH / 2 : VH;
  __device__ __forceinline__ static float get(const uint32_t (&v)[N], int t) {
    if constexpr (!WBF16)
      return __uint_as_float(v[t]);
    else if constexpr (PACKED)
      return __uint_as_float((t & 1) ? (v[t >> 1] & 0xffff0000u) : (v[t >> 1] << 16));
    else
      return __uint_as_float(v[t] << 16);
  }
};

template <int KIND, int VH, bool WBF16, bool VEC>
__device__ __forceinline__ void load_b(const GemmArgs& a, const GemmGroup& G, int n, int rs, int r_end, int pl,
                                       uint32_t (&v)[Bits<KIND, VH, WBF16, VEC>::N]) {
  if constexpr (KIND == kGemmOut) {  // B(r = (k,q,ci), n = co) = W[k][p][ci][co]
    if constexpr (VEC) {  // the VH reductions share (k, q): C_in is a multiple of 16
      int ci;
      const int64_t kp = w_row_halves(a, G, rs < r_end ? rs : 0, a.C_in, pl, (int)(threadIdx.x & 63) >> 5, ci);
      const int64_t base = (kp * a.C_in + ci) * a.C_out + n;
#pragma unroll
      for (int t = 0; t < VH; ++t) v[t] = raw_w<WBF16>(a.W, base + (int64_t)t * a.C_out);
    } else {
#pragma unroll
      for (int t = 0; t < VH; ++t) {
        int ci;
        const int r = min(rs + t, G.Kr - 1);
        const int64_t kp = w_row(a, G, r, a.C_in, pl, ci);
        v[t] = raw_w<WBF16>(a.W, (kp * a.C_in + ci) * a.C_out + n);
      }
    }
  } else if constexpr (KIND == kGemmGs || KIND == kGemmGx) {
    // gS: B(r = co, n = (k,q,ci)) = W[k][p][ci][co];  g_x: B(r = (k,q,co), n = ci) = W[k][p][ci][co]
    int64_t base;
    if constexpr (KIND == kGemmGs) {
      int ci;
      const int64_t kp = w_row(a, G, n, a.C_in, pl, ci);
      base = (kp * a.C_in + ci) * a.C_out + (VEC ? (rs < r_end ? rs : 0) : 0);
    } else if constexpr (VEC) {  // the VH reductions share (k, q): C_out is a multiple of 16
      int co;
      const int64_t kp = w_row_halves(a, G, rs < r_end ? rs : 0, a.C_out, pl, (int)(threadIdx.x & 63) >> 5, co);
      base = (kp * a.C_in + n) * a.C_out + co;
    } else {
      base = 0;
    }
    if constexpr (VEC) {
#pragma unroll
      for (int j = 0; j < VH / 4; ++j) {
        if constexpr (WBF16) {
          const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.W) + base + 4 * j);
          v[2 * j] = u.x;
          v[2 * j + 1] = u.y;
        } else {
          const floatx4 x = *reinterpret_cast<const floatx4*>(static_cast<const float*>(a.W) + base + 4 * j);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[4 * j + e] = __float_as_uint(x[e]);
        }
      }
    } else if constexpr (KIND == kGemmGs) {
#pragma unroll
      for (int t = 0; t < VH; ++t) v[t] = raw_w<WBF16>(a.W, base + min(rs + t, r_end - 1));
    } else {
#pragma unroll
      for (int t = 0; t < VH; ++t) {
        int co;
        const int r = min(rs + t, G.Kr - 1);
        const int64_t kp = w_row(a, G, r, a.C_out, pl, co);
        v[t] = raw_w<WBF16>(a.W, (kp * a.C_in + n) * a.C_out + co);
      }
    }
  } else {  // Gw: B(r = (v, m3), n = co) = g_out[v][row_off + m3][co]; rows stepped without division
    const int r0 = min(rs, G.Kr - 1);
    int node = r0 / G.n, mm = r0 - node * G.n;
    const float* base = a.feat + (int64_t)G.row_off * a.C_out + n;
#pragma unroll
    for (int t = 0; t < VH; ++t) {
      v[t] = __float_as_uint(base[((int64_t)node * a.D_feat + mm) * a.C_out]);
      // next row; past the end of the reduction the last row is read again
      const bool adv = rs + t + 1 < G.Kr;
      const bool wrap = mm + 1 == G.n;
      const int mm2 = wrap ? 0 : mm + 1, node2 = wrap ? node + 1 : node;
      mm = adv ? mm2 : mm;
      node = adv ? node2 : node;
    }
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

template <int KIND, int MT, int NT, int VH, bool WBF16, bool VEC>
struct Chunk {
  using B = Bits<KIND, VH, WBF16, VEC>;
  float a[MT][VH];
  uint32_t b[NT][B::N];  // raw; widened in mul
  int valid;  // reductions of this lane half inside the range (<= 0: none)
  __device__ __forceinline__ void load(const GemmArgs& ar, const GemmGroup& G, const int (&m)[MT], const int (&n)[NT],
                                       int rs, int r_end, int pl) {
    valid = r_end - rs;
#pragma unroll
    for (int u = 0; u < MT; ++u) load_a<KIND, VH, VEC>(ar, G, m[u], rs, r_end, a[u]);
#pragma unroll
    for (int j = 0; j < NT; ++j) load_b<KIND, VH, WBF16, VEC>(ar, G, n[j], rs, r_end, pl, b[j]);
  }
  __device__ __forceinline__ void mul(floatx16 (&acc)[MT][NT]) const {
#pragma unroll
    for (int t = 0; t < VH; ++t) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const float bv = B::get(b[j], t);
#pragma unroll
        for (int u = 0; u < MT; ++u) {
          const float av = t < valid ? a[u][t] : 0.f;  // past the end of the reduction
          acc[u][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc[u][j], 0, 0, 0);
        }
      }
    }
  }
};

// Waves per SIMD the register allocation must leave room for (accumulators,
// three chunk buffers and addressing fit; left to itself the compiler spreads
// the accumulators over extra registers and halves the occupancy).
constexpr int gemm_min_waves(int mt, int nt, int vh) {
  return 16 * mt * nt + 3 * vh * (mt + nt) <= 112 ? 3 : 2;
}

template <int KIND, int MT, int NT, int VH, bool WBF16, bool VEC>
__global__ __launch_bounds__(64 * kMaxWaveSplit) __attribute__((amdgpu_waves_per_eu(gemm_min_waves(MT, NT, VH))))
void gemm_kernel(const GemmArgs /*args*/) {
  // Read the arguments in place: a by-value copy indexed by a runtime group
  // would be spilled to scratch.
  const GemmArgs& a = *(const GemmArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  extern __shared__ float red[];  // (waves - 1) x MT x NT x 16 x 64 partial tiles
  const int b = blockIdx.x;
  int gi = 0;
  while (gi + 1 < a.ngroups && b >= a.g[gi + 1].tile_begin) ++gi;
  const GemmGroup& G = a.g[gi];
  const int tile = b - G.tile_begin;
  if (tile >= G.tiles) return;  // uniform over the block
  const int tm = tile / G.tiles_n, tn = tile - tm * G.tiles_n;
  const int m0 = tm * 32 * MT, n0 = tn * 32 * NT;
  // wave index and loop bounds in scalar registers: the chunk loop then needs
  // no exec masking and the accumulators stay in place across iterations
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nw = blockDim.x >> 6;
  const int i = lane & 31, h = lane >> 5;
  constexpr int KC = 2 * VH;

  int rb = 0, re = G.Kr;
  if constexpr (KIND == kGemmGw) {
    const int per = ceil_div(ceil_div(G.Kr, a.splits), KC) * KC;
    rb = min(G.Kr, (int)blockIdx.y * per);
    re = min(G.Kr, rb + per);
  }
  // The block's waves take interleaved chunks (wave w: chunks w, w + nw, ..),
  // so that at any time they read neighbouring segments of the same rows
  // rather than one row region each.
  const int first = rb + w * KC, stride = nw * KC;
  int m[MT];
#pragma unroll
  for (int u = 0; u < MT; ++u) m[u] = min(m0 + 32 * u + i, G.M - 1);
  int n[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) n[j] = min(n0 + 32 * j + i, G.N - 1);

  floatx16 acc[MT][NT];
#pragma unroll
  for (int u = 0; u < MT; ++u)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[u][j][r] = 0.f;

  // the group's path list, one entry per lane, for the W row lookups
  const int pl = (KIND == kGemmGw || G.npg <= 0) ? 0 : a.path_list[G.plist + min(lane, G.npg - 1)];
  const int nch = re > first ? ceil_div(re - first, stride) : 0;
  auto at = [&](int c) { return first + c * stride + VH * h; };
  if constexpr (KIND == kGemmGs) {
    // short reduction (C_out): one chunk ahead, loads guarded so that no
    // chunk past the end is fetched
    Chunk<KIND, MT, NT, VH, WBF16, VEC> c0, c1;
    if (0 < nch) c0.load(a, G, m, n, at(0), re, pl);
    for (int c = 0; c < nch; c += 2) {
      if (c + 1 < nch) c1.load(a, G, m, n, at(c + 1), re, pl);
      c0.mul(acc);
      if (c + 2 < nch) c0.load(a, G, m, n, at(c + 2), re, pl);
      if (c + 1 < nch) c1.mul(acc);
    }
  } else {
    // Three chunk buffers: chunks c+1 and c+2 are in flight while chunk c is
    // multiplied.  Every load is issued unconditionally (a chunk past the end
    // has no valid reductions and reads clamped addresses) and only the
    // multiplies are guarded: guarded loads make the compiler copy the
    // accumulators around the branches.
    // The main loop body is straight-line, so every entry to its header has
    // the same loads in flight (chunks c and c+1, in that order) and the
    // compiler's wait before chunk c's multiplies leaves the younger ones
    // outstanding; a guarded multiply inside the loop makes it drain all
    // loads instead.  The 0 to 2 chunks left over are multiplied after it.
    // Scheduling barriers keep each load group ahead of the multiplies that
    // precede its use (the scheduler would otherwise sink the loads next to
    // their consumers, one chunk of prefetch at best).
    Chunk<KIND, MT, NT, VH, WBF16, VEC> c0, c1, c2;
    c0.load(a, G, m, n, at(0), re, pl);
    c1.load(a, G, m, n, at(1), re, pl);
    int c = 0;
    for (; c + 3 <= nch; c += 3) {
      c2.load(a, G, m, n, at(c + 2), re, pl);
      __builtin_amdgcn_sched_barrier(0);
      c0.mul(acc);
      __builtin_amdgcn_sched_barrier(0);
      c0.load(a, G, m, n, at(c + 3), re, pl);
      __builtin_amdgcn_sched_barrier(0);
      c1.mul(acc);
      __builtin_amdgcn_sched_barrier(0);
      c1.load(a, G, m, n, at(c + 4), re, pl);
      __builtin_amdgcn_sched_barrier(0);
      c2.mul(acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (c < nch) c0.mul(acc);
    if (c + 1 < nch) c1.mul(acc);
  }

  if (nw > 1) {  // fixed-order sum of the waves' partial tiles
    if (w > 0) {
#pragma unroll
      for (int u = 0; u < MT; ++u)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) red[((((w - 1) * MT + u) * NT + j) * 16 + r) * 64 + lane] = acc[u][j][r];
    }
    __syncthreads();
    if (w > 0) return;
    for (int ww = 1; ww < nw; ++ww)
#pragma unroll
      for (int u = 0; u < MT; ++u)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[u][j][r] += red[((((ww - 1) * MT + u) * NT + j) * 16 + r) * 64 + lane];
  }
  // D layout of 32x32x2: register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int u = 0; u < MT; ++u)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gm = m0 + 32 * u + 8 * (r >> 2) + 4 * h + (r & 3);
        const int gn = n0 + 32 * j + i;
        if (gm < G.M && gn < G.N) store_c<KIND>(a, G, gm, gn, acc[u][j][r]);
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
  // summed in split order; eight loads are issued before their adds
  const float* src = a.part + G.part_off + (int64_t)j * G.N + co;
  const int64_t step = (int64_t)G.M * G.N;
  float s = 0.f;
  int sp = 0;
  for (; sp + 8 <= a.splits; sp += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[(sp + u) * step];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; sp < a.splits; ++sp) s += src[sp * step];
  const int cpk = G.npg * a.C_in;
  const int k = j / cpk, r2 = j - k * cpk, q = r2 / a.C_in, ci = r2 - q * a.C_in;
  const int path = a.path_list[G.plist + q];
  a.gw[(((int64_t)k * a.P + path) * a.C_in + ci) * a.C_out + co] = s;
}

__global__ void fill_kernel(float* p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Rows of C features -> bf16 planes of CS >= C values per row, zero past C.
// fp32 input: hi = v rounded to bf16, lo = (v - hi) rounded again; bf16 input
// (lo == NULL): a padded copy.  One thread per plane element (n < 2^31).
__global__ void planes_kernel(const void* x, int x_bf16, uint16_t* hi, uint16_t* lo, uint32_t n, uint32_t C,
                              uint32_t CS) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t r = i / CS, c = i - r * CS;
  if (x_bf16) {
    hi[i] = c < C ? static_cast<const uint16_t*>(x)[(size_t)r * C + c] : (uint16_t)0;
    return;
  }
  const float v = c < C ? static_cast<const float*>(x)[(size_t)r * C + c] : 0.f;
  const __bf16 h = (__bf16)v;
  const __bf16 l = (__bf16)(v - (float)h);
  hi[i] = __builtin_bit_cast(uint16_t, h);
  lo[i] = __builtin_bit_cast(uint16_t, l);
}

// The nrows * C floats of rows row_off.. of a node are contiguous.
__global__ void zero_rows_kernel(float* base, int64_t N, int D, int C, int row_off, int nrows) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)nrows * C;
  if (i >= N * per) return;
  const int64_t node = i / per, r = i - node * per;
  base[(node * D + row_off) * C + r] = 0.f;
}

// Tile of one wave: MT 32-row tiles x NT 32-column tiles.  A value loaded
// for the B operand then serves MT matrix-core products and a row value NT;
// since these products have few columns, the B operand (read from L2 by every
// row tile) costs more than the node-sized A stream, so waves take two row
// tiles when that still leaves enough waves to fill the chip (measured: a
// gain for gW and for 64 or more columns, a loss for the 32-column out and
// g_x products).  gS (reduction C_out, store-bound) takes two column tiles
// per wave when the reduction has at least 64 terms and one otherwise
// (measured both ways).
struct Shape {
  int mt, nt, vh;
};
Shape gemm_shape(int kind, int max_cols, bool two_rows, int kr = 0) {
  if (kind == kGemmGs) return kr >= 64 ? Shape{1, 2, 16} : Shape{1, 1, 16};
  if (two_rows) return max_cols <= 32 ? Shape{2, 1, 8} : Shape{2, 2, 8};
  return max_cols <= 32 ? Shape{1, 1, 16} : (max_cols <= 64 ? Shape{1, 2, 16} : Shape{1, 4, 8});
}
constexpr int64_t kFillWaves = 4096;

template <int KIND, int MT, int NT, int VH, bool WBF16, bool VEC>
hipError_t launch_inst(const GemmArgs& a, dim3 grid, int waves, hipStream_t s) {
  const size_t lds = (size_t)(waves - 1) * MT * NT * 16 * 64 * sizeof(float);
  hipLaunchKernelGGL((gemm_kernel<KIND, MT, NT, VH, WBF16, VEC>), grid, dim3(64 * waves), lds, s, a);
  return hipGetLastError();
}

template <int KIND, int MT, int NT, int VH, bool WBF16>
hipError_t launch_vec(const GemmArgs& a, dim3 grid, int waves, hipStream_t s) {
  return a.vec != 0 ? launch_inst<KIND, MT, NT, VH, WBF16, true>(a, grid, waves, s)
                    : launch_inst<KIND, MT, NT, VH, WBF16, false>(a, grid, waves, s);
}

template <int KIND, bool WBF16>
hipError_t launch_kind(const GemmArgs& a, Shape sh, dim3 grid, int waves, hipStream_t s) {
  if (sh.mt == 1 && sh.nt == 1 && sh.vh == 16) return launch_vec<KIND, 1, 1, 16, WBF16>(a, grid, waves, s);
  if (sh.mt == 2 && sh.nt == 1 && sh.vh == 8) return launch_vec<KIND, 2, 1, 8, WBF16>(a, grid, waves, s);
  if (sh.mt == 2 && sh.nt == 2 && sh.vh == 8) return launch_vec<KIND, 2, 2, 8, WBF16>(a, grid, waves, s);
  if (sh.mt == 1 && sh.nt == 2 && sh.vh == 16) return launch_vec<KIND, 1, 2, 16, WBF16>(a, grid, waves, s);
  if (KIND != kGemmGs && sh.mt == 1 && sh.nt == 4 && sh.vh == 8) return launch_vec<KIND, 1, 4, 8, WBF16>(a, grid, waves, s);
  return hipErrorInvalidValue;
}

}  // namespace

int64_t gemm_wave_tiles(int kind, int M, int N, int max_cols) {
  if (M <= 0 || N <= 0) return 0;
  const Shape sh = gemm_shape(kind, max_cols, true);
  return (int64_t)ceil_div(M, 32 * sh.mt) * ceil_div(N, 32 * sh.nt);
}

hipError_t launch_gemm(int kind, GemmArgs& a, hipStream_t s) {
  if (a.ngroups <= 0) return hipSuccess;
  int max_cols = 0, max_kr = 0;
  for (int g = 0; g < a.ngroups; ++g) max_cols = a.g[g].N > max_cols ? a.g[g].N : max_cols;
  const int splits = kind == kGemmGw ? a.splits : 1;
  Shape sh = gemm_shape(kind, max_cols, true, a.C_out);
  {
    int64_t t2 = 0;
    for (int g = 0; g < a.ngroups; ++g)
      if (a.g[g].M > 0 && a.g[g].N > 0 && a.g[g].Kr > 0)
        t2 += (int64_t)ceil_div(a.g[g].M, 32 * sh.mt) * ceil_div(a.g[g].N, 32 * sh.nt);
    if (!(kind == kGemmGw || max_cols > 32) || t2 * splits * kMaxWaveSplit < kFillWaves)
      sh = gemm_shape(kind, max_cols, false, a.C_out);
  }
  int64_t total = 0;
  for (int g = 0; g < a.ngroups; ++g) {
    GemmGroup& G = a.g[g];
    G.tiles_n = G.N > 0 ? ceil_div(G.N, 32 * sh.nt) : 0;
    G.tiles = (G.M > 0 && G.N > 0 && G.Kr > 0) ? ceil_div(G.M, 32 * sh.mt) * G.tiles_n : 0;
    G.tile_begin = (int32_t)total;
    total += G.tiles;
    if (G.tiles > 0 && G.Kr > max_kr) max_kr = G.Kr;
  }
  if (total == 0) return hipSuccess;
  if (total > INT32_MAX) return hipErrorInvalidValue;
  // Split the reduction over the waves of a block while the launch is small
  // and every wave keeps at least four chunks of the reduction.
  const int kc = 2 * sh.vh;
  int waves = 1;
  while (waves < kMaxWaveSplit && total * splits * waves < kTargetWaves &&
         (int64_t)max_kr >= (int64_t)splits * waves * 2 * 4 * kc)
    waves *= 2;
  const dim3 grid((unsigned)total, (unsigned)splits, 1);
  const bool wb = a.w_bf16 != 0;
  TimingScope ts(kcGemmOut + kind, s);
  switch (kind) {
    case kGemmOut: return wb ? launch_kind<kGemmOut, true>(a, sh, grid, waves, s) : launch_kind<kGemmOut, false>(a, sh, grid, waves, s);
    case kGemmGs: return wb ? launch_kind<kGemmGs, true>(a, sh, grid, waves, s) : launch_kind<kGemmGs, false>(a, sh, grid, waves, s);
    case kGemmGx: return wb ? launch_kind<kGemmGx, true>(a, sh, grid, waves, s) : launch_kind<kGemmGx, false>(a, sh, grid, waves, s);
    case kGemmGw: return launch_kind<kGemmGw, false>(a, sh, grid, waves, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gw_reduce(const ReduceArgs& a, int64_t total, hipStream_t s) {
  if (total <= 0) return hipSuccess;
  TimingScope ts(kcGwReduce, s);
  hipLaunchKernelGGL(gw_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a, total);
  return hipGetLastError();
}

hipError_t launch_zero_rows(float* base, int64_t N, int D, int C, int row_off, int nrows, hipStream_t s) {
  const int64_t n = N * nrows * (int64_t)C;
  if (n <= 0) return hipSuccess;
  if (row_off < 0 || nrows < 0 || row_off + nrows > D) return hipErrorInvalidValue;
  TimingScope ts(kcFill, s);
  hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, base, N, D, C, row_off,
                     nrows);
  return hipGetLastError();
}

hipError_t launch_planes(const void* x, bool x_bf16, int64_t rows, int C, int CS, uint16_t* hi, uint16_t* lo,
                         hipStream_t s) {
  const int64_t n = rows * CS;
  if (n <= 0) return hipSuccess;
  if (n >= INT32_MAX || CS < C || (!x_bf16 && !lo)) return hipErrorInvalidValue;
  TimingScope ts(kcFill, s);
  hipLaunchKernelGGL(planes_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, x_bf16 ? 1 : 0, hi, lo,
                     (uint32_t)n, (uint32_t)C, (uint32_t)CS);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TimingScope ts(kcFill, s);
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace tpconv
