// Dense contractions with the shared weights W on the bf16 matrix cores at
// fp32 accuracy.
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
// Every product runs on v_mfma_f32_32x32x16_bf16 with each fp32 operand split
// into bf16 hi + lo and the tile formed as hi*hi' + hi*lo' + lo*hi' (each
// exact in the fp32 accumulator; a bf16 operand has no lo part).  W and g_out
// come pre-split into bf16 planes (W also transposed per (k, p), so that every
// B operand is contiguous along its reduction); the node-sized states S and T
// are split in registers as they are loaded.
//
// These products are skinny (32..128 columns) and stream a node-sized
// operand once, so the kernel is built for bytes in flight rather than for
// LDS reuse.  Every wave owns a (32*MT)-row x (32*NT)-column tile and loads its
// operands straight into registers: lane (i, h) (i = lane % 32, h = lane / 32)
// supplies row i of A and column i of B at the reduction indices
// r0 + VH*h + t (t = 0..VH-1) of a chunk of 2*VH, the s-th product of a chunk
// taking t = 8s..8s+7 from both halves.  An operand that is contiguous along
// the reduction is then read as 16-byte vectors per lane; one that is
// contiguous along its row or column index is read as coalesced rows.  The
// next chunks are loaded while the current one is multiplied.  Small problems
// split the reduction over the 1, 2 or 4 waves of a block (interleaved chunks,
// so that the waves read neighbouring segments of a row); the waves' partial
// tiles are summed in a fixed order through LDS, so results do not depend on
// timing.
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
  if constexpr (KIND == kGemmOut || KIND == kGemmGx) {
    const float* row = a.state + G.state_off + (int64_t)m * G.Kr;
    // VEC: Kr is a multiple of 16 and rs of VH, so a whole run is in or out
    const int rc = VEC ? (rs < r_end ? rs : r_end - VH) : (rs < r_end ? rs : r_end - 1);
    load_run<VH, VEC>(row + (rc > 0 ? rc : 0), r_end - rs, v);
  } else {  // Gw: A(j, r) = S_g[r][j], contiguous along j across the lanes
    const float* p = a.state + G.state_off + m;
#pragma unroll
    for (int t = 0; t < VH; ++t) v[t] = p[(int64_t)min(rs + t, G.Kr - 1) * G.M];
  }
}

// VH consecutive bf16 p[0..VH) as VH/2 packed words (16-byte loads).
template <int VH>
__device__ __forceinline__ void load_words(const uint16_t* p, uint32_t (&w)[VH / 2]) {
#pragma unroll
  for (int j = 0; j < VH / 8; ++j) {
    const uint4 u = *reinterpret_cast<const uint4*>(p + 8 * j);
    w[4 * j] = u.x;
    w[4 * j + 1] = u.y;
    w[4 * j + 2] = u.z;
    w[4 * j + 3] = u.w;
  }
}
__device__ __forceinline__ uint32_t pack2(uint16_t lo, uint16_t hi) { return (uint32_t)lo | ((uint32_t)hi << 16); }

// A operand of gS from the g_out planes: values t = 0..VH-1 of row m at
// reductions (co) rs + t.  The planes are zero past C_out up to their
// channel stride, a multiple of 32, so a chunk never leaves its row.
template <int VH>
__device__ __forceinline__ void load_a_planes(const GemmArgs& a, const GemmGroup& G, int m, int rs,
                                              uint32_t (&h)[VH / 2], uint32_t (&l)[VH / 2]) {
  const int node = m / G.n, mm = m - node * G.n;
  const int64_t off = ((int64_t)node * a.D_feat + G.row_off + mm) * a.feat_cs + rs;
  load_words<VH>(a.feat_hi + off, h);
  load_words<VH>(a.feat_lo + off, l);
}

// B operand: values t = 0..VH-1 of column n at reductions rs + t as packed
// bf16 words (hi, and lo where LO); indices past the end of the reduction
// read inside the tensor (their A values are zero).
template <int KIND, int VH, bool LO, bool VEC>
__device__ __forceinline__ void load_b(const GemmArgs& a, const GemmGroup& G, int n, int rs, int r_end, int pl,
                                       uint32_t (&bh)[VH / 2], uint32_t (&bl)[LO ? VH / 2 : 1]) {
  if constexpr (KIND == kGemmGw) {  // B(r = (v, m3), n = co) = g_out planes; rows stepped without division
    const int r0 = min(rs, G.Kr - 1);
    int node = r0 / G.n, mm = r0 - node * G.n;
    const int64_t col = (int64_t)G.row_off * a.feat_cs + n;
    uint16_t vh[VH], vl[VH];
#pragma unroll
    for (int t = 0; t < VH; ++t) {
      const int64_t o = ((int64_t)node * a.D_feat + mm) * a.feat_cs + col;
      vh[t] = a.feat_hi[o];
      vl[t] = a.feat_lo[o];
      // next row; past the end of the reduction the last row is read again
      const bool adv = rs + t + 1 < G.Kr;
      const bool wrap = mm + 1 == G.n;
      const int mm2 = wrap ? 0 : mm + 1, node2 = wrap ? node + 1 : node;
      mm = adv ? mm2 : mm;
      node = adv ? node2 : node;
    }
#pragma unroll
    for (int t = 0; t < VH / 2; ++t) {
      bh[t] = pack2(vh[2 * t], vh[2 * t + 1]);
      if constexpr (LO) bl[t] = pack2(vl[2 * t], vl[2 * t + 1]);
    }
  } else {
    // out: B(r = (k,q,ci), n = co) = W^T planes [k][p][co][ci]
    // gS:  B(r = co, n = (k,q,ci)) = W planes [k][p][ci][co]
    // g_x: B(r = (k,q,co), n = ci) = W planes [k][p][ci][co]
    const uint16_t* ph = KIND == kGemmOut ? a.wt_hi : a.w_hi;
    const uint16_t* plo = KIND == kGemmOut ? a.wt_lo : a.w_lo;
    // element index of reduction r (any r below the end of the reduction)
    auto index = [&](int r) -> int64_t {
      if constexpr (KIND == kGemmGs) {
        int ci;
        const int64_t kp = w_row(a, G, n, a.C_in, pl, ci);
        return (kp * a.C_in + ci) * a.C_out + r;
      } else {
        int c;
        const int64_t kp = w_row(a, G, r, KIND == kGemmOut ? a.C_in : a.C_out, pl, c);
        return KIND == kGemmOut ? (kp * a.C_out + n) * a.C_in + c : (kp * a.C_in + n) * a.C_out + c;
      }
    };
    if constexpr (VEC) {
      // the VH reductions of a lane half are consecutive elements: C_in and
      // C_out are multiples of 16, so they share (k, q)
      int64_t base;
      if constexpr (KIND == kGemmGs) {
        base = index(rs < r_end ? rs : 0);
      } else {
        int c;
        const int64_t kp = w_row_halves(a, G, rs < r_end ? rs : 0, KIND == kGemmOut ? a.C_in : a.C_out, pl,
                                        (int)(threadIdx.x & 63) >> 5, c);
        base = KIND == kGemmOut ? (kp * a.C_out + n) * a.C_in + c : (kp * a.C_in + n) * a.C_out + c;
      }
      load_words<VH>(ph + base, bh);
      if constexpr (LO) load_words<VH>(plo + base, bl);
    } else {
      uint16_t vh[VH], vl[VH];
#pragma unroll
      for (int t = 0; t < VH; ++t) {
        const int64_t o = index(min(rs + t, r_end - 1));
        vh[t] = ph[o];
        if constexpr (LO) vl[t] = plo[o];
      }
#pragma unroll
      for (int t = 0; t < VH / 2; ++t) {
        bh[t] = pack2(vh[2 * t], vh[2 * t + 1]);
        if constexpr (LO) bl[t] = pack2(vl[2 * t], vl[2 * t + 1]);
      }
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

__device__ __forceinline__ floatx16 mfma32(u32x4 a, u32x4 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// WLO: W has a lo plane (fp32 weights).  A is fp32 (split here) except for
// gS, whose A is the g_out planes; B of gW is the g_out planes (always with lo).
template <int KIND, int MT, int NT, int VH, bool WLO, bool VEC>
struct Chunk {
  static constexpr bool APLANE = KIND == kGemmGs;
  static constexpr bool BLO = WLO || KIND == kGemmGw;
  static constexpr int AW = VH / 2;
  float a[APLANE ? 1 : MT][VH];
  uint32_t pah[APLANE ? MT : 1][AW], pal[APLANE ? MT : 1][AW];
  uint32_t bh[NT][AW], bl[NT][BLO ? AW : 1];
  int valid;  // reductions of this lane half inside the range (<= 0: none)
  __device__ __forceinline__ void load(const GemmArgs& ar, const GemmGroup& G, const int (&m)[MT], const int (&n)[NT],
                                       int rs, int r_end, int pl) {
    valid = r_end - rs;
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      if constexpr (APLANE)
        load_a_planes<VH>(ar, G, m[u], rs, pah[u], pal[u]);
      else
        load_a<KIND, VH, VEC>(ar, G, m[u], rs, r_end, a[u]);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) load_b<KIND, VH, BLO, VEC>(ar, G, n[j], rs, r_end, pl, bh[j], bl[j]);
  }
  __device__ __forceinline__ void mul(floatx16 (&acc)[MT][NT], const SplitConsts& sk) const {
#pragma unroll
    for (int s = 0; s < VH / 8; ++s) {
      u32x4 Ah[MT], Al[MT];
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        if constexpr (APLANE) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            Ah[u][t] = pah[u][4 * s + t];
            Al[u][t] = pal[u][4 * s + t];
          }
        } else {
          float v[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) v[t] = 8 * s + t < valid ? a[u][8 * s + t] : 0.f;  // past the end: zero
          split8(v, Ah[u], Al[u], sk);
        }
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        u32x4 Bh, Bl;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          Bh[t] = bh[j][4 * s + t];
          if constexpr (BLO) Bl[t] = bl[j][4 * s + t];
        }
#pragma unroll
        for (int u = 0; u < MT; ++u) {
          acc[u][j] = mfma32(Ah[u], Bh, acc[u][j]);
          if constexpr (BLO) acc[u][j] = mfma32(Ah[u], Bl, acc[u][j]);
          acc[u][j] = mfma32(Al[u], Bh, acc[u][j]);
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

template <int KIND, int MT, int NT, int VH, bool WLO, bool VEC>
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

  const SplitConsts sk;
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
  if constexpr (KIND == kGemmGs || KIND == kGemmGw) {
    // one chunk ahead, loads guarded so that no chunk past the end is
    // fetched (gS: a short reduction, C_out; gW: B gathered element by
    // element, whose registers leave room for one chunk in flight only)
    Chunk<KIND, MT, NT, VH, WLO, VEC> c0, c1;
    if (0 < nch) c0.load(a, G, m, n, at(0), re, pl);
    for (int c = 0; c < nch; c += 2) {
      if (c + 1 < nch) c1.load(a, G, m, n, at(c + 1), re, pl);
      c0.mul(acc, sk);
      if (c + 2 < nch) c0.load(a, G, m, n, at(c + 2), re, pl);
      if (c + 1 < nch) c1.mul(acc, sk);
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
    Chunk<KIND, MT, NT, VH, WLO, VEC> c0, c1, c2;
    c0.load(a, G, m, n, at(0), re, pl);
    c1.load(a, G, m, n, at(1), re, pl);
    int c = 0;
    for (; c + 3 <= nch; c += 3) {
      c2.load(a, G, m, n, at(c + 2), re, pl);
      __builtin_amdgcn_sched_barrier(0);
      c0.mul(acc, sk);
      __builtin_amdgcn_sched_barrier(0);
      c0.load(a, G, m, n, at(c + 3), re, pl);
      __builtin_amdgcn_sched_barrier(0);
      c1.mul(acc, sk);
      __builtin_amdgcn_sched_barrier(0);
      c1.load(a, G, m, n, at(c + 4), re, pl);
      __builtin_amdgcn_sched_barrier(0);
      c2.mul(acc, sk);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (c < nch) c0.mul(acc, sk);
    if (c + 1 < nch) c1.mul(acc, sk);
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
  // D layout of the 32x32 products: register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32
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

// Products with many row tiles: a block of RW waves takes RW consecutive
// 32-row tiles and one block of 32*NT columns.  The chunk of B
// that all of them need is loaded once per block into LDS, in two buffers
// (chunk c+1 is written while chunk c is read), instead of once per wave
// from L2; each wave then reads its column fragments from LDS.  A comes
// straight from memory into registers, one chunk ahead.  Needs 16-byte
// operand loads (channel counts that are multiples of 16).
template <int NT, int VH>
struct __attribute__((aligned(16))) BStage {  // one chunk of B as bf16: [plane][column][reduction]
  static constexpr int KC = 2 * VH;
  static constexpr int RS = KC + 8;  // row stride: 16-byte aligned rows, spread over the banks
  uint16_t v[2][32 * NT][RS];
};

template <int KIND, int NT, int VH, bool WLO, int RW>
__global__ __launch_bounds__(64 * RW) __attribute__((amdgpu_waves_per_eu(NT >= 4 ? 2 : 3)))
void gemm_lds_kernel(const GemmArgs /*args*/) {
  const GemmArgs& a = *(const GemmArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr bool APLANE = KIND == kGemmGs;
  constexpr bool BLO = WLO || KIND == kGemmGw;
  constexpr int KC = 2 * VH, NC = 32 * NT;
  constexpr int NQ = NC * KC / 8;                                  // 8-element pieces of a chunk, per plane
  constexpr int QP = (NQ + 64 * RW - 1) / (64 * RW);  // pieces per thread
  __shared__ BStage<NT, VH> stage[2];
  const int b = blockIdx.x;
  int gi = 0;
  while (gi + 1 < a.ngroups && b >= a.g[gi + 1].tile_begin) ++gi;
  const GemmGroup& G = a.g[gi];
  const int tile = b - G.tile_begin;
  if (tile >= G.tiles) return;  // uniform over the block
  const int tm = tile / G.tiles_n, tn = tile - tm * G.tiles_n;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 31, h = lane >> 5;
  const int m0 = (tm * RW + w) * 32, n0 = tn * NC;
  int rb = 0, re = G.Kr;
  // gW, and out / g_x with too few row tiles, split the reduction over blocks
  const bool split = KIND == kGemmGw || ((KIND == kGemmOut || KIND == kGemmGx) && a.splits > 1);
  if (split) {
    const int per = ceil_div(ceil_div(G.Kr, a.splits), KC) * KC;
    rb = min(G.Kr, (int)blockIdx.y * per);
    re = min(G.Kr, rb + per);
  }
  const int nch = re > rb ? ceil_div(re - rb, KC) : 0;
  const int m = min(m0 + i, G.M - 1);
  const int pl = (KIND == kGemmGw || G.npg <= 0) ? 0 : a.path_list[G.plist + min(lane, G.npg - 1)];
  const SplitConsts sk;

  // gW: the g_out row (node, mm) of each of this thread's pieces, advanced
  // by one chunk at a time without division; rows past the last one read the
  // last one (their A values are zero)
  int gnode[QP], gmm[QP];
  const int dnode = KC / G.n, dmm = KC - dnode * G.n;
  const int lnode = (G.Kr - 1) / G.n, lmm = (G.Kr - 1) - lnode * G.n;
  if constexpr (KIND == kGemmGw) {
#pragma unroll
    for (int p = 0; p < QP; ++p) {
      const int r = rb + (tid + p * 64 * RW) / (NC / 8);
      gnode[p] = r / G.n;
      gmm[p] = r - gnode[p] * G.n;
    }
  }
  // piece q (the p-th of this thread) of chunk c (hi, and lo where BLO): 8
  // consecutive reductions of one column (W planes), or for gW 8 consecutive
  // columns of one reduction (g_out planes); clamped inside the tensors
  // (their A values are zero)
  auto piece_load = [&](int c, int q, int p, uint4& vh, uint4& vl) {
    const int r0 = rb + c * KC;
    int64_t idx;
    const uint16_t *ph, *plo;
    if constexpr (KIND == kGemmGw) {
      const int red = q / (NC / 8), cg = q - red * (NC / 8);
      const bool past = r0 + red > G.Kr - 1;
      const int node = past ? lnode : gnode[p], mm = past ? lmm : gmm[p];
      const int co = min(n0 + 8 * cg, a.feat_cs - 8);
      idx = ((int64_t)node * a.D_feat + G.row_off + mm) * a.feat_cs + co;
      ph = a.feat_hi;
      plo = a.feat_lo;
      // the next chunk's row
      gmm[p] += dmm;
      gnode[p] += dnode;
      if (gmm[p] >= G.n) {
        gmm[p] -= G.n;
        gnode[p] += 1;
      }
    } else {
      const int col = q / (KC / 8), part = q - col * (KC / 8);
      const int n = min(n0 + col, G.N - 1);
      const int r = min(r0 + 8 * part, G.Kr - 8);
      int c2;
      if constexpr (KIND == kGemmOut) {
        const int64_t kp = w_row(a, G, r, a.C_in, pl, c2);
        idx = (kp * a.C_out + n) * a.C_in + c2;
      } else if constexpr (KIND == kGemmGs) {
        const int64_t kp = w_row(a, G, n, a.C_in, pl, c2);
        idx = (kp * a.C_in + c2) * a.C_out + r;
      } else {
        const int64_t kp = w_row(a, G, r, a.C_out, pl, c2);
        idx = (kp * a.C_in + n) * a.C_out + c2;
      }
      ph = KIND == kGemmOut ? a.wt_hi : a.w_hi;
      plo = KIND == kGemmOut ? a.wt_lo : a.w_lo;
    }
    vh = *reinterpret_cast<const uint4*>(ph + idx);
    if constexpr (BLO) vl = *reinterpret_cast<const uint4*>(plo + idx);
  };
  auto piece_store = [&](BStage<NT, VH>& st, int q, const uint4& vh, const uint4& vl) {
    if constexpr (KIND == kGemmGw) {
      const int red = q / (NC / 8), cg = q - red * (NC / 8);
      const uint32_t wh[4] = {vh.x, vh.y, vh.z, vh.w}, wl[4] = {vl.x, vl.y, vl.z, vl.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        st.v[0][8 * cg + e][red] = (uint16_t)(wh[e >> 1] >> (16 * (e & 1)));
        st.v[1][8 * cg + e][red] = (uint16_t)(wl[e >> 1] >> (16 * (e & 1)));
      }
    } else {
      const int col = q / (KC / 8), part = q - col * (KC / 8);
      *reinterpret_cast<uint4*>(&st.v[0][col][8 * part]) = vh;
      if constexpr (BLO) *reinterpret_cast<uint4*>(&st.v[1][col][8 * part]) = vl;
    }
  };
  auto a_load = [&](int c, float (&av)[VH], uint32_t (&ah)[VH / 2], uint32_t (&al)[VH / 2]) {
    const int rs = rb + c * KC + VH * h;
    if constexpr (APLANE)
      load_a_planes<VH>(a, G, m, rs < re ? rs : re - VH, ah, al);
    else
      load_a<KIND, VH, true>(a, G, m, rs, re, av);
  };

  floatx16 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;

  // A and the B pieces of chunk c+1 are in flight while chunk c is multiplied
  float av[VH], avn[VH];
  uint32_t pah[VH / 2], pal[VH / 2], pahn[VH / 2], paln[VH / 2];
  uint4 sh[QP], sl[QP];
  if (nch > 0) {
#pragma unroll
    for (int p = 0; p < QP; ++p)
      if (tid + p * 64 * RW < NQ) piece_load(0, tid + p * 64 * RW, p, sh[p], sl[p]);
#pragma unroll
    for (int p = 0; p < QP; ++p)
      if (tid + p * 64 * RW < NQ) piece_store(stage[0], tid + p * 64 * RW, sh[p], sl[p]);
    a_load(0, av, pah, pal);
    // chunk 0 of A has arrived before the loop: the loop is then entered
    // with no load in flight into the registers it multiplies, as from its
    // own back edge, and the waits the compiler places for the next chunk's
    // loads stay after the multiplies
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  }
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    // the next chunk's loads are issued unconditionally (past the last chunk
    // they read clamped addresses inside the tensors and are not used): a
    // guarded load splits the loop body, and where the paths join the
    // compiler waits for every load in flight before the multiplies
#pragma unroll
    for (int p = 0; p < QP; ++p)
      if (tid + p * 64 * RW < NQ) piece_load(c + 1, tid + p * 64 * RW, p, sh[p], sl[p]);
    a_load(c + 1, avn, pahn, paln);
    // keep the loads ahead of the multiplies (the scheduler would otherwise
    // sink them next to their use at the end of the chunk)
    __builtin_amdgcn_sched_barrier(0);
    const BStage<NT, VH>& st = stage[c & 1];
    const int valid = re - (rb + c * KC + VH * h);
#pragma unroll
    for (int s2 = 0; s2 < VH / 8; ++s2) {
      u32x4 Ah, Al;
      if constexpr (APLANE) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          Ah[t] = pah[4 * s2 + t];
          Al[t] = pal[4 * s2 + t];
        }
      } else {
        float v[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = 8 * s2 + t < valid ? av[8 * s2 + t] : 0.f;  // past the end: zero
        split8(v, Ah, Al, sk);
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const u32x4 Bh = *reinterpret_cast<const u32x4*>(&st.v[0][32 * j + i][VH * h + 8 * s2]);
        acc[j] = mfma32(Ah, Bh, acc[j]);
        if constexpr (BLO) {
          const u32x4 Bl = *reinterpret_cast<const u32x4*>(&st.v[1][32 * j + i][VH * h + 8 * s2]);
          acc[j] = mfma32(Ah, Bl, acc[j]);
        }
        acc[j] = mfma32(Al, Bh, acc[j]);
      }
    }
    // chunk c+1's pieces into the other buffer (after the last chunk the
    // store is unused; that buffer was last read before the previous barrier)
#pragma unroll
    for (int p = 0; p < QP; ++p)
      if (tid + p * 64 * RW < NQ) piece_store(stage[(c + 1) & 1], tid + p * 64 * RW, sh[p], sl[p]);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < VH; ++t) av[t] = avn[t];
#pragma unroll
    for (int t = 0; t < VH / 2; ++t) {
      pah[t] = pahn[t];
      pal[t] = paln[t];
    }
  }
  if (m0 >= G.M) return;
  const bool to_part = (KIND == kGemmOut || KIND == kGemmGx) && a.splits > 1;
  // D layout of the 32x32 products: register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int gm = m0 + 8 * (r >> 2) + 4 * h + (r & 3);
      const int gn = n0 + 32 * j + i;
      if (gm < G.M && gn < G.N) {
        if (to_part)
          a.part[G.part_off + ((int64_t)blockIdx.y * G.M + gm) * G.N + gn] = acc[j][r];
        else
          store_c<KIND>(a, G, gm, gn, acc[j][r]);
      }
    }
}

// out / g_x from their split partial sums, summed in split order (the
// element's group found by a linear scan over at most kMaxGroups groups).
template <int KIND>
__global__ void rows_reduce_kernel(const GemmArgs /*args*/, int64_t total) {
  const GemmArgs& a = *(const GemmArgs*)__builtin_amdgcn_kernarg_segment_ptr();
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
  const int m = (int)(rem / G.N), n = (int)(rem - (int64_t)m * G.N);
  const float* src = a.part + G.part_off + rem;
  const int64_t step = (int64_t)G.M * G.N;
  float v = 0.f;
  for (int sp = 0; sp < a.splits; ++sp) v += src[sp * step];
  store_c<KIND>(a, G, m, n, v);
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

// W [KP][Ci][Co] -> bf16 planes in its layout and transposed per (k, p) to
// [KP][Co][Ci]: fp32 split into hi + lo, bf16 copied (lo == NULL).
__global__ void w_planes_kernel(const void* W, int w_bf16, int64_t n, int Ci, int Co, uint16_t* hi, uint16_t* lo,
                                uint16_t* thi, uint16_t* tlo) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t per = (int64_t)Ci * Co, kp = i / per;
  const int rem = (int)(i - kp * per), ci = rem / Co, co = rem - ci * Co;
  const int64_t t = kp * per + (int64_t)co * Ci + ci;
  if (w_bf16) {
    const uint16_t v = static_cast<const uint16_t*>(W)[i];
    hi[i] = v;
    thi[t] = v;
    return;
  }
  const float v = static_cast<const float*>(W)[i];
  const __bf16 h = (__bf16)v;
  const __bf16 l = (__bf16)(v - (float)h);
  hi[i] = thi[t] = __builtin_bit_cast(uint16_t, h);
  lo[i] = tlo[t] = __builtin_bit_cast(uint16_t, l);
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

template <int KIND, int MT, int NT, int VH, bool WLO, bool VEC>
hipError_t launch_inst(const GemmArgs& a, dim3 grid, int waves, hipStream_t s) {
  const size_t lds = (size_t)(waves - 1) * MT * NT * 16 * 64 * sizeof(float);
  hipLaunchKernelGGL((gemm_kernel<KIND, MT, NT, VH, WLO, VEC>), grid, dim3(64 * waves), lds, s, a);
  return hipGetLastError();
}

template <int KIND, int MT, int NT, int VH, bool WLO>
hipError_t launch_vec(const GemmArgs& a, dim3 grid, int waves, hipStream_t s) {
  if constexpr (VH == 8) {
    return a.vec != 0 ? launch_inst<KIND, MT, NT, VH, WLO, true>(a, grid, waves, s)
                      : launch_inst<KIND, MT, NT, VH, WLO, false>(a, grid, waves, s);
  } else {  // 16 reductions per lane half only with 16-byte operand loads
    return a.vec != 0 ? launch_inst<KIND, MT, NT, VH, WLO, true>(a, grid, waves, s) : hipErrorInvalidValue;
  }
}

template <int KIND, bool WLO>
hipError_t launch_kind(const GemmArgs& a, Shape sh, dim3 grid, int waves, hipStream_t s) {
  if (sh.mt == 1 && sh.nt == 1 && sh.vh == 8) return launch_vec<KIND, 1, 1, 8, WLO>(a, grid, waves, s);
  if (sh.mt == 1 && sh.nt == 2 && sh.vh == 8) return launch_vec<KIND, 1, 2, 8, WLO>(a, grid, waves, s);
  if (sh.mt == 1 && sh.nt == 1 && sh.vh == 16) return launch_vec<KIND, 1, 1, 16, WLO>(a, grid, waves, s);
  if (sh.mt == 2 && sh.nt == 1 && sh.vh == 8) return launch_vec<KIND, 2, 1, 8, WLO>(a, grid, waves, s);
  if (sh.mt == 2 && sh.nt == 2 && sh.vh == 8) return launch_vec<KIND, 2, 2, 8, WLO>(a, grid, waves, s);
  if (sh.mt == 1 && sh.nt == 2 && sh.vh == 16) return launch_vec<KIND, 1, 2, 16, WLO>(a, grid, waves, s);
  if (KIND != kGemmGs && sh.mt == 1 && sh.nt == 4 && sh.vh == 8) return launch_vec<KIND, 1, 4, 8, WLO>(a, grid, waves, s);
  return hipErrorInvalidValue;
}

// Waves per block (row tiles sharing a B chunk), and reductions per lane
// half: 16 for column blocks of one or two tiles (measured faster for out,
// g_x and gW there; not for gS, nor with four tiles, whose registers then
// leave too little room).
constexpr int lds_rows(int nt) { return 4; }

template <int KIND, int NT, bool WLO>
hipError_t launch_lds(const GemmArgs& a, dim3 grid, hipStream_t s) {
  constexpr int VH = (NT <= 2 && KIND != kGemmGs) ? 16 : 8;
  constexpr int RW = lds_rows(NT);
  hipLaunchKernelGGL((gemm_lds_kernel<KIND, NT, VH, WLO, RW>), grid, dim3(64 * RW), 0, s, a);
  return hipGetLastError();
}

template <int KIND, bool WLO>
hipError_t launch_lds_nt(const GemmArgs& a, int nt, dim3 grid, hipStream_t s) {
  if (nt == 1) return launch_lds<KIND, 1, WLO>(a, grid, s);
  if (nt == 2) return launch_lds<KIND, 2, WLO>(a, grid, s);
  return launch_lds<KIND, 4, WLO>(a, grid, s);
}

// The LDS-staged kernel for launches of at least this many waves (with
// 16-byte operand loads); smaller ones split the reduction instead.
constexpr int64_t kLdsMinWaves = 2048;

// Column tiles of the LDS-staged kernel: the whole (up to 128) columns in one block.
int lds_nt(int max_cols) { return max_cols <= 32 ? 1 : (max_cols <= 64 ? 2 : 4); }

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
  // gW reads no W; the other kinds take the lo plane of fp32 weights
  const bool wlo = a.w_lo != nullptr;
  if (kind != kGemmGw && (!a.w_hi || !a.wt_hi || (wlo != (a.wt_lo != nullptr)))) return hipErrorInvalidValue;
  if ((kind == kGemmGs || kind == kGemmGw) && (!a.feat_hi || !a.feat_lo || a.feat_cs % 32 != 0))
    return hipErrorInvalidValue;
  if (a.vec) {  // many row tiles: blocks of kLdsWaves row tiles sharing B through LDS
    const int nt = lds_nt(kind == kGemmGs ? 128 : max_cols), rw = lds_rows(nt);
    int64_t blocks = 0;
    for (int g = 0; g < a.ngroups; ++g) {
      const GemmGroup& G = a.g[g];
      if (G.M > 0 && G.N > 0 && G.Kr > 0) blocks += (int64_t)ceil_div(ceil_div(G.M, 32), rw) * ceil_div(G.N, 32 * nt);
    }
    const int ysplits = (kind == kGemmOut || kind == kGemmGx) ? a.splits : splits;
    if (blocks * rw * splits >= kLdsMinWaves) {
      if ((kind == kGemmOut || kind == kGemmGx) && ysplits > 1 && !a.part) return hipErrorInvalidValue;
      int64_t total = 0;
      for (int g = 0; g < a.ngroups; ++g) {
        GemmGroup& G = a.g[g];
        G.tiles_n = G.N > 0 ? ceil_div(G.N, 32 * nt) : 0;
        G.tiles = (G.M > 0 && G.N > 0 && G.Kr > 0) ? ceil_div(ceil_div(G.M, 32), rw) * G.tiles_n : 0;
        G.tile_begin = (int32_t)total;
        total += G.tiles;
      }
      if (total > INT32_MAX) return hipErrorInvalidValue;
      const dim3 grid((unsigned)total, (unsigned)ysplits, 1);
      TimingScope ts(kcGemmOut + kind, s);
      switch (kind) {
        case kGemmOut: return wlo ? launch_lds_nt<kGemmOut, true>(a, nt, grid, s) : launch_lds_nt<kGemmOut, false>(a, nt, grid, s);
        case kGemmGs: return wlo ? launch_lds_nt<kGemmGs, true>(a, nt, grid, s) : launch_lds_nt<kGemmGs, false>(a, nt, grid, s);
        case kGemmGx: return wlo ? launch_lds_nt<kGemmGx, true>(a, nt, grid, s) : launch_lds_nt<kGemmGx, false>(a, nt, grid, s);
        case kGemmGw: return launch_lds_nt<kGemmGw, false>(a, nt, grid, s);
        default: return hipErrorInvalidValue;
      }
    }
  }
  Shape sh = gemm_shape(kind, max_cols, true, a.C_out);
  {
    int64_t t2 = 0;
    for (int g = 0; g < a.ngroups; ++g)
      if (a.g[g].M > 0 && a.g[g].N > 0 && a.g[g].Kr > 0)
        t2 += (int64_t)ceil_div(a.g[g].M, 32 * sh.mt) * ceil_div(a.g[g].N, 32 * sh.nt);
    if (!(kind == kGemmGw || max_cols > 32) || t2 * splits * kMaxWaveSplit < kFillWaves)
      sh = gemm_shape(kind, max_cols, false, a.C_out);
  }
  // element-by-element operands keep 8 reductions per lane half (registers)
  if (!a.vec) sh.vh = 8;
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
  TimingScope ts(kcGemmOut + kind, s);
  switch (kind) {
    case kGemmOut: return wlo ? launch_kind<kGemmOut, true>(a, sh, grid, waves, s) : launch_kind<kGemmOut, false>(a, sh, grid, waves, s);
    case kGemmGs: return wlo ? launch_kind<kGemmGs, true>(a, sh, grid, waves, s) : launch_kind<kGemmGs, false>(a, sh, grid, waves, s);
    case kGemmGx: return wlo ? launch_kind<kGemmGx, true>(a, sh, grid, waves, s) : launch_kind<kGemmGx, false>(a, sh, grid, waves, s);
    case kGemmGw: return launch_kind<kGemmGw, false>(a, sh, grid, waves, s);
    default: return hipErrorInvalidValue;
  }
}

int gemm_rows_splits(int kind, const GemmArgs& a) {
  if ((kind != kGemmOut && kind != kGemmGx) || !a.vec || a.ngroups <= 0) return 1;
  int max_cols = 0, max_kr = 0;
  for (int g = 0; g < a.ngroups; ++g) {
    max_cols = a.g[g].N > max_cols ? a.g[g].N : max_cols;
    max_kr = a.g[g].Kr > max_kr ? a.g[g].Kr : max_kr;
  }
  const int nt = lds_nt(max_cols), rw = lds_rows(nt);
  int64_t blocks = 0;
  for (int g = 0; g < a.ngroups; ++g) {
    const GemmGroup& G = a.g[g];
    if (G.M > 0 && G.N > 0 && G.Kr > 0) blocks += (int64_t)ceil_div(ceil_div(G.M, 32), rw) * ceil_div(G.N, 32 * nt);
  }
  const int64_t waves = blocks * rw;
  if (waves < kLdsMinWaves) return 1;  // the reduction-splitting kernel takes it
  const int kc = 2 * (nt <= 2 ? 16 : 8);
  // about four waves per SIMD, every split at least 64 chunks long
  int sp = 1;
  while (sp < 4 && waves * sp < 4096 && max_kr >= 2 * sp * 64 * kc) sp *= 2;
  return sp;
}

hipError_t launch_rows_reduce(int kind, const GemmArgs& a, hipStream_t s) {
  int64_t total = 0;
  for (int g = 0; g < a.ngroups; ++g) total += (int64_t)a.g[g].M * a.g[g].N;
  if (total <= 0 || a.splits <= 1) return hipSuccess;
  if ((total + 255) / 256 > INT32_MAX || !a.part) return hipErrorInvalidValue;
  TimingScope ts(kcGwReduce, s);
  const dim3 grid((unsigned)((total + 255) / 256));
  if (kind == kGemmOut)
    hipLaunchKernelGGL(rows_reduce_kernel<kGemmOut>, grid, dim3(256), 0, s, a, total);
  else if (kind == kGemmGx)
    hipLaunchKernelGGL(rows_reduce_kernel<kGemmGx>, grid, dim3(256), 0, s, a, total);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
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

hipError_t launch_w_planes(const void* W, bool w_bf16, int64_t kp, int C_in, int C_out, uint16_t* hi, uint16_t* lo,
                           uint16_t* thi, uint16_t* tlo, hipStream_t s) {
  const int64_t n = kp * C_in * (int64_t)C_out;
  if (n <= 0) return hipSuccess;
  if (!hi || !thi || (!w_bf16 && (!lo || !tlo)) || (n + 255) / 256 > INT32_MAX) return hipErrorInvalidValue;
  TimingScope ts(kcFill, s);
  hipLaunchKernelGGL(w_planes_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, W, w_bf16 ? 1 : 0, n, C_in,
                     C_out, hi, lo, thi, tlo);
  return hipGetLastError();
}

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  TimingScope ts(kcFill, s);
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace tpconv
