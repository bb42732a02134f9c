// Position gradient of the receiver-side stream, as dense products on the
// matrix cores ("Sobek" page, abstract: the streaming form extends through
// the backward pass; no per-edge adjoint is stored).
//
// For a receiver v with state cotangent gS_v[k, p, c, m3] and an edge e from
// sender s, the position gradient needs
//   gU_e[p,c,m3] = sum_k R_e[k] gS_v[k,p,c,m3],   gD_e = the same with R'_e,
//   alpha_e      = sum <gD_e[p], U_e[p]>,          U_e = CG(x_s, Y_e),
//   gY_e[m2]     = sum C^p[m1,m2,m3] x_s[c,m1] gU_e[p,c,m3],
//   g_r          = alpha_e r_hat + J_Y^T gY_e.
// Contracting the channels first turns the bulk of the work into one product
// per receiver and path bundle (all paths of a bundle share the input irrep
// l1, so they gather the same rows of x):
//   Z[(p,m3,k), (m1,e)] = sum_c gS_v[k,p,c,m3] x_s(e)[l1,c,m1],
// after which only short per-edge sums remain:
//   Q[p,m3,m1] = sum_k R_e[k] Z,  P[p,m3,m1] = sum_k R'_e[k] Z,
//   alpha_e    = sum C^p[m1,m2,m3] Y_e[m2] P,   gY_e[m2] = sum C^p[m1,m2,m3] Q.
// Z runs on v_mfma_f32_16x16x32_bf16 with fp32 accuracy: every fp32 operand
// is split into a bf16 pair hi + lo (hi = x rounded to bf16, lo = x - hi
// rounded again, so hi + lo carries 16 significant bits and the rest is
// below 2^-17 |x|), and a tile is the sum of the products hi*lo', lo*hi' and
// hi*hi' (lo*lo' is below 2^-17 of the product and is dropped), each exact in
// the fp32 accumulator.  Features already stored in bf16 have no lo part
// (two products).  Rows (p, m3, k) of gS_v are the A operand (16 per tile,
// loaded and split once per receiver and kept in registers), columns are 16
// edges for one m1 (the gathered rows of x, pre-split into two bf16 planes:
// the B operand), and the reduction runs over a 32-channel slice (lane group
// g of the wave supplies channels 8g..8g+7 of the slice).  Lane (i, g) then
// holds rows 4g..4g+3 of column i, i.e. four k-values of one (p, m3) for
// edge i: it forms its share of Q and P, applies the coupling with the table
// values as immediates, and its share of g_r; the four lane groups of an
// edge are summed with two lane swaps.
//
// Work decomposition: one block per receiver.  Its waves share the geometry
// of a 64-edge batch (radial basis, R', harmonics and their Jacobian, written
// to LDS once) and each takes its own list of (channel slice, path bundle)
// pairs, balanced by cost on the host since the waves meet at every batch; each
// wave adds its per-edge share of g_r into its own LDS row, and after the
// batch the rows are summed in a fixed order, so the sender's share goes out
// as three fp32 atomic adds per edge.  The receiver's share is summed over
// its edges and added once.
#pragma once

#include <type_traits>
#include <utility>

#include "stream_impl.h"

namespace tpconv {

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>), in order.
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Compile-time view of a bundle's member paths and of its output components
// j = (member path, m3), numbered path by path.
template <class... Ps>
struct PosPack {
  static constexpr int n = sizeof...(Ps);
  static constexpr int L1 = First<Ps...>::type::l1;
  static constexpr int NIN = 2 * L1 + 1;
  static constexpr int l2s[n] = {Ps::l2...};
  static constexpr int l3s[n] = {Ps::l3...};
  static constexpr int TOT = ((2 * Ps::l3 + 1) + ...);
  static constexpr int member_of(int j) {
    int acc = 0;
    for (int q = 0; q < n; ++q) {
      if (j < acc + 2 * l3s[q] + 1) return q;
      acc += 2 * l3s[q] + 1;
    }
    return -1;
  }
  static constexpr int m3_of(int j) {
    int acc = 0;
    for (int q = 0; q < n; ++q) {
      if (j < acc + 2 * l3s[q] + 1) return j - acc;
      acc += 2 * l3s[q] + 1;
    }
    return -1;
  }
  static constexpr bool uses_l2(int l) {
    for (int q = 0; q < n; ++q)
      if (l2s[q] == l) return true;
    return false;
  }
};


constexpr int kPosSlice = 32;       // channels of one wave's reduction range
constexpr int kPosNcl = kPosSlice / 4;  // channels per lane group (8 bf16 of one MFMA operand)
constexpr int kPosMaxWaves = kPosMaxBlockWaves;  // waves per block
constexpr int kPosBatch = 64;       // edges whose geometry is in LDS at a time

// Batch geometry of the position derivative of the force loss (HESS): what
// the position gradient uses plus R'', the tangent phi = gg_pos[s] - gg_pos[v]
// (with 1/d in its fourth entry) and the directional Hessians (d^2 Y / dr^2) phi.
template <int K, int LMAX>
struct __attribute__((aligned(16))) HessLds {
  static constexpr int B = kPosBatch;
  static constexpr int NSH = sh_count(LMAX);
  int nbr[B];
  float R[B][K];
  float Rd[B][K];
  float Rdd[B][K];
  float Y[B][LMAX + 1][8];
  float J[B][NSH][4];
  float HYp[B][NSH][4];
  float rhat[B][4];
  float phi[B][4];
};

// The batch geometry in static LDS; each wave's share of the per-edge vector,
// gr[w][e][3], in dynamic LDS sized by the block's wave count.
template <int K, int LMAX, bool HESS>
struct PosLds {
  typename std::conditional<HESS, HessLds<K, LMAX>, EdgeLds<K, LMAX, kBwdPos, kPosBatch>>::type geo;
};
typedef float PosRow[kPosBatch][3];

// Geometry of edge e into slot j for the position derivative of the force loss.
//   HY phi = d^-2 [H_P(u) phi - l grad P(u) (u.phi) - l u (grad P(u).phi) - l P(u) (phi - (l+2) (u.phi) u)]
// (Y = P(r) / |r|^l, with P homogeneous of degree l evaluated at u = r / d).
template <int LMAX, int K>
__device__ __forceinline__ void edge_prep_hess(const StreamArgs& a, int self, float psx, float psy, float psz, int e,
                                               int j, HessLds<K, LMAX>& L) {
  constexpr int NSH = sh_count(LMAX);
  const int nb = a.nbr[e];
  const float rx = a.pos[3 * (int64_t)nb] - psx, ry = a.pos[3 * (int64_t)nb + 1] - psy,
              rz = a.pos[3 * (int64_t)nb + 2] - psz;
  const float d = sqrtf(rx * rx + ry * ry + rz * rz);
  float ux = 0.f, uy = 0.f, uz = 0.f, inv_d = 0.f;
  if (d > 0.f) {
    inv_d = 1.f / d;
    ux = rx * inv_d;
    uy = ry * inv_d;
    uz = rz * inv_d;
  }
  float R[K], dR[K], d2R[K];
  radial2<K>(d, a.inv_cutoff, a.pref, a.env_p, a.env_a, a.env_b, a.env_c, a.env_d, R, dR, d2R);
  if (a.mlp) mlp_radial<K, 2>(a.mlp, -1, R, dR, d2R);
  float Y[NSH], G[NSH][3], HP[NSH][3];
  sh_eval<LMAX>(ux, uy, uz, Y);
  sh_poly_grad<LMAX>(ux, uy, uz, G);
  const float fx = a.ggpos[3 * (int64_t)nb] - a.ggpos[3 * (int64_t)self];
  const float fy = a.ggpos[3 * (int64_t)nb + 1] - a.ggpos[3 * (int64_t)self + 1];
  const float fz = a.ggpos[3 * (int64_t)nb + 2] - a.ggpos[3 * (int64_t)self + 2];
  sh_poly_hess_dir<LMAX>(ux, uy, uz, fx, fy, fz, HP);
  const float uphi = ux * fx + uy * fy + uz * fz;
  const float uu[3] = {ux, uy, uz}, ff[3] = {fx, fy, fz};
  L.nbr[j] = nb;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    L.R[j][k] = R[k];
    L.Rd[j][k] = dR[k];
    L.Rdd[j][k] = d2R[k];
  }
  const float inv_d2 = inv_d * inv_d;
#pragma unroll
  for (int i = 0; i < NSH; ++i) {
    const int li = sh_degree_of_row(i);
    const float l = (float)li;
    L.Y[j][li][i - li * li] = Y[i];
    const float gphi = G[i][0] * fx + G[i][1] * fy + G[i][2] * fz;
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      L.J[j][i][c] = (G[i][c] - l * Y[i] * uu[c]) * inv_d;
      L.HYp[j][i][c] = (HP[i][c] - l * G[i][c] * uphi - l * uu[c] * gphi -
                        l * Y[i] * (ff[c] - (l + 2.f) * uphi * uu[c])) * inv_d2;
    }
  }
  L.rhat[j][0] = ux;
  L.rhat[j][1] = uy;
  L.rhat[j][2] = uz;
  L.phi[j][0] = fx;
  L.phi[j][1] = fy;
  L.phi[j][2] = fz;
  L.phi[j][3] = inv_d;
}

// Eight consecutive bf16 values p[c0 .. c0+8) as one MFMA operand (a 16-byte
// load when `vec`; otherwise each value on its own, clamped into the row: a
// channel past C meets a zero A entry, so any finite value will do).
__device__ __forceinline__ u32x4 load_bf16x8(const uint16_t* p, int c0, int C, bool vec) {
  if (vec) return *reinterpret_cast<const u32x4*>(p + c0);
  u32x4 v;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    v[t] = (uint32_t)p[min(c0 + 2 * t, C - 1)] | ((uint32_t)p[min(c0 + 2 * t + 1, C - 1)] << 16);
  return v;
}

// hi / lo bf16 split of eight fp32 values (hardware round to nearest even).
__device__ __forceinline__ void split_bf16x8(const float (&v)[kPosNcl], u32x4& hi, u32x4& lo) {
  bf16x8 h, l;
#pragma unroll
  for (int t = 0; t < kPosNcl; ++t) {
    h[t] = (__bf16)v[t];
    l[t] = (__bf16)(v[t] - (float)h[t]);
  }
  hi = __builtin_bit_cast(u32x4, h);
  lo = __builtin_bit_cast(u32x4, l);
}

__device__ __forceinline__ floatx4 mfma_bf16(u32x4 a, u32x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// LO: the gathered features have a lo plane (fp32 features, pre-split);
// without it they are bf16 values used as stored.  VEC: C is a multiple of
// the slice, so every operand is one aligned 16-byte (or two) load.  HESS:
// the per-edge vector is H_e phi_e (the position derivative of the force
// loss) instead of g_r.
template <int LMAX, int K, bool LO, bool VEC, bool HESS>
struct PosWave {
  static constexpr int NSH = (LMAX + 1) * (LMAX + 1);

  // kPosNcl consecutive fp32 values (vector loads when `vec`, else clamped).
  __device__ __forceinline__ static void load8(const float* p, int c0, int C, bool vec, float (&v)[kPosNcl]) {
    if (vec) {
      const floatx4 u0 = *reinterpret_cast<const floatx4*>(p + c0);
      const floatx4 u1 = *reinterpret_cast<const floatx4*>(p + c0 + 4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[t] = u0[t];
        v[4 + t] = u1[t];
      }
    } else {
#pragma unroll
      for (int t = 0; t < kPosNcl; ++t) v[t] = p[min(c0 + t, C - 1)];
    }
  }
  __device__ __forceinline__ static void load8(const uint16_t* p, int c0, int C, bool vec, float (&v)[kPosNcl]) {
    const u32x4 u = load_bf16x8(p, c0, C, vec);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[2 * t] = __uint_as_float(u[t] << 16);
      v[2 * t + 1] = __uint_as_float(u[t] & 0xffff0000u);
    }
  }

  // Rows 16 T + i of the bundle's A operand: gS_v[k, p, c, m3] for
  // j = (p, m3) = row / K, k = row % K, channels c0..c0+7 (zero past C and for
  // padding rows), split into bf16 hi and lo.  Channel-wise weights:
  // gS = W[k, p, c] grad_out[v][m3 row][c].
  template <class PK>
  __device__ __forceinline__ static void load_a(const StreamArgs& a, int unit, int node, int row, int c0, u32x4& hi,
                                                u32x4& lo) {
    const int j = row / K, k = row % K;
    int I = -1, m3 = 0, acc = 0;
#pragma unroll
    for (int q = 0; q < PK::n; ++q) {
      const int no = 2 * PK::l3s[q] + 1;
      if (j >= acc && j < acc + no) {
        I = q;
        m3 = j - acc;
      }
      acc += no;
    }
    const int C = a.C;
    float A[kPosNcl];
    if (I < 0) {
#pragma unroll
      for (int t = 0; t < kPosNcl; ++t) A[t] = 0.f;
    } else {
      const StreamPath& Q = a.paths[a.unit_paths[unit][I]];
      constexpr bool vec = VEC;
      if (a.cw) {
        const int64_t wrow = ((int64_t)k * a.npaths + Q.path) * C;
        const float* go = a.gout + ((int64_t)node * a.gout_rows + Q.out_row + m3) * C;
        float gv[kPosNcl], wv[kPosNcl];
        load8(go, c0, C, vec, gv);
        if (a.w_bf16)
          load8(static_cast<const uint16_t*>(a.W) + wrow, c0, C, vec, wv);
        else
          load8(static_cast<const float*>(a.W) + wrow, c0, C, vec, wv);
#pragma unroll
        for (int t = 0; t < kPosNcl; ++t) A[t] = wv[t] * gv[t];
      } else {
        const int no = 2 * Q.l3 + 1;
        const float* p = a.gstate + Q.state_base + ((int64_t)(node * no + m3) * K + k) * Q.cols_per_k + Q.q * C;
        load8(p, c0, C, vec, A);
      }
#pragma unroll
      for (int t = 0; t < kPosNcl; ++t) A[t] = c0 + t < C ? A[t] : 0.f;
    }
    split_bf16x8(A, hi, lo);
  }

  // HESS: one component J with the tile's fixed m1 adds its shares of
  // A_i[m2] = sum_k R^(i)_k b_k[m2] (i = 0, 1, 2: R, R', R'') with
  // b_k[m2] = sum C^p[m1,m2,m3] Z[(p,m3,k),(m1,e)].
  template <class PK, int J, int M1>
  __device__ __forceinline__ static void couple3(float q0, float q1, float q2, float (&A0)[NSH], float (&A1)[NSH],
                                                 float (&A2)[NSH]) {
    if constexpr (J < PK::TOT) {
      constexpr int I = PK::member_of(J), M3 = PK::m3_of(J);
      constexpr int L1 = PK::L1, L2 = PK::l2s[I], L3 = PK::l3s[I];
      static_for<2 * L2 + 1>([&](auto M2) {
        constexpr float c = cg_coef(L1, L2, L3, M1, decltype(M2)::value, M3);
        constexpr int row = L2 * L2 + decltype(M2)::value;
        if constexpr (c != 0.f) {
          A0[row] = __builtin_fmaf(c, q0, A0[row]);
          A1[row] = __builtin_fmaf(c, q1, A1[row]);
          A2[row] = __builtin_fmaf(c, q2, A2[row]);
        }
      });
    }
  }

  // One component J = (member path, m3) with the tile's fixed m1: the share
  // q (of Q) and pd (of P) of this lane enter alpha and gY.
  template <class PK, int J, int M1, int NY>
  __device__ __forceinline__ static void couple(float q, float pd, const float (&y)[NY][2 * LMAX + 1], float& alpha,
                                                float (&gy)[NSH]) {
    if constexpr (J < PK::TOT) {
      constexpr int I = PK::member_of(J), M3 = PK::m3_of(J);
      constexpr int L1 = PK::L1, L2 = PK::l2s[I], L3 = PK::l3s[I];
      float yd = 0.f;
      static_for<2 * L2 + 1>([&](auto M2) {
        constexpr float c = cg_coef(L1, L2, L3, M1, decltype(M2)::value, M3);
        if constexpr (c != 0.f) {
          yd = __builtin_fmaf(c, y[L2][decltype(M2)::value], yd);
          gy[L2 * L2 + decltype(M2)::value] = __builtin_fmaf(c, q, gy[L2 * L2 + decltype(M2)::value]);
        }
      });
      alpha = __builtin_fmaf(pd, yd, alpha);
    }
  }

  // One (channel slice, bundle) pair over the batch in LDS: adds this wave's
  // share of g_r for every edge of the batch to gr[w][e].
  template <class... Ps>
  __device__ __forceinline__ static void run(const StreamArgs& a, int unit, int node, int slice, int nb,
                                             PosLds<K, LMAX, HESS>& S, float (&gr)[kPosBatch][3]) {
    using PK = PosPack<Ps...>;
    constexpr int NIN = PK::NIN;
    constexpr int TILES = (K * PK::TOT + 15) / 16;
    const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
    const int C = a.C;
    const int c0 = slice * kPosSlice + g * kPosNcl;
    constexpr bool vec = VEC;
    // this lane's four k of its rows: 4 (g % 2) .. (K = 8) or 4 g .. (K = 16)
    const int kb = K == 8 ? 4 * (g & 1) : 4 * g;
    const bool upper = g >= 2;  // K = 8: the lane's rows belong to the tile's second component

    u32x4 Ah[TILES], Al[TILES];
    static_for<TILES>([&](auto T) { load_a<PK>(a, unit, node, 16 * decltype(T)::value + i, c0, Ah[T], Al[T]); });

    const uint16_t* fhi = static_cast<const uint16_t*>(a.feat);
    const uint16_t* flo = static_cast<const uint16_t*>(a.feat_lo);
    const int64_t frow = a.paths[a.unit_paths[unit][0]].feat_row;
    auto gather = [&](int t, int m1, u32x4& vh, u32x4& vl) {
      const int e = min(t * 16 + i, nb - 1);
      const int64_t off = ((int64_t)S.geo.nbr[e] * a.feat_rows + frow + m1) * a.feat_cs;
      vh = load_bf16x8(fhi + off, c0, C, vec);
      if constexpr (LO) vl = load_bf16x8(flo + off, c0, C, vec);
    };
    const int ntiles = (nb + 15) >> 4;
    // one step (tile, m1) of gathered rows in flight ahead of its use
    u32x4 xh, xl;
    gather(0, 0, xh, xl);

    for (int t = 0; t < ntiles; ++t) {
      const int e = t * 16 + i;
      const int ee = min(e, nb - 1);
      float r4[4], rd4[4], rdd4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        r4[r] = S.geo.R[ee][kb + r];
        rd4[r] = S.geo.Rd[ee][kb + r];
        if constexpr (HESS) rdd4[r] = S.geo.Rdd[ee][kb + r];
      }
      float y[LMAX + 1][2 * LMAX + 1];
#pragma unroll
      for (int l = 0; l <= LMAX; ++l)
#pragma unroll
        for (int m = 0; m < 2 * LMAX + 1; ++m) y[l][m] = (m <= 2 * l && PK::uses_l2(l)) ? S.geo.Y[ee][l][m] : 0.f;
      float alpha = 0.f, gy[NSH], A1[HESS ? NSH : 1], A2[HESS ? NSH : 1];
#pragma unroll
      for (int r = 0; r < NSH; ++r) gy[r] = 0.f;
      if constexpr (HESS) {
#pragma unroll
        for (int r = 0; r < NSH; ++r) A1[r] = A2[r] = 0.f;
      }
      const int tn = min(t + 1, ntiles - 1);
      static_for<NIN>([&](auto M1c) {
        constexpr int M1 = decltype(M1c)::value;
        const u32x4 bh = xh, bl = xl;
        if constexpr (M1 + 1 < NIN)
          gather(t, M1 + 1, xh, xl);  // the next step's rows, in flight during this step
        else
          gather(tn, 0, xh, xl);
        floatx4 acc[TILES];
#pragma unroll
        for (int T = 0; T < TILES; ++T) {
          acc[T] = mfma_bf16(Al[T], bh, floatx4{0.f, 0.f, 0.f, 0.f});
          if constexpr (LO) acc[T] = mfma_bf16(Ah[T], bl, acc[T]);
          acc[T] = mfma_bf16(Ah[T], bh, acc[T]);
        }
        static_for<TILES>([&](auto Tc) {
          constexpr int T = decltype(Tc)::value;
          float q = 0.f, pd = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            q = __builtin_fmaf(r4[r], acc[T][r], q);
            pd = __builtin_fmaf(rd4[r], acc[T][r], pd);
          }
          if constexpr (HESS) {  // gy holds A0 = sum_k R_k b_k
            float q2 = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) q2 = __builtin_fmaf(rdd4[r], acc[T][r], q2);
            if constexpr (K == 16) {
              couple3<PK, T, M1>(q, pd, q2, gy, A1, A2);
            } else {
              couple3<PK, 2 * T, M1>(upper ? 0.f : q, upper ? 0.f : pd, upper ? 0.f : q2, gy, A1, A2);
              couple3<PK, 2 * T + 1, M1>(upper ? q : 0.f, upper ? pd : 0.f, upper ? q2 : 0.f, gy, A1, A2);
            }
          } else if constexpr (K == 16) {
            couple<PK, T, M1>(q, pd, y, alpha, gy);
          } else {
            couple<PK, 2 * T, M1>(upper ? 0.f : q, upper ? 0.f : pd, y, alpha, gy);
            couple<PK, 2 * T + 1, M1>(upper ? q : 0.f, upper ? pd : 0.f, y, alpha, gy);
          }
        });
        // The step's coupling must land in alpha / gY here: left alone, the
        // compiler sinks every step's couplings to the end of the tile, which
        // keeps all of their Q and P values live at once.
        asm volatile("" : "+v"(alpha));
#pragma unroll
        for (int r = 0; r < NSH; ++r) asm volatile("" : "+v"(gy[r]));
        if constexpr (HESS) {
#pragma unroll
          for (int r = 0; r < NSH; ++r) asm volatile("" : "+v"(A1[r]), "+v"(A2[r]));
        }
      });
      float vec3[3];
      if constexpr (HESS) {
        // this lane's share of H_e phi = a2 (r.phi) r + a1 (phi - (r.phi) r) / d + r (J^T A1 . phi)
        //   + (r.phi) J^T A1 + sum A0[m] (HY_m phi),  a_i = A_i . Y
        float a1 = 0.f, a2 = 0.f, jb[3] = {0.f, 0.f, 0.f}, hy[3] = {0.f, 0.f, 0.f};
#pragma unroll
        for (int l = 0; l <= LMAX; ++l) {
          if (!PK::uses_l2(l)) continue;
#pragma unroll
          for (int m = 0; m < 2 * l + 1; ++m) {
            const int row = l * l + m;
            const float yv = S.geo.Y[ee][l][m];
            a1 = __builtin_fmaf(A1[row], yv, a1);
            a2 = __builtin_fmaf(A2[row], yv, a2);
#pragma unroll
            for (int cc = 0; cc < 3; ++cc) {
              jb[cc] = __builtin_fmaf(A1[row], S.geo.J[ee][row][cc], jb[cc]);
              hy[cc] = __builtin_fmaf(gy[row], S.geo.HYp[ee][row][cc], hy[cc]);
            }
          }
        }
        const float ph[3] = {S.geo.phi[ee][0], S.geo.phi[ee][1], S.geo.phi[ee][2]};
        const float inv_d = S.geo.phi[ee][3];
        const float rh[3] = {S.geo.rhat[ee][0], S.geo.rhat[ee][1], S.geo.rhat[ee][2]};
        const float rphi = rh[0] * ph[0] + rh[1] * ph[1] + rh[2] * ph[2];
        const float jphi = jb[0] * ph[0] + jb[1] * ph[1] + jb[2] * ph[2];
#pragma unroll
        for (int cc = 0; cc < 3; ++cc)
          vec3[cc] = a2 * rphi * rh[cc] + a1 * inv_d * (ph[cc] - rphi * rh[cc]) + rh[cc] * jphi + rphi * jb[cc] + hy[cc];
      } else {
        // this lane's share of g_r = alpha r_hat + J^T gY (harmonic degrees the bundle uses)
#pragma unroll
        for (int cc = 0; cc < 3; ++cc) vec3[cc] = alpha * S.geo.rhat[ee][cc];
#pragma unroll
        for (int l = 1; l <= LMAX; ++l) {
          if (!PK::uses_l2(l)) continue;
#pragma unroll
          for (int m = 0; m < 2 * l + 1; ++m)
#pragma unroll
            for (int cc = 0; cc < 3; ++cc)
              vec3[cc] = __builtin_fmaf(gy[l * l + m], S.geo.J[ee][l * l + m][cc], vec3[cc]);
        }
      }
#pragma unroll
      for (int cc = 0; cc < 3; ++cc) vec3[cc] = half32_add(row16_add(vec3[cc]));
      if (g == 0 && e < nb) {
#pragma unroll
        for (int cc = 0; cc < 3; ++cc) gr[e][cc] += vec3[cc];
      }
    }
  }
};

// A bundle (BUNDLED) or single-path unit for the position gradient.
template <int LMAX, int K, bool LO, bool VEC, bool HESS>
struct PosUnitRunner {
  const StreamArgs& a;
  int unit, node, slice, nb;
  PosLds<K, LMAX, HESS>& S;
  float (&gr)[kPosBatch][3];
  template <class... Ps>
  __device__ __forceinline__ void run(const StreamArgs&) {
    PosWave<LMAX, K, LO, VEC, HESS>::template run<Ps...>(a, unit, node, slice, nb, S, gr);
  }
};

// Waves per SIMD the register allocation must leave room for (lmax 3 with
// K = 8, and lmax 3 for the Hessian, need more than the 168 registers of three).
constexpr int pos_min_waves(int lmax, int K, bool hess) {
  return lmax <= 1 ? 4 : (lmax == 3 && (K == 8 || hess) ? 2 : 3);
}

template <int LMAX, int K, bool LO, bool VEC, bool BUNDLED, bool HESS>
__global__ __launch_bounds__(64 * kPosMaxWaves) __attribute__((amdgpu_waves_per_eu(pos_min_waves(LMAX, K, HESS))))
void pos_kernel(const StreamArgs /*args*/, int64_t nodes) {
  const StreamArgs& a = *(const StreamArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  __shared__ PosLds<K, LMAX, HESS> S;
  extern __shared__ float pos_rows[];
  PosRow* gr = reinterpret_cast<PosRow*>(pos_rows);
  const uint32_t item = (uint32_t)xcd_item(blockIdx.x, gridDim.x);
  if (item >= (uint32_t)nodes) return;  // uniform over the block
  const int node = a.order ? a.order[item] : (int)item;
  const int nw = (int)(blockDim.x >> 6);
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int npairs = a.nunits * a.nslices;
  const float psx = a.pos[3 * (int64_t)node], psy = a.pos[3 * (int64_t)node + 1], psz = a.pos[3 * (int64_t)node + 2];
  const int e0 = a.ptr[node], e1 = a.ptr[node + 1];
  float vs0 = 0.f, vs1 = 0.f, vs2 = 0.f;  // receiver share (wave 0, one edge per lane)
  for (int b0 = e0; b0 < e1; b0 += kPosBatch) {
    const int nb = min(kPosBatch, e1 - b0);
    __syncthreads();
    if ((int)threadIdx.x < nb) {
      if constexpr (HESS)
        edge_prep_hess(a, node, psx, psy, psz, b0 + (int)threadIdx.x, (int)threadIdx.x, S.geo);
      else
        edge_prep(a, node, psx, psy, psz, b0 + (int)threadIdx.x, (int)threadIdx.x, S.geo);
    }
#pragma unroll
    for (int cc = 0; cc < 3; ++cc) gr[w][lane][cc] = 0.f;
    __syncthreads();
    for (int k = a.pair_begin[w]; k < a.pair_begin[w + 1]; ++k) {
      const int pr = a.pair_order[k];
      const int unit = pr % a.nunits, slice = pr / a.nunits;
      PosUnitRunner<LMAX, K, LO, VEC, HESS> run{a, unit, node, slice, nb, S, gr[w]};
      if constexpr (BUNDLED) {
        Bundles<LMAX, K, 2>::run(unit, run, a);
      } else {
        const StreamPath& P = a.paths[a.unit_paths[unit][0]];
        switch (P.l1 * 16 + P.l2 * 4 + P.l3) {
#define TPCONV_CASE(A_, B_, C_)                          \
  case A_ * 16 + B_ * 4 + C_:                            \
    if constexpr (A_ <= LMAX && B_ <= LMAX && C_ <= LMAX) \
      run.template run<P3<A_, B_, C_>>(a);               \
    break;
          TPCONV_PATH_CASES(TPCONV_CASE)
#undef TPCONV_CASE
          default:
            break;
        }
      }
    }
    __syncthreads();
    if (w == 0 && lane < nb) {  // fixed-order sum over the waves, then the sender's share (+) and the receiver's (-)
      float v0 = 0.f, v1 = 0.f, v2 = 0.f;
      for (int ww = 0; ww < nw; ++ww) {
        v0 += gr[ww][lane][0];
        v1 += gr[ww][lane][1];
        v2 += gr[ww][lane][2];
      }
      const int64_t s3 = 3 * (int64_t)S.geo.nbr[lane];
      if (a.gpos_fx) {
        const int F = *a.fx_shift;
        atomicAdd(&a.gpos_fx[s3 + 0], to_fixed(v0, F));
        atomicAdd(&a.gpos_fx[s3 + 1], to_fixed(v1, F));
        atomicAdd(&a.gpos_fx[s3 + 2], to_fixed(v2, F));
      } else {
        atomicAdd(&a.gpos[s3 + 0], v0);
        atomicAdd(&a.gpos[s3 + 1], v1);
        atomicAdd(&a.gpos[s3 + 2], v2);
      }
      vs0 -= v0;
      vs1 -= v1;
      vs2 -= v2;
    }
  }
  if (w == 0) {
    vs0 = channel_sum(vs0, 6);
    vs1 = channel_sum(vs1, 6);
    vs2 = channel_sum(vs2, 6);
    if (lane == 0 && e1 > e0) {
      if (a.gpos_fx) {
        const int F = *a.fx_shift;
        atomicAdd(&a.gpos_fx[3 * (int64_t)node + 0], to_fixed(vs0, F));
        atomicAdd(&a.gpos_fx[3 * (int64_t)node + 1], to_fixed(vs1, F));
        atomicAdd(&a.gpos_fx[3 * (int64_t)node + 2], to_fixed(vs2, F));
      } else {
        atomicAdd(&a.gpos[3 * (int64_t)node + 0], vs0);
        atomicAdd(&a.gpos[3 * (int64_t)node + 1], vs1);
        atomicAdd(&a.gpos[3 * (int64_t)node + 2], vs2);
      }
    }
  }
}

// LO: the features are fp32, pre-split into the bf16 planes a.feat (hi) and
// a.feat_lo (lo); otherwise a.feat holds them in bf16.
template <bool LO, bool HESS>
hipError_t launch_pos(int lmax, int K, const StreamArgs& a, hipStream_t s) {
  if (LO != (a.feat_lo != nullptr)) return hipErrorInvalidValue;
  const int64_t nodes = a.num_nodes;
  const int npairs = a.nunits * a.nslices;
  if (nodes == 0 || npairs == 0) return hipSuccess;
  const int64_t grid = (nodes + 7) / 8 * 8;
  if (grid > INT32_MAX || a.pos_waves < 1 || a.pos_waves > kPosMaxWaves || a.pair_begin[0] != 0 ||
      a.pair_begin[a.pos_waves] != npairs)
    return hipErrorInvalidValue;
  const dim3 block(64 * a.pos_waves);
  const size_t rows = sizeof(PosRow) * (size_t)a.pos_waves;
  // 16-byte operand loads: whole slices, 16-byte aligned feature and state rows
  const bool vec = a.C % kPosSlice == 0 && a.feat_cs == a.C && (reinterpret_cast<uintptr_t>(a.feat) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.feat_lo) & 15) == 0;
#define TPCONV_LAUNCH(LM, KK)                                                                                      \
  if (lmax == LM && K == KK) {                                                                                     \
    if (vec && a.bundled)                                                                                          \
      hipLaunchKernelGGL((pos_kernel<LM, KK, LO, true, true, HESS>), dim3((unsigned)grid), block, rows, s, a, nodes);      \
    else if (vec)                                                                                                  \
      hipLaunchKernelGGL((pos_kernel<LM, KK, LO, true, false, HESS>), dim3((unsigned)grid), block, rows, s, a, nodes);     \
    else if (a.bundled)                                                                                            \
      hipLaunchKernelGGL((pos_kernel<LM, KK, LO, false, true, HESS>), dim3((unsigned)grid), block, rows, s, a, nodes);     \
    else                                                                                                           \
      hipLaunchKernelGGL((pos_kernel<LM, KK, LO, false, false, HESS>), dim3((unsigned)grid), block, rows, s, a, nodes);    \
    return hipGetLastError();                                                                                      \
  }
  TPCONV_LAUNCH(0, 8) TPCONV_LAUNCH(0, 16)
  TPCONV_LAUNCH(1, 8) TPCONV_LAUNCH(1, 16)
  TPCONV_LAUNCH(2, 8) TPCONV_LAUNCH(2, 16)
  TPCONV_LAUNCH(3, 8) TPCONV_LAUNCH(3, 16)
#undef TPCONV_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace tpconv
