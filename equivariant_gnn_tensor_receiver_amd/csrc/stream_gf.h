// Accumulating edge streams as dense products per node on the matrix cores
// ("Sobek" page, abstract: edge-local products are consumed straight into a
// bounded receiver-side state; the same schedule, mirrored, gives the sender
// state of the backward pass and the tangent states of the double backward).
//
// For a node v and a unit of paths that gather the same feature block, the
// receiver state is
//   S_v[k, p, c, m3] = sum_e R_e[k] sum_m1 g_e[p, m1, m3] x_s(e)[c, m1],
//   g_e[p, m1, m3]   = sum_m2 C^p[m1, m2, m3] Y_e[l2, m2],
// so for each m1 it grows by one dense product over the node's edges,
//   S^T[(p, m3, k), c] += sum_e A[(p, m3, k), e] X[e, c],
//   A[(p, m3, k), e] = R_e[k] g_e[p, m1, m3],   X[e, c] = x_s(e)[c, m1].
// The sender state T_s[k, p, c, m1] is the same product with m1 and m3
// exchanged (gathered rows of grad_out, reduction over their m3), and the
// tangent states use A = R_dot g(Y) + R g(Y_dot).  Nothing edge-sized leaves
// the registers and LDS of the wave.
//
// The products run on v_mfma_f32_16x16x32_bf16 at fp32 accuracy: A is split
// into bf16 hi + lo in registers as it is formed (hi = A rounded to bf16,
// lo = A - hi rounded again), the gathered features come pre-split into two
// bf16 planes (or are bf16 already, without a lo plane), and a tile is the sum
// hi*hi' + hi*lo' + lo*hi', each product exact in the fp32 accumulator.  Lane
// (i, g) supplies A row i at edges 8g..8g+7 and X column (channel) i at the
// same edges, and receives accumulator rows 4g..4g+3 of column i.
//
// Work decomposition: one wave per (node, unit, 32-channel slice).  The
// node's edges come in batches of 64: lane e computes the geometry of edge e
// (radial basis and harmonics, for tangents also their derivatives along the
// tangent) and, for each gathered row m1 in turn, the coupling values g_e of
// every output component of the unit, into wave-private LDS.  Each batch is
// two 32-edge reduction steps per m1.  The state tile (K * TOT rows by 32
// channels) stays in registers over all batches and is written once; no
// atomics.
#pragma once

#include <type_traits>

#include "stream_pos.h"

namespace tpconv {

constexpr int kGfBatch = 64;              // edges whose geometry is in LDS at a time
constexpr int kGfStride = kGfBatch + 4;   // row stride of the per-edge LDS tables (spreads the banks)
constexpr int kGfMaxTot = 16;             // output components of a unit (K * TOT <= 128 rows)
constexpr int kGfSlice = 32;              // channels of one wave (two 16-column tiles)

template <int K, bool TAN>
struct __attribute__((aligned(16))) GfLds {
  uint32_t noff[kGfBatch];                  // byte offset of each slot's neighbour in the planes (past the batch: the node's)
  float R[K][kGfStride];                    // R_e[k] (tangents: R_dot), 0 past the batch
  float Rt[TAN ? K : 1][kGfStride];         // tangents: R_e[k]
  float g[kGfMaxTot + 1][kGfStride];        // g_e of the current gathered row; row kGfMaxTot stays 0
  float gd[TAN ? kGfMaxTot + 1 : 1][kGfStride];  // tangents: the same with Y_dot
};

// Compile-time view of a unit: its member paths, the degree of the gathered
// block and its output components j = (member, o), numbered member by member
// (o = m3 on the receiver side, m1 on the sender side).
template <bool RECV, class... Ps>
struct GfPack {
  static constexpr int n = sizeof...(Ps);
  static constexpr int l1s[n] = {Ps::l1...};
  static constexpr int l2s[n] = {Ps::l2...};
  static constexpr int l3s[n] = {Ps::l3...};
  static constexpr int LG = RECV ? First<Ps...>::type::l1 : First<Ps...>::type::l3;
  static constexpr int NIN = 2 * LG + 1;
  static constexpr int nout(int q) { return RECV ? 2 * l3s[q] + 1 : 2 * l1s[q] + 1; }
  static constexpr int TOT = ((RECV ? 2 * Ps::l3 + 1 : 2 * Ps::l1 + 1) + ...);
  static constexpr int member_of(int j) {
    int acc = 0;
    for (int q = 0; q < n; ++q) {
      if (j < acc + nout(q)) return q;
      acc += nout(q);
    }
    return -1;
  }
  static constexpr int o_of(int j) {
    int acc = 0;
    for (int q = 0; q < n; ++q) {
      if (j < acc + nout(q)) return j - acc;
      acc += nout(q);
    }
    return -1;
  }
};

// Wave-level LDS ordering: the lanes of one wave exchange values through its
// private LDS region; LDS operations of a wave execute in order, so only the
// compiler must keep them in program order.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LO: the gathered features have a lo plane (fp32 split into a.feat = hi and
// a.feat_lo = lo); otherwise a.feat holds the bf16 values.  Both come with a
// channel stride a.feat_cs that is a multiple of the slice (zero-padded), so
// every 32-bit channel-pair load is aligned and inside its row.
template <int LMAX, int K, int MODE, bool LO>
struct GfWave {
  static constexpr bool RECV = ModeTraits<MODE>::recv;
  static constexpr bool TAN = ModeTraits<MODE>::tangent;
  static constexpr int NSH = sh_count(LMAX);

  // Geometry of slot e of the batch starting at edge b0 (nb edges): LDS
  // tables and this lane's harmonics (and their tangent derivatives).
  __device__ __forceinline__ static void prep(const StreamArgs& a, int node, float psx, float psy, float psz,
                                              int b0, int nb, int e, uint32_t nodebytes, GfLds<K, TAN>& L,
                                              float (&y)[NSH], float (&yd)[TAN ? NSH : 1]) {
    if (e < nb) {
      const int nbr = a.nbr[b0 + e];
      const float qx = a.pos[3 * (int64_t)nbr], qy = a.pos[3 * (int64_t)nbr + 1], qz = a.pos[3 * (int64_t)nbr + 2];
      // r = pos[sender] - pos[receiver]
      const float rx = RECV ? qx - psx : psx - qx;
      const float ry = RECV ? qy - psy : psy - qy;
      const float rz = RECV ? qz - psz : psz - qz;
      const float d = sqrtf(rx * rx + ry * ry + rz * rz);
      float ux = 0.f, uy = 0.f, uz = 0.f, inv_d = 0.f;
      if (d > 0.f) {
        inv_d = 1.f / d;
        ux = rx * inv_d;
        uy = ry * inv_d;
        uz = rz * inv_d;
      }
      float R[K], dR[K];
      radial<K, TAN>(d, a.cutoff, a.inv_cutoff, a.pref, a.env_p, a.env_a, a.env_b, a.env_c, a.env_d, R, dR);
      if (a.mlp) mlp_radial<K, TAN ? 1 : 0>(a.mlp, a.mlp_col, R, dR, nullptr);
      sh_eval<LMAX>(ux, uy, uz, y);
      L.noff[e] = (uint32_t)nbr * nodebytes;
      if constexpr (TAN) {
        float G[NSH][3];
        sh_poly_grad<LMAX>(ux, uy, uz, G);
        const int s = RECV ? nbr : node, v = RECV ? node : nbr;
        const float fx = a.ggpos[3 * (int64_t)s] - a.ggpos[3 * (int64_t)v];
        const float fy = a.ggpos[3 * (int64_t)s + 1] - a.ggpos[3 * (int64_t)v + 1];
        const float fz = a.ggpos[3 * (int64_t)s + 2] - a.ggpos[3 * (int64_t)v + 2];
        const float rphi = ux * fx + uy * fy + uz * fz;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          L.R[k][e] = dR[k] * rphi;
          L.Rt[k][e] = R[k];
        }
#pragma unroll
        for (int r = 0; r < NSH; ++r)
          yd[r] = (G[r][0] * fx + G[r][1] * fy + G[r][2] * fz - (float)sh_degree_of_row(r) * y[r] * rphi) * inv_d;
      } else {
#pragma unroll
        for (int k = 0; k < K; ++k) L.R[k][e] = R[k];
      }
    } else {
      L.noff[e] = (uint32_t)node * nodebytes;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        L.R[k][e] = 0.f;
        if constexpr (TAN) L.Rt[k][e] = 0.f;
      }
#pragma unroll
      for (int r = 0; r < NSH; ++r) {
        y[r] = 0.f;
        if constexpr (TAN) yd[r] = 0.f;
      }
    }
  }

  // Coupling values of gathered row G for every output component of the unit
  // at this lane's edge slot e.
  template <class PK, int G>
  __device__ __forceinline__ static void couple_table(const float (&y)[NSH], const float (&yd)[TAN ? NSH : 1], int e,
                                                      GfLds<K, TAN>& L) {
    static_for<PK::TOT>([&](auto Jc) {
      constexpr int J = decltype(Jc)::value;
      constexpr int q = PK::member_of(J), o = PK::o_of(J);
      constexpr int L1 = PK::l1s[q], L2 = PK::l2s[q], L3 = PK::l3s[q];
      float v = 0.f, vd = 0.f;
      static_for<2 * L2 + 1>([&](auto M2c) {
        constexpr int M2 = decltype(M2c)::value;
        constexpr float c = RECV ? cg_coef(L1, L2, L3, G, M2, o) : cg_coef(L1, L2, L3, o, M2, G);
        if constexpr (c != 0.f) {
          v = __builtin_fmaf(c, y[L2 * L2 + M2], v);
          if constexpr (TAN) vd = __builtin_fmaf(c, yd[L2 * L2 + M2], vd);
        }
      });
      L.g[J][e] = v;
      if constexpr (TAN) L.gd[J][e] = vd;
    });
  }

  // First element of the state row (component J, k = 0) of this unit and the
  // stride between consecutive k.
  template <class PK, int J>
  __device__ __forceinline__ static float* state_row(const StreamArgs& a, int unit, int node, int64_t& kstride) {
    return state_row_of<PK, J>(a, a.state, unit, node, kstride);
  }
  template <class PK, int J, class F>
  __device__ __forceinline__ static F* state_row_of(const StreamArgs& a, F* base, int unit, int node,
                                                    int64_t& kstride) {
    constexpr int q = PK::member_of(J), o = PK::o_of(J), NO = PK::nout(q);
    const StreamPath& Q = a.paths[a.unit_paths[unit][q]];
    kstride = Q.cols_per_k;
    return base + Q.state_base + (int64_t)(node * NO + o) * K * Q.cols_per_k + Q.q * a.C;
  }

  // Radial MLP weight gradient: sum over this wave's state tile of the tile
  // times the same elements of a.dot_state (the cotangent gS), per k, into
  // a.dot_part[item][k] (item = this wave's work item).  Lane (i, g) holds
  // k = kb + r, kb = 4 g (K = 16) or 4 (g & 1) (K = 8), for every tile.  All
  // loads are issued first, unconditionally (addresses clamped inside the
  // node's rows, out-of-range terms masked to zero), then the lanes of one k
  // are added by a fixed pattern of lane swaps.
  template <class PK, int TILES>
  __device__ __forceinline__ static void dot_out(const StreamArgs& a, int unit, int node, int slice, uint32_t item,
                                                 const floatx4 (&acc)[TILES][2], GfLds<K, TAN>& /*L*/) {
    constexpr int TOT = PK::TOT;
    const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
    const int C = a.C;
    const int cp = slice * kGfSlice + 2 * i;
    const int c0 = cp < C ? cp : C - 1, c1 = cp + 1 < C ? cp + 1 : C - 1;
    const bool upper = K == 8 && g >= 2;
    const int kb = K == 16 ? 4 * g : 4 * (g & 1);
    float gv[TILES][4][2];
    bool live[TILES];
    static_for<TILES>([&](auto Tc) {
      constexpr int T = decltype(Tc)::value;
      constexpr int JA = K == 16 ? T : 2 * T;
      constexpr int JB = K == 16 ? T : 2 * T + 1;
      int64_t ks_a, ks_b = 0;
      const float* pa = state_row_of<PK, JA>(a, a.dot_state, unit, node, ks_a);
      const float* pb = pa;
      if constexpr (JB < TOT) pb = state_row_of<PK, JB>(a, a.dot_state, unit, node, ks_b);
      live[T] = !(upper && JB >= TOT);
      const bool use_b = upper && JB < TOT;
      const float* p = use_b ? pb : pa;
      const int64_t ks = use_b ? ks_b : ks_a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        gv[T][r][0] = p[(kb + r) * ks + c0];
        gv[T][r][1] = p[(kb + r) * ks + c1];
      }
    });
    const bool m0 = cp < C, m1 = cp + 1 < C;
    float d[4] = {0.f, 0.f, 0.f, 0.f};
    static_for<TILES>([&](auto Tc) {
      constexpr int T = decltype(Tc)::value;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x0 = live[T] && m0 ? gv[T][r][0] : 0.f, x1 = live[T] && m1 ? gv[T][r][1] : 0.f;
        d[r] = __builtin_fmaf(acc[T][0][r], x0, d[r]);
        d[r] = __builtin_fmaf(acc[T][1][r], x1, d[r]);
      }
    });
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      d[r] = channel_sum(d[r], 4);                 // the 16 lanes of a row
      if constexpr (K == 8) d[r] = half32_add(d[r]);  // rows g and g + 2 hold the same k
    }
    if (i == 0 && (K == 16 || g < 2)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) a.dot_part[(int64_t)item * K + kb + r] = d[r];
    }
  }

  template <class... Ps>
  __device__ __forceinline__ static void run(const StreamArgs& a, int node, int unit, int slice, uint32_t item,
                                             GfLds<K, TAN>& L) {
    using PK = GfPack<RECV, Ps...>;
    constexpr int TOT = PK::TOT, NIN = PK::NIN;
    static_assert(TOT <= kGfMaxTot, "unit has more output components than the LDS table holds");
    constexpr int TILES = (K * TOT + 15) / 16;
    const int lane = threadIdx.x & 63, i = lane & 15, g = lane >> 4;
    const int C = a.C;
    const int k = i & (K - 1);  // row 16 T + i has k = i % K (K divides 16)
    // lane i holds channels cp and cp + 1 (column i of the even and odd tiles)
    const int cp = slice * kGfSlice + 2 * i;
    const char* fhi = static_cast<const char*>(a.feat);
    const char* flo = static_cast<const char*>(a.feat_lo);
    const int CS = a.feat_cs;  // channel stride of the gathered planes (a multiple of the slice)
    const uint32_t rowbytes = (uint32_t)CS * 2;
    const uint32_t nodebytes = (uint32_t)a.feat_rows * rowbytes;
    const uint32_t lanebytes = (uint32_t)a.paths[a.unit_paths[unit][0]].feat_row * rowbytes + (uint32_t)cp * 2;

    const SplitConsts sk;
    floatx4 acc[TILES][2];
#pragma unroll
    for (int T = 0; T < TILES; ++T) acc[T][0] = acc[T][1] = floatx4{0.f, 0.f, 0.f, 0.f};

    const float psx = a.pos[3 * (int64_t)node], psy = a.pos[3 * (int64_t)node + 1],
                psz = a.pos[3 * (int64_t)node + 2];
    const int e0 = a.ptr[node], e1 = a.ptr[node + 1];
    for (int b0 = e0; b0 < e1; b0 += kGfBatch) {
      const int nb = min(kGfBatch, e1 - b0);
      const int nh = nb > 32 ? 2 : 1;
      float y[NSH], yd[TAN ? NSH : 1];
      wave_lds_sync();  // the previous batch's reads come first
      prep(a, node, psx, psy, psz, b0, nb, lane, nodebytes, L, y, yd);
      wave_lds_sync();
      // one 32-bit word (two channels) per edge and plane: row m1 of the
      // neighbours of this lane's eight edges of step h
      auto gather = [&](int m1, int h, uint32_t (&wh)[8], uint32_t (&wl)[8]) {
        const uint32_t rb = (uint32_t)m1 * rowbytes + lanebytes;
        const uint4 n0 = *reinterpret_cast<const uint4*>(&L.noff[32 * h + 8 * g]);
        const uint4 n1 = *reinterpret_cast<const uint4*>(&L.noff[32 * h + 8 * g + 4]);
        const uint32_t nb8[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const uint32_t o = nb8[t] + rb;
          wh[t] = *reinterpret_cast<const uint32_t*>(fhi + o);
          if constexpr (LO) wl[t] = *reinterpret_cast<const uint32_t*>(flo + o);
        }
      };
      // the two B operands (even and odd channels) of eight edges
      auto pack = [&](const uint32_t (&w)[8], u32x4& even, u32x4& odd) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          even[t] = __builtin_amdgcn_perm(w[2 * t + 1], w[2 * t], 0x05040100u);
          odd[t] = __builtin_amdgcn_perm(w[2 * t + 1], w[2 * t], 0x07060302u);
        }
      };
      uint32_t wh[8], wl[8];
      gather(0, 0, wh, wl);

      static_for<NIN>([&](auto Gc) {
        constexpr int G = decltype(Gc)::value;
        couple_table<PK, G>(y, yd, lane, L);
        wave_lds_sync();
        static_for<2>([&](auto Hc) {
          constexpr int h = decltype(Hc)::value;
          if (h >= nh) return;  // uniform: a batch of at most 32 edges has one step
          u32x4 ch0, ch1, cl0, cl1;
          pack(wh, ch0, ch1);
          if constexpr (LO) pack(wl, cl0, cl1);
          // the next step's rows, in flight during this step
          if (h + 1 < nh)
            gather(G, 1, wh, wl);
          else if constexpr (G + 1 < NIN)
            gather(G + 1, 0, wh, wl);
          float r8[8], rt8[8];
          {
            const floatx4 u0 = *reinterpret_cast<const floatx4*>(&L.R[k][32 * h + 8 * g]);
            const floatx4 u1 = *reinterpret_cast<const floatx4*>(&L.R[k][32 * h + 8 * g + 4]);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              r8[t] = u0[t];
              r8[4 + t] = u1[t];
            }
            if constexpr (TAN) {
              const floatx4 w0 = *reinterpret_cast<const floatx4*>(&L.Rt[k][32 * h + 8 * g]);
              const floatx4 w1 = *reinterpret_cast<const floatx4*>(&L.Rt[k][32 * h + 8 * g + 4]);
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                rt8[t] = w0[t];
                rt8[4 + t] = w1[t];
              }
            }
          }
          // the coupling values of tile T's rows at this lane's eight edges
          // (rows past the unit read the zero row)
          auto gload = [&](auto Tc, floatx4 (&gv)[TAN ? 4 : 2]) {
            constexpr int T = decltype(Tc)::value;
            int j;
            if constexpr (K == 16) {
              j = T;
            } else if constexpr (2 * T + 1 < TOT) {
              j = 2 * T + (i >> 3);
            } else {
              j = (i >> 3) ? kGfMaxTot : 2 * T;
            }
            const float* gp = &L.g[j][32 * h + 8 * g];
            gv[0] = *reinterpret_cast<const floatx4*>(gp);
            gv[1] = *reinterpret_cast<const floatx4*>(gp + 4);
            if constexpr (TAN) {
              const float* dp = &L.gd[j][32 * h + 8 * g];
              gv[2] = *reinterpret_cast<const floatx4*>(dp);
              gv[3] = *reinterpret_cast<const floatx4*>(dp + 4);
            }
          };
          floatx4 gnext[TAN ? 4 : 2];
          gload(std::integral_constant<int, 0>{}, gnext);
          static_for<TILES>([&](auto Tc) {
            constexpr int T = decltype(Tc)::value;
            floatx4 gv[TAN ? 4 : 2];
#pragma unroll
            for (int q = 0; q < (TAN ? 4 : 2); ++q) gv[q] = gnext[q];
            // the next tile's values, in flight during this tile
            if constexpr (T + 1 < TILES) gload(std::integral_constant<int, T + 1>{}, gnext);
            float av[8];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              av[t] = r8[t] * gv[0][t];
              av[4 + t] = r8[4 + t] * gv[1][t];
            }
            if constexpr (TAN) {
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                av[t] = __builtin_fmaf(rt8[t], gv[2][t], av[t]);
                av[4 + t] = __builtin_fmaf(rt8[4 + t], gv[3][t], av[4 + t]);
              }
            }
            u32x4 ah, al;
            split8(av, ah, al, sk);
            acc[T][0] = mfma_bf16(ah, ch0, acc[T][0]);
            acc[T][1] = mfma_bf16(ah, ch1, acc[T][1]);
            if constexpr (LO) {
              acc[T][0] = mfma_bf16(ah, cl0, acc[T][0]);
              acc[T][1] = mfma_bf16(ah, cl1, acc[T][1]);
            }
            acc[T][0] = mfma_bf16(al, ch0, acc[T][0]);
            acc[T][1] = mfma_bf16(al, ch1, acc[T][1]);
          });
        });
        wave_lds_sync();  // this row's table reads before the next row's writes
      });
    }

    // rows 4g..4g+3 of each tile: component j and k = (16 T + 4 g + r) % K;
    // column i of the even / odd tile: channel cp / cp + 1
    if (a.dot_state) {  // the tile's dot with the cotangent instead of a store
      dot_out<PK, TILES>(a, unit, node, slice, item, acc, L);
      return;
    }
    static_for<TILES>([&](auto Tc) {
      constexpr int T = decltype(Tc)::value;
      constexpr int JA = K == 16 ? T : 2 * T;       // rows of lane groups 0, 1 (K = 8) or all (K = 16)
      constexpr int JB = K == 16 ? T : 2 * T + 1;   // rows of lane groups 2, 3 (K = 8)
      int64_t ks_a, ks_b = 0;
      float* pa = state_row<PK, JA>(a, unit, node, ks_a);
      float* pb = nullptr;
      if constexpr (JB < TOT) pb = state_row<PK, JB>(a, unit, node, ks_b);
      const bool upper = K == 8 && g >= 2;
      if (upper && JB >= TOT) return;
      float* p = upper ? pb : pa;
      const int64_t ks = upper ? ks_b : ks_a;
      const int kb = K == 16 ? 4 * g : 4 * (g & 1);
      if (cp + 1 < C && (C & 1) == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<float2*>(p + (kb + r) * ks + cp) = make_float2(acc[T][0][r], acc[T][1][r]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (cp < C) p[(kb + r) * ks + cp] = acc[T][0][r];
          if (cp + 1 < C) p[(kb + r) * ks + cp + 1] = acc[T][1][r];
        }
      }
    });
  }
};

template <int LMAX, int K, int MODE, bool LO>
struct GfUnitRunner {
  int node, unit, slice;
  uint32_t item;
  GfLds<K, ModeTraits<MODE>::tangent>& L;
  template <class... Ps>
  __device__ __forceinline__ void run(const StreamArgs& a) {
    GfWave<LMAX, K, MODE, LO>::template run<Ps...>(a, node, unit, slice, item, L);
  }
};

// Waves per SIMD the register allocation must leave room for: the tangent
// modes and lmax 3 need more than the 168 registers of three.
constexpr int gf_min_waves(int lmax, int K, int mode) {
  return (lmax == 3 || mode == kJvp || mode == kSndT) ? 2 : 3;
}

// One wave per (node, unit, slice); items ordered node-major so that the
// units of a node run side by side on one XCD.
template <int LMAX, int K, int MODE, bool LO, bool BUNDLED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(gf_min_waves(LMAX, K, MODE))))
void gf_kernel(const StreamArgs /*args*/, int64_t items) {
  const StreamArgs& a = *(const StreamArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr bool TAN = ModeTraits<MODE>::tangent;
  __shared__ GfLds<K, TAN> L;
  const uint32_t item = (uint32_t)xcd_item(blockIdx.x, gridDim.x);
  if (item >= (uint32_t)items) return;  // uniform over the block
  const uint32_t ns = (uint32_t)a.nslices, nu = (uint32_t)a.nunits;
  const int slice = (int)(item % ns);
  const uint32_t t = item / ns;
  const int unit = (int)(t % nu);
  const int node = a.order ? a.order[t / nu] : (int)(t / nu);
  const int lane = threadIdx.x & 63;
  L.g[kGfMaxTot][lane] = 0.f;
  if constexpr (TAN) L.gd[kGfMaxTot][lane] = 0.f;
  GfUnitRunner<LMAX, K, MODE, LO> run{node, unit, slice, item, L};
  if constexpr (BUNDLED) {
    Bundles<LMAX, K, ModeTraits<MODE>::recv ? 0 : 1>::run(unit, run, a);
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

// LO: fp32 features pre-split into a.feat (hi) and a.feat_lo (lo); otherwise
// a.feat holds bf16 features.  Byte offsets into the gathered planes are
// 32-bit: N * feat_rows * feat_cs * 2 must stay below 2^32 (checked by the
// caller).
template <int MODE, bool LO>
hipError_t launch_gf(int lmax, int K, const StreamArgs& a, hipStream_t s) {
  if (LO != (a.feat_lo != nullptr) || a.feat_cs % kGfSlice != 0 || a.nslices * kGfSlice != a.feat_cs)
    return hipErrorInvalidValue;
  const int64_t items = (int64_t)a.num_nodes * a.nunits * a.nslices;
  if (items == 0) return hipSuccess;
  const int64_t grid = (items + 7) / 8 * 8;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
#define TPCONV_LAUNCH(LM, KK)                                                                                     \
  if (lmax == LM && K == KK) {                                                                                    \
    if (a.bundled)                                                                                                \
      hipLaunchKernelGGL((gf_kernel<LM, KK, MODE, LO, true>), dim3((unsigned)grid), dim3(64), 0, s, a, items);    \
    else                                                                                                          \
      hipLaunchKernelGGL((gf_kernel<LM, KK, MODE, LO, false>), dim3((unsigned)grid), dim3(64), 0, s, a, items);   \
    return hipGetLastError();                                                                                     \
  }
  TPCONV_LAUNCH(0, 8) TPCONV_LAUNCH(0, 16)
  TPCONV_LAUNCH(1, 8) TPCONV_LAUNCH(1, 16)
  TPCONV_LAUNCH(2, 8) TPCONV_LAUNCH(2, 16)
  TPCONV_LAUNCH(3, 8) TPCONV_LAUNCH(3, 16)
#undef TPCONV_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace tpconv
