// Shared pieces of the edge streams ("Sobek" page, abstract: edge-local
// products consumed directly into bounded receiver-side state): the modes,
// the per-batch edge geometry in LDS (radial basis, harmonics and, where
// needed, their derivatives, computed by one lane per edge), cross-lane sums
// and the dispatch over the paths of single-path units.  The accumulating
// streams are in stream_gf.h, the position streams in stream_pos.h.
#pragma once

#include <type_traits>

#include "cg_tables.inc"
#include "device_common.h"
#include "kernels.h"

namespace tpconv {

typedef float floatx4 __attribute__((ext_vector_type(4)));


template <int MODE>
struct ModeTraits {
  static constexpr bool recv = (MODE == kFwd || MODE == kJvp || MODE == kBwdPos);
  static constexpr bool tangent = (MODE == kJvp || MODE == kSndT);
  static constexpr bool bwdpos = (MODE == kBwdPos);
  static constexpr int batch = (MODE == kFwd || MODE == kSnd) ? 64 : 32;
};

// Geometry of one batch of BATCH edges (wave-private, or shared by the waves
// of a block).  Harmonic blocks are padded to 8 floats per degree and Jacobian
// rows to 4 so that reads are 16-byte aligned.
template <int K, int LMAX, int MODE, int BATCH = ModeTraits<MODE>::batch>
struct __attribute__((aligned(16))) EdgeLds {
  static constexpr int B = BATCH;
  static constexpr int NSH = sh_count(LMAX);
  static constexpr int BT = ModeTraits<MODE>::tangent ? B : 1;
  static constexpr int BP = ModeTraits<MODE>::bwdpos ? B : 1;
  int nbr[B];
  float R[B][K];
  float Y[B][LMAX + 1][8];
  float Rd[(ModeTraits<MODE>::tangent || ModeTraits<MODE>::bwdpos) ? B : 1][K];  // R_dot or R'
  float Yd[BT][LMAX + 1][8];
  float J[BP][NSH][4];
  float rhat[BP][4];
};

// Geometry of one edge into LDS slot j.
template <int LMAX, int K, int MODE, int BATCH>
__device__ __forceinline__ void edge_prep(const StreamArgs& a, int self, float psx, float psy, float psz, int e,
                                          int j, EdgeLds<K, LMAX, MODE, BATCH>& L) {
  constexpr int NSH = sh_count(LMAX);
  constexpr bool RECV = ModeTraits<MODE>::recv;
  constexpr bool DER = ModeTraits<MODE>::tangent || ModeTraits<MODE>::bwdpos;
  const int nb = a.nbr[e];
  const float qx = a.pos[3 * (int64_t)nb], qy = a.pos[3 * (int64_t)nb + 1], qz = a.pos[3 * (int64_t)nb + 2];
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
  radial<K, DER>(d, a.cutoff, a.inv_cutoff, a.pref, a.env_p, a.env_a, a.env_b, a.env_c, a.env_d, R, dR);
  if (a.mlp) mlp_radial<K, DER ? 1 : 0>(a.mlp, -1, R, dR, nullptr);
  float Y[NSH];
  sh_eval<LMAX>(ux, uy, uz, Y);
  L.nbr[j] = nb;
#pragma unroll
  for (int k = 0; k < K; ++k) L.R[j][k] = R[k];
#pragma unroll
  for (int i = 0; i < NSH; ++i) {
    const int l = sh_degree_of_row(i);
    L.Y[j][l][i - l * l] = Y[i];
  }
  if constexpr (DER) {
    float G[NSH][3];
    sh_poly_grad<LMAX>(ux, uy, uz, G);
    if constexpr (ModeTraits<MODE>::tangent) {
      const int s = RECV ? nb : self, v = RECV ? self : nb;
      const float fx = a.ggpos[3 * (int64_t)s] - a.ggpos[3 * (int64_t)v];
      const float fy = a.ggpos[3 * (int64_t)s + 1] - a.ggpos[3 * (int64_t)v + 1];
      const float fz = a.ggpos[3 * (int64_t)s + 2] - a.ggpos[3 * (int64_t)v + 2];
      const float rphi = ux * fx + uy * fy + uz * fz;
#pragma unroll
      for (int k = 0; k < K; ++k) L.Rd[j][k] = dR[k] * rphi;
#pragma unroll
      for (int i = 0; i < NSH; ++i) {
        const int l = sh_degree_of_row(i);
        L.Yd[j][l][i - l * l] = (G[i][0] * fx + G[i][1] * fy + G[i][2] * fz - (float)l * Y[i] * rphi) * inv_d;
      }
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k) L.Rd[j][k] = dR[k];
      L.rhat[j][0] = ux;
      L.rhat[j][1] = uy;
      L.rhat[j][2] = uz;
      const float uu[3] = {ux, uy, uz};
#pragma unroll
      for (int i = 0; i < NSH; ++i) {
        const float l = (float)sh_degree_of_row(i);
#pragma unroll
        for (int c = 0; c < 3; ++c) L.J[j][i][c] = (G[i][c] - l * Y[i] * uu[c]) * inv_d;
      }
    }
  }
}

// v + (v read through the DPP lane pattern CTRL): one VALU op, no LDS traffic.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// v + the same lane of the other 16-lane row of its 32-lane half.
__device__ __forceinline__ float row16_add(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// v + the same lane of the other 32-lane half.
__device__ __forceinline__ float half32_add(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the channel lanes of one edge slot (lanes c = 0..CT-1 of a group),
// every lane of the group receiving the sum.  After the two quad steps each
// quad is uniform, so the half-row and row mirrors pair it with the right
// neighbours.
__device__ __forceinline__ float channel_sum(float v, int ct_log2) {
  if (ct_log2 >= 1) v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
  if (ct_log2 >= 2) v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
  if (ct_log2 >= 3) v = dpp_add<0x141>(v);  // row_half_mirror
  if (ct_log2 >= 4) v = dpp_add<0x140>(v);  // row_mirror
  if (ct_log2 >= 5) v = row16_add(v);
  if (ct_log2 >= 6) v = half32_add(v);
  return v;
}

template <class P0, class... Ps>
struct First {
  using type = P0;
};

#define TPCONV_PATH_CASES(X)                                                                                  \
  X(0, 0, 0) X(0, 1, 1) X(0, 2, 2) X(0, 3, 3) X(1, 0, 1) X(1, 1, 0) X(1, 1, 1) X(1, 1, 2) X(1, 2, 1)          \
  X(1, 2, 2) X(1, 2, 3) X(1, 3, 2) X(1, 3, 3) X(2, 0, 2) X(2, 1, 1) X(2, 1, 2) X(2, 1, 3) X(2, 2, 0)          \
  X(2, 2, 1) X(2, 2, 2) X(2, 2, 3) X(2, 3, 1) X(2, 3, 2) X(2, 3, 3) X(3, 0, 3) X(3, 1, 2) X(3, 1, 3)          \
  X(3, 2, 1) X(3, 2, 2) X(3, 2, 3) X(3, 3, 0) X(3, 3, 1) X(3, 3, 2) X(3, 3, 3)

}  // namespace tpconv
