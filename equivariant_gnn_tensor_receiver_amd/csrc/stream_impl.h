// Edge-streaming kernels: the receiver-side (and mirrored sender-side)
// accumulation of the Sobek reassociation ("Sobek" page, abstract: edge-local
// products consumed directly into bounded receiver-side state).
//
// Work decomposition: one wavefront per (node, channel tile, path).  The node's
// edges are streamed in batches; lane j of the wave computes the geometry of
// edge j of the batch (radial basis, harmonics and, where needed, their
// derivatives) into wave-private LDS.  Then lanes map to (channel, edge slot):
// each lane gathers the neighbour's feature rows of its path for its channel
// (coalesced across channels), forms the CG coupling with the baked table on
// VALU, and accumulates the outer product with R into registers.  Edge slots
// are summed with cross-lane shuffles at the end; the state of a (node, path,
// channel) is written once.  No per-edge value is ever written to memory and
// no atomics touch the state.
#pragma once

#include "cg_tables.inc"
#include "device_common.h"
#include "kernels.h"

namespace tpconv {

template <int MODE>
struct ModeTraits {
  static constexpr bool recv = (MODE == kFwd || MODE == kJvp || MODE == kBwdPos);
  static constexpr bool tangent = (MODE == kJvp || MODE == kSndT);
  static constexpr bool bwdpos = (MODE == kBwdPos);
  static constexpr int batch = (MODE == kFwd || MODE == kSnd) ? 64 : 32;
};

template <int K, int NSH, int MODE>
struct EdgeLds {
  static constexpr int B = ModeTraits<MODE>::batch;
  static constexpr int BT = ModeTraits<MODE>::tangent ? B : 1;
  static constexpr int BP = ModeTraits<MODE>::bwdpos ? B : 1;
  int nbr[B];
  float R[B][K];
  float Y[B][NSH];
  float Rd[(ModeTraits<MODE>::tangent || ModeTraits<MODE>::bwdpos) ? B : 1][K];  // R_dot or R'
  float Yd[BT][NSH];
  float J[BP][NSH][3];
  float rhat[BP][3];
};

// Geometry of one edge into LDS slot j.
template <int LMAX, int K, int MODE>
__device__ __forceinline__ void edge_prep(const StreamArgs& a, int self, float psx, float psy, float psz, int e,
                                          int j, EdgeLds<K, sh_count(LMAX), MODE>& L) {
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
  float Y[NSH];
  sh_eval<LMAX>(ux, uy, uz, Y);
  L.nbr[j] = nb;
#pragma unroll
  for (int k = 0; k < K; ++k) L.R[j][k] = R[k];
#pragma unroll
  for (int i = 0; i < NSH; ++i) L.Y[j][i] = Y[i];
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
        const float l = (float)sh_degree_of_row(i);
        L.Yd[j][i] = (G[i][0] * fx + G[i][1] * fy + G[i][2] * fz - l * Y[i] * rphi) * inv_d;
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

template <int LMAX, int K, int MODE, typename FT, int L1, int L2, int L3>
__device__ __forceinline__ void run_path(const StreamArgs& a, const StreamPath& P, int node, int tile,
                                         EdgeLds<K, sh_count(LMAX), MODE>& L) {
  constexpr int N1 = 2 * L1 + 1, N2 = 2 * L2 + 1, N3 = 2 * L3 + 1;
  constexpr bool RECV = ModeTraits<MODE>::recv;
  constexpr int NIN = RECV ? N1 : N3;
  constexpr int NOUT = RECV ? N3 : N1;
  constexpr int B = ModeTraits<MODE>::batch;
  constexpr int Y0 = L2 * L2;
  using Tab = CG<L1, L2, L3>;

  const int lane = threadIdx.x;
  const int ctl = a.ct_log2;
  const int CT = 1 << ctl;
  const int ES = 64 >> ctl;
  const int cl = lane & (CT - 1);
  const int es = lane >> ctl;
  const int c = tile * CT + cl;
  const int C = a.C;
  const FT* feat = static_cast<const FT*>(a.feat);

  float acc[K][NOUT];
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int o = 0; o < NOUT; ++o) acc[k][o] = 0.f;

  float gs[ModeTraits<MODE>::bwdpos ? K : 1][N3];
  float vself[3] = {0.f, 0.f, 0.f};
  if constexpr (ModeTraits<MODE>::bwdpos) {
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
      for (int o = 0; o < N3; ++o)
        gs[k][o] = a.gstate[P.state_base + ((int64_t)(node * N3 + o) * K + k) * P.cols_per_k + P.q * C + c];
  }

  const float psx = a.pos[3 * (int64_t)node], psy = a.pos[3 * (int64_t)node + 1],
              psz = a.pos[3 * (int64_t)node + 2];
  const int e0 = a.ptr[node], e1 = a.ptr[node + 1];
  for (int b0 = e0; b0 < e1; b0 += B) {
    const int nb = min(B, e1 - b0);
    __syncthreads();
    if (lane < nb) edge_prep<LMAX, K, MODE>(a, node, psx, psy, psz, b0 + lane, lane, L);
    __syncthreads();
    for (int j0 = 0; j0 < nb; j0 += ES) {
      const int j = j0 + es;
      if (j >= nb) continue;
      const int nbv = L.nbr[j];
      float av[NIN];
      const int64_t fbase = ((int64_t)nbv * a.feat_rows + P.feat_row) * C + c;
#pragma unroll
      for (int i = 0; i < NIN; ++i) av[i] = load_feat(feat, fbase + (int64_t)i * C);
      float y[N2];
#pragma unroll
      for (int i = 0; i < N2; ++i) y[i] = L.Y[j][Y0 + i];
      float r[K];
#pragma unroll
      for (int k = 0; k < K; ++k) r[k] = L.R[j][k];

      if constexpr (MODE == kFwd || MODE == kSnd) {
        float u[NOUT];
        if constexpr (RECV) Tab::fwd(av, y, u); else Tab::snd(av, y, u);
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
          for (int o = 0; o < NOUT; ++o) acc[k][o] = __builtin_fmaf(r[k], u[o], acc[k][o]);
      } else if constexpr (MODE == kJvp || MODE == kSndT) {
        float yd[N2], rd[K];
#pragma unroll
        for (int i = 0; i < N2; ++i) yd[i] = L.Yd[j][Y0 + i];
#pragma unroll
        for (int k = 0; k < K; ++k) rd[k] = L.Rd[j][k];
        float u[NOUT], ud[NOUT];
        if constexpr (RECV) {
          Tab::fwd(av, y, u);
          Tab::fwd(av, yd, ud);
        } else {
          Tab::snd(av, y, u);
          Tab::snd(av, yd, ud);
        }
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
          for (int o = 0; o < NOUT; ++o)
            acc[k][o] = __builtin_fmaf(rd[k], u[o], __builtin_fmaf(r[k], ud[o], acc[k][o]));
      } else {  // kBwdPos
        float u[N3];
        Tab::fwd(av, y, u);
        float alpha = 0.f;
        float gU[N3];
#pragma unroll
        for (int o = 0; o < N3; ++o) gU[o] = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          float gR = 0.f;
#pragma unroll
          for (int o = 0; o < N3; ++o) {
            gR = __builtin_fmaf(gs[k][o], u[o], gR);
            gU[o] = __builtin_fmaf(r[k], gs[k][o], gU[o]);
          }
          alpha = __builtin_fmaf(gR, L.Rd[j][k], alpha);
        }
        float gy[N2];
#pragma unroll
        for (int i = 0; i < N2; ++i) gy[i] = 0.f;
        Tab::ybar(av, gU, gy);
        float vec[3];
#pragma unroll
        for (int cc = 0; cc < 3; ++cc) {
          float v = alpha * L.rhat[j][cc];
#pragma unroll
          for (int i = 0; i < N2; ++i) v = __builtin_fmaf(gy[i], L.J[j][Y0 + i][cc], v);
          vec[cc] = v;
        }
        for (int off = 1; off < CT; off <<= 1)
#pragma unroll
          for (int cc = 0; cc < 3; ++cc) vec[cc] += __shfl_xor(vec[cc], off);
        if (cl == 0) {
#pragma unroll
          for (int cc = 0; cc < 3; ++cc) {
            atomicAdd(&a.gpos[3 * (int64_t)nbv + cc], vec[cc]);
            vself[cc] -= vec[cc];
          }
        }
      }
    }
  }

  if constexpr (ModeTraits<MODE>::bwdpos) {
    for (int off = CT; off < 64; off <<= 1)
#pragma unroll
      for (int cc = 0; cc < 3; ++cc) vself[cc] += __shfl_xor(vself[cc], off);
    if (lane == 0 && e1 > e0) {
#pragma unroll
      for (int cc = 0; cc < 3; ++cc) atomicAdd(&a.gpos[3 * (int64_t)node + cc], vself[cc]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
      for (int o = 0; o < NOUT; ++o) {
        float v = acc[k][o];
        for (int off = CT; off < 64; off <<= 1) v += __shfl_xor(v, off);
        if (es == 0)
          a.state[P.state_base + ((int64_t)(node * NOUT + o) * K + k) * P.cols_per_k + P.q * C + c] = v;
      }
  }
}

#define TPCONV_PATH_CASES(X)                                                                                  \
  X(0, 0, 0) X(0, 1, 1) X(0, 2, 2) X(0, 3, 3) X(1, 0, 1) X(1, 1, 0) X(1, 1, 1) X(1, 1, 2) X(1, 2, 1)          \
  X(1, 2, 2) X(1, 2, 3) X(1, 3, 2) X(1, 3, 3) X(2, 0, 2) X(2, 1, 1) X(2, 1, 2) X(2, 1, 3) X(2, 2, 0)          \
  X(2, 2, 1) X(2, 2, 2) X(2, 2, 3) X(2, 3, 1) X(2, 3, 2) X(2, 3, 3) X(3, 0, 3) X(3, 1, 2) X(3, 1, 3)          \
  X(3, 2, 1) X(3, 2, 2) X(3, 2, 3) X(3, 3, 0) X(3, 3, 1) X(3, 3, 2) X(3, 3, 3)

template <int LMAX, int K, int MODE, typename FT>
__global__ __launch_bounds__(64) void stream_kernel(const StreamArgs a, int64_t items) {
  __shared__ EdgeLds<K, sh_count(LMAX), MODE> L;
  const int64_t item = xcd_item(blockIdx.x, gridDim.x);
  if (item >= items) return;
  const int p = (int)(item % a.npaths);
  const int64_t t = item / a.npaths;
  const int tile = (int)(t % a.ntiles);
  const int node = (int)(t / a.ntiles);
  const StreamPath& P = a.paths[p];
  switch (P.l1 * 16 + P.l2 * 4 + P.l3) {
#define TPCONV_CASE(A, B, C)                                                    \
  case A * 16 + B * 4 + C:                                                      \
    if constexpr (A <= LMAX && B <= LMAX && C <= LMAX)                          \
      run_path<LMAX, K, MODE, FT, A, B, C>(a, P, node, tile, L);                \
    break;
    TPCONV_PATH_CASES(TPCONV_CASE)
#undef TPCONV_CASE
    default:
      break;
  }
}

template <int MODE, typename FT>
hipError_t launch_stream_mode(int lmax, int K, const StreamArgs& a, int64_t items, hipStream_t s) {
  const int64_t grid = (items + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
#define TPCONV_LAUNCH(LM, KK)                                                                      \
  if (lmax == LM && K == KK) {                                                                     \
    hipLaunchKernelGGL((stream_kernel<LM, KK, MODE, FT>), dim3((unsigned)grid), dim3(64), 0, s, a, items); \
    return hipGetLastError();                                                                      \
  }
  TPCONV_LAUNCH(0, 8) TPCONV_LAUNCH(0, 16)
  TPCONV_LAUNCH(1, 8) TPCONV_LAUNCH(1, 16)
  TPCONV_LAUNCH(2, 8) TPCONV_LAUNCH(2, 16)
  TPCONV_LAUNCH(3, 8) TPCONV_LAUNCH(3, 16)
#undef TPCONV_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace tpconv
