// Edge-streaming kernels: the receiver-side (and mirrored sender-side)
// accumulation of the Sobek reassociation ("Sobek" page, abstract: edge-local
// products consumed directly into bounded receiver-side state).
//
// Work decomposition: one wavefront per (node, channel tile, unit).  A unit is
// a compile-time bundle of paths that gather the same feature block (the same
// l1 on the receiver side, the same l3 on the sender side); plans whose irreps
// are not the natural ones use single-path units.  The node's edges are
// streamed in batches; lane j of the wave computes the geometry of edge j of
// the batch (radial basis, harmonics and, where needed, their derivatives)
// into wave-private LDS.  Then lanes map to (channel, edge slot): each lane
// gathers the neighbour's feature rows for its channel (coalesced across
// channels; the next edge's rows are loaded while the current one is used),
// forms every member path's CG coupling with the baked tables on VALU and
// accumulates the outer product with R into registers.  Edge slots are summed
// across lanes at the end and each (node, path, channel) state entry is
// written once.  No per-edge value is ever written to memory and no atomics
// touch the state.
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

// Sum over the edge slots of a wave (lanes c, c + CT, c + 2 CT, ...).
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

// Sum over the edge slots (lanes with the same channel, lane % CT) of every
// value in v: rotations within each 16-lane row by CT, 2CT, .. 8, then across
// rows and halves.  The launch-uniform ct_log2 makes every branch scalar, one
// per stage for all values.
template <int N>
__device__ __forceinline__ void edge_slot_sum(float (&v)[N], int ct_log2) {
  if (ct_log2 >= 6) return;
  if (ct_log2 <= 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = dpp_add<0x121>(v[i]);  // row_ror:1
  }
  if (ct_log2 <= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = dpp_add<0x122>(v[i]);  // row_ror:2
  }
  if (ct_log2 <= 2) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = dpp_add<0x124>(v[i]);  // row_ror:4
  }
  if (ct_log2 <= 3) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = dpp_add<0x128>(v[i]);  // row_ror:8
  }
  if (ct_log2 <= 4) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = row16_add(v[i]);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = half32_add(v[i]);
}

// channel_sum of three values, interleaved so that one scalar branch covers a
// step and the DPP read-after-write waits of one value overlap the others.
__device__ __forceinline__ void channel_sum3(float (&v)[3], int ct_log2) {
  if (ct_log2 >= 1) { v[0] = dpp_add<0xB1>(v[0]); v[1] = dpp_add<0xB1>(v[1]); v[2] = dpp_add<0xB1>(v[2]); }
  if (ct_log2 >= 2) { v[0] = dpp_add<0x4E>(v[0]); v[1] = dpp_add<0x4E>(v[1]); v[2] = dpp_add<0x4E>(v[2]); }
  if (ct_log2 >= 3) { v[0] = dpp_add<0x141>(v[0]); v[1] = dpp_add<0x141>(v[1]); v[2] = dpp_add<0x141>(v[2]); }
  if (ct_log2 >= 4) { v[0] = dpp_add<0x140>(v[0]); v[1] = dpp_add<0x140>(v[1]); v[2] = dpp_add<0x140>(v[2]); }
  if (ct_log2 >= 5) { v[0] = row16_add(v[0]); v[1] = row16_add(v[1]); v[2] = row16_add(v[2]); }
  if (ct_log2 >= 6) { v[0] = half32_add(v[0]); v[1] = half32_add(v[1]); v[2] = half32_add(v[2]); }
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

template <int MODE, class P>
constexpr int out_dim() {
  return ModeTraits<MODE>::recv ? 2 * P::l3 + 1 : 2 * P::l1 + 1;
}

// The kernel arguments travel as an explicit reference parameter through the
// (inlined) call chain; storing a reference to them in this object would make
// the compiler copy the whole argument block to scratch memory.
template <int MODE, typename FT, int LMAX, int K, int BATCH = ModeTraits<MODE>::batch>
struct StreamCtx {
  int node, tile, unit;
  EdgeLds<K, LMAX, MODE, BATCH>& L;

  static constexpr bool RECV = ModeTraits<MODE>::recv;
  static constexpr bool TAN = ModeTraits<MODE>::tangent;

  static constexpr int NSH = (LMAX + 1) * (LMAX + 1);
  // Whether the LDS geometry of the next step is held in registers: not where
  // those registers would take the kernel below two waves per SIMD.
  static constexpr bool kAccGeoAhead = !(LMAX >= 3 && K == 16 && TAN);

  // Geometry of one edge slot as the accumulating modes use it, read from LDS
  // one step ahead of its use: the matrix-core operand R[4 kq + lane % 4] (and
  // R_dot), the harmonics (entries that no member path reads are never
  // loaded) and the mask of a slot past the last edge.
  struct AccGeo {
    float r[K / 4], rd[K / 4], mask;
    float y[LMAX + 1][2 * LMAX + 1];
    float yd[TAN ? LMAX + 1 : 1][2 * LMAX + 1];
  };

  // One edge for the member paths OFF.. of the unit (compile-time recursion);
  // accumulating modes.
  template <int OFF, int TOT, int NIN, class P, class... Rest>
  __device__ __forceinline__ void edge(const float (&av)[NIN], const AccGeo& g, floatx4 (&acc)[K / 4][TOT]) {
    constexpr int N2 = 2 * P::l2 + 1;
    constexpr int NO = out_dim<MODE, P>();
    using Tab = CG<P::l1, P::l2, P::l3>;
    const float(&r)[K / 4] = g.r;
    const float(&rd)[K / 4] = g.rd;
    float y[N2];
#pragma unroll
    for (int i = 0; i < N2; ++i) y[i] = g.y[P::l2][i];
    float u[NO];
    if constexpr (RECV) Tab::fwd(av, y, u); else Tab::snd(av, y, u);
    if constexpr (!TAN) {
      // state += R (x) U on the matrix cores: r[kq] holds R[4 kq + lane % 4]
#pragma unroll
      for (int kq = 0; kq < K / 4; ++kq)
#pragma unroll
        for (int o = 0; o < NO; ++o)
          acc[kq][OFF + o] = __builtin_amdgcn_mfma_f32_4x4x1f32(r[kq], u[o], acc[kq][OFF + o], 0, 0, 0);
    } else {
      float yd[N2], ud[NO];
#pragma unroll
      for (int i = 0; i < N2; ++i) yd[i] = g.yd[TAN ? P::l2 : 0][i];
      if constexpr (RECV) Tab::fwd(av, yd, ud); else Tab::snd(av, yd, ud);
#pragma unroll
      for (int kq = 0; kq < K / 4; ++kq)
#pragma unroll
        for (int o = 0; o < NO; ++o) {
          acc[kq][OFF + o] = __builtin_amdgcn_mfma_f32_4x4x1f32(r[kq], ud[o], acc[kq][OFF + o], 0, 0, 0);
          acc[kq][OFF + o] = __builtin_amdgcn_mfma_f32_4x4x1f32(rd[kq], u[o], acc[kq][OFF + o], 0, 0, 0);
        }
    }
    if constexpr (sizeof...(Rest) > 0) edge<OFF + NO, TOT, NIN, Rest...>(av, g, acc);
  }

  // Write the member paths' slot-summed state (each entry once).
  template <int I, int OFF, int TOT, class P, class... Rest>
  __device__ __forceinline__ void store(const StreamArgs& a, const float (&v)[K * TOT], int c, bool owner) {
    constexpr int NO = out_dim<MODE, P>();
    const StreamPath& Q = a.paths[a.unit_paths[unit][I]];
    if (owner) {
#pragma unroll
      for (int k = 0; k < K; ++k)
#pragma unroll
        for (int o = 0; o < NO; ++o)
          a.state[Q.state_base + ((int64_t)(node * NO + o) * K + k) * Q.cols_per_k + Q.q * a.C + c] =
              v[k * TOT + OFF + o];
    }
    if constexpr (sizeof...(Rest) > 0) store<I + 1, OFF + NO, TOT, Rest...>(a, v, c, owner);
  }

  template <class... Ps>
  __device__ __forceinline__ void run(const StreamArgs& a) {
    run_acc<Ps...>(a);
  }

  // Accumulating modes: lanes are (channel, edge slot); each lane gathers its
  // channel of one edge per step and accumulates S[k, q, c, m] in registers.
  template <class... Ps>
  __device__ __forceinline__ void run_acc(const StreamArgs& a) {
    using P0 = typename First<Ps...>::type;
    constexpr int NIN = RECV ? 2 * P0::l1 + 1 : 2 * P0::l3 + 1;
    constexpr int TOT = (out_dim<MODE, Ps>() + ...);
    constexpr int B = BATCH;
    const int lane = threadIdx.x & 63;
    const int ctl = a.ct_log2;
    const int CT = 1 << ctl;
    const int ES = 64 >> ctl;
    const int cl = lane & (CT - 1);
    const int es = lane >> ctl;
    const int C = a.C;
    // Channel tiles have at least 4 lanes (the 4x4 outer products pair lanes
    // in fours); lanes past the last channel read channel C-1 and write nothing.
    const int c_lane = tile * CT + cl;
    const bool c_ok = c_lane < C;
    const int c = c_ok ? c_lane : C - 1;
    const int q4 = lane & 3;
    const FT* feat = static_cast<const FT*>(a.feat);
    const int64_t fcol = (int64_t)a.paths[a.unit_paths[unit][0]].feat_row * C + c;

    floatx4 acc[K / 4][TOT];
#pragma unroll
    for (int kq = 0; kq < K / 4; ++kq)
#pragma unroll
      for (int o = 0; o < TOT; ++o) acc[kq][o] = floatx4{0.f, 0.f, 0.f, 0.f};

    const float psx = a.pos[3 * (int64_t)node], psy = a.pos[3 * (int64_t)node + 1],
                psz = a.pos[3 * (int64_t)node + 2];
    const int e0 = a.ptr[node], e1 = a.ptr[node + 1];
    for (int b0 = e0; b0 < e1; b0 += B) {
      const int nb = min(B, e1 - b0);
      __syncthreads();
      if ((int)threadIdx.x < nb) edge_prep(a, node, psx, psy, psz, b0 + (int)threadIdx.x, (int)threadIdx.x, L);
      __syncthreads();
      // Branch-free edge loop: the gathers and the LDS geometry for the next
      // edge slot are issued before the current slot is used, and the
      // neighbour index one slot further ahead (edge indices clamped into the
      // batch, so every load is unconditional); a slot past the last edge is
      // masked by zeroing x.  The loop is unrolled by two over alternating
      // buffers so that no register copy waits on a load in flight; divergent
      // branches or such copies would make the compiler wait for every
      // outstanding load.
      const int last = nb - 1;
      const int nslots = (nb + ES - 1) >> (6 - ctl);  // ES = 2^(6 - ctl)
      using Raw = FeatRaw<FT>;
      auto nbr_of = [&](int slot) { return L.nbr[min(slot * ES + es, last)]; };
      auto gather = [&](int nbr, typename Raw::type (&v)[NIN]) {
        const int64_t f = (int64_t)nbr * a.feat_rows * C + fcol;
#pragma unroll
        for (int i = 0; i < NIN; ++i) v[i] = Raw::load(feat, f + (int64_t)i * C);
      };
      auto geo = [&](int slot, AccGeo& g) {
        const int j = slot * ES + es;
        const int jj = min(j, last);
        g.mask = j < nb ? 1.f : 0.f;  // applied to x at use (multiply, not select: no branch around the reads)
#pragma unroll
        for (int kq = 0; kq < K / 4; ++kq) {
          g.r[kq] = L.R[jj][4 * kq + q4];
          g.rd[kq] = TAN ? L.Rd[jj][4 * kq + q4] : 0.f;
        }
#pragma unroll
        for (int l = 0; l <= LMAX; ++l)
#pragma unroll
          for (int i = 0; i < 2 * LMAX + 1; ++i) {
            g.y[l][i] = i <= 2 * l ? L.Y[jj][l][i] : 0.f;
            if constexpr (TAN) g.yd[l][i] = i <= 2 * l ? L.Yd[jj][l][i] : 0.f;
          }
      };
      auto step = [&](const typename Raw::type (&raw)[NIN], const AccGeo& g) {
        float av[NIN];
#pragma unroll
        for (int i = 0; i < NIN; ++i) av[i] = Raw::f32(raw[i]) * g.mask;  // every term is linear in x
        edge<0, TOT, NIN, Ps...>(av, g, acc);
      };
      // scheduling barriers keep each load ahead of its use (the scheduler
      // would otherwise move the loads next to their consumers); where the
      // geometry registers would cost a wave of occupancy it is read at use
      auto run_step = [&](int slot, const typename Raw::type (&raw)[NIN], const AccGeo& g) {
        if constexpr (kAccGeoAhead) {
          step(raw, g);
        } else {
          AccGeo gl;
          geo(slot, gl);
          step(raw, gl);
        }
      };
      typename Raw::type bA[NIN], bB[NIN];
      AccGeo gA, gB;
      gather(nbr_of(0), bA);
      if constexpr (kAccGeoAhead) geo(0, gA);
      int nb1 = nbr_of(1), nb2;
      int t = 0;
      for (; t + 1 < nslots; t += 2) {
        gather(nb1, bB);
        nb2 = nbr_of(t + 2);
        if constexpr (kAccGeoAhead) geo(t + 1, gB);
        __builtin_amdgcn_sched_barrier(0);
        run_step(t, bA, gA);
        __builtin_amdgcn_sched_barrier(0);
        gather(nb2, bA);
        nb1 = nbr_of(t + 3);
        if constexpr (kAccGeoAhead) geo(t + 2, gA);
        __builtin_amdgcn_sched_barrier(0);
        run_step(t + 1, bB, gB);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (t < nslots) run_step(t, bA, gA);  // an odd last slot (its rows are in bA)
    }
    float v[K * TOT];
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
      for (int o = 0; o < TOT; ++o) v[k * TOT + o] = acc[k >> 2][o][k & 3];
    edge_slot_sum(v, ctl);
    store<0, 0, TOT, Ps...>(a, v, c, es == 0 && c_ok);
  }

};

#define TPCONV_PATH_CASES(X)                                                                                  \
  X(0, 0, 0) X(0, 1, 1) X(0, 2, 2) X(0, 3, 3) X(1, 0, 1) X(1, 1, 0) X(1, 1, 1) X(1, 1, 2) X(1, 2, 1)          \
  X(1, 2, 2) X(1, 2, 3) X(1, 3, 2) X(1, 3, 3) X(2, 0, 2) X(2, 1, 1) X(2, 1, 2) X(2, 1, 3) X(2, 2, 0)          \
  X(2, 2, 1) X(2, 2, 2) X(2, 2, 3) X(2, 3, 1) X(2, 3, 2) X(2, 3, 3) X(3, 0, 3) X(3, 1, 2) X(3, 1, 3)          \
  X(3, 2, 1) X(3, 2, 2) X(3, 2, 3) X(3, 3, 0) X(3, 3, 1) X(3, 3, 2) X(3, 3, 3)

// The argument block is read in place from the kernel-argument segment (it is
// the first argument, at offset 0).  Naming the by-value parameter instead
// would let the compiler copy the whole 2.7 KB block to scratch memory when
// the inlined code reads it in many places.

// Waves per SIMD the register allocation must leave room for: the lmax <= 2,
// K = 8 forward and sender streams fit three waves (168 registers) when asked
// to, which hides more of the gather latency than the compiler's own choice.
constexpr int stream_min_waves(int lmax, int K, int mode) {
  return (lmax <= 2 && K == 8 && (mode == kFwd || mode == kSnd)) ? 3 : 1;
}

// BUNDLED selects the natural path bundles or single-path units; the two are
// separate kernels so that each gets the register allocation of its own code
// (the single-path dispatch covers every path up to LMAX).
template <int LMAX, int K, int MODE, typename FT, bool BUNDLED>
__global__ __launch_bounds__(64)
__attribute__((amdgpu_waves_per_eu(stream_min_waves(LMAX, K, MODE))))
void stream_kernel(const StreamArgs /*args*/, int64_t items) {
  const StreamArgs& a = *(const StreamArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int BATCH = ModeTraits<MODE>::batch;
  __shared__ EdgeLds<K, LMAX, MODE, BATCH> L;
  // 32-bit index arithmetic (the launch keeps items below 2^31): a 64-bit
  // division here costs hundreds of instructions per wave.
  const uint32_t item = (uint32_t)xcd_item(blockIdx.x, gridDim.x);
  if (item >= (uint32_t)items) return;  // uniform over the block
  const uint32_t nu = (uint32_t)a.nunits, nt = (uint32_t)a.ntiles;
  const int unit = (int)(item % nu);
  const uint32_t t = item / nu;
  const int tile = (int)(t % nt);
  const int node = a.order ? a.order[t / nt] : (int)(t / nt);
  StreamCtx<MODE, FT, LMAX, K, BATCH> ctx{node, tile, unit, L};
  if constexpr (BUNDLED) {
    Bundles<LMAX, K, ModeTraits<MODE>::recv ? 0 : 1>::run(unit, ctx, a);
    return;
  }
  const StreamPath& P = a.paths[a.unit_paths[unit][0]];
  switch (P.l1 * 16 + P.l2 * 4 + P.l3) {
#define TPCONV_CASE(A, B, C)                                 \
  case A * 16 + B * 4 + C:                                   \
    if constexpr (A <= LMAX && B <= LMAX && C <= LMAX)       \
      ctx.template run<P3<A, B, C>>(a);                      \
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
  if (grid > INT32_MAX) return hipErrorInvalidValue;
#define TPCONV_LAUNCH(LM, KK)                                                                           \
  if (lmax == LM && K == KK) {                                                                          \
    if (a.bundled)                                                                                      \
      hipLaunchKernelGGL((stream_kernel<LM, KK, MODE, FT, true>), dim3((unsigned)grid), dim3(64), 0, s, a, items); \
    else                                                                                                \
      hipLaunchKernelGGL((stream_kernel<LM, KK, MODE, FT, false>), dim3((unsigned)grid), dim3(64), 0, s, a, items); \
    return hipGetLastError();                                                                           \
  }
  TPCONV_LAUNCH(0, 8) TPCONV_LAUNCH(0, 16)
  TPCONV_LAUNCH(1, 8) TPCONV_LAUNCH(1, 16)
  TPCONV_LAUNCH(2, 8) TPCONV_LAUNCH(2, 16)
  TPCONV_LAUNCH(3, 8) TPCONV_LAUNCH(3, 16)
#undef TPCONV_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace tpconv
