// Device helpers: the bf16 hi + lo split, XCD-aware block order, edge
// geometry (radial basis, real harmonics and their derivatives) in fp32.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tpconv {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// The bf16 pairs (-1, 0) and (0, -1) for split8, held in scalar registers.
// As literals the compiler encodes (-1, 0) as the 32-bit inline constant -1.0,
// which the hardware reads as (0, -1); opaque register values avoid that.
struct SplitConsts {
  bf16x2 neg_x, neg_y;
  __device__ __forceinline__ SplitConsts() {
    uint32_t x = 0x0000bf80u, y = 0xbf800000u;
    asm volatile("" : "+s"(x), "+s"(y));
    neg_x = __builtin_bit_cast(bf16x2, x);
    neg_y = __builtin_bit_cast(bf16x2, y);
  }
};

// hi / lo bf16 split of eight fp32 values: hi rounds to nearest even, and
// lo = v - hi, exact in fp32, comes from a bf16 dot product of hi with
// (-1, 0) or (0, -1) accumulated onto v, then rounds again.
__device__ __forceinline__ void split8(const float (&v)[8], u32x4& hi, u32x4& lo, const SplitConsts& k) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const bf16x2 h = {(__bf16)v[2 * t], (__bf16)v[2 * t + 1]};
    const float l0 = __builtin_amdgcn_fdot2_f32_bf16(h, k.neg_x, v[2 * t], false);
    const float l1 = __builtin_amdgcn_fdot2_f32_bf16(h, k.neg_y, v[2 * t + 1], false);
    const bf16x2 l = {(__bf16)l0, (__bf16)l1};
    hi[t] = __builtin_bit_cast(uint32_t, h);
    lo[t] = __builtin_bit_cast(uint32_t, l);
  }
}

__device__ __forceinline__ float load_feat(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_feat(const uint16_t* p, int64_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}

// Blocks are handed to the 8 XCDs round-robin (block b runs on XCD b % 8).
// Remap so that consecutive work items share an XCD and therefore its L2:
// item = (b % 8) * (grid / 8) + b / 8.  grid must be a multiple of 8.
__device__ __forceinline__ int64_t xcd_item(int64_t b, int64_t grid) {
  const int64_t per = grid >> 3;
  return (b & 7) * per + (b >> 3);
}

// Bessel radial basis with the polynomial envelope, fp32.
//   R_k(d)  = pref sin(k w d) / d * u(d / c),  w = pi / c
//   R'_k(d) = pref [(k w) cos(k w d) / d - sin(k w d) / d^2] u + pref sin(k w d) / d * u'(d/c) / c
// sin/cos of k w d come from one sincos and the angle-addition recurrence.
template <int K, bool DERIV>
__device__ __forceinline__ void radial(float d, float cutoff, float inv_cutoff, float pref, int p, float ea,
                                       float eb, float ec, float ed, float* R, float* dR) {
  const float w = 3.14159265358979f * inv_cutoff;
  if (d <= 0.f) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      R[k] = pref * w * (float)(k + 1);
      if (DERIV) dR[k] = 0.f;
    }
    return;
  }
  const float x = d * inv_cutoff;
  if (x >= 1.f) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      R[k] = 0.f;
      if (DERIV) dR[k] = 0.f;
    }
    return;
  }
  float xp1 = 1.f;  // x^(p-1)
  for (int i = 0; i < p - 1; ++i) xp1 *= x;
  const float xp = xp1 * x;
  const float u = 1.f - ea * xp + eb * xp * x - ec * xp * x * x;
  const float omx = 1.f - x;
  const float du = -ed * xp1 * omx * omx * inv_cutoff;  // du/dd
  float s1, c1;
  __sincosf(w * d, &s1, &c1);
  const float inv_d = 1.f / d;
  float sk = s1, ck = c1;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const float b = pref * sk * inv_d;
    R[k] = b * u;
    if (DERIV) {
      const float db = pref * ((float)(k + 1) * w * ck * inv_d - sk * inv_d * inv_d);
      dR[k] = db * u + b * du;
    }
    const float sn = sk * c1 + ck * s1;
    const float cn = ck * c1 - sk * s1;
    sk = sn;
    ck = cn;
  }
}

// R, R' and R'' of the Bessel basis (the position derivative of the force
// loss): with f = sin(k w d) / d and u = u(d / c),
//   R = pref f u,  R' = pref (f' u + f u_d),  R'' = pref (f'' u + 2 f' u_d + f u_dd),
//   f' = k w cos / d - sin / d^2,  f'' = -(k w)^2 sin / d - 2 k w cos / d^2 + 2 sin / d^3,
//   u_d = u'(x) / c,  u_dd = u''(x) / c^2,  u''(x) = -ed [(p-1) x^(p-2) (1-x)^2 - 2 x^(p-1) (1-x)].
// At d = 0 (limit R, R' = R'' = 0) and d >= c (all 0) as in radial().
template <int K>
__device__ __forceinline__ void radial2(float d, float inv_cutoff, float pref, int p, float ea, float eb, float ec,
                                        float ed, float* R, float* dR, float* d2R) {
  const float w = 3.14159265358979f * inv_cutoff;
  const float x = d * inv_cutoff;
  if (d <= 0.f || x >= 1.f) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      R[k] = d <= 0.f ? pref * w * (float)(k + 1) : 0.f;
      dR[k] = 0.f;
      d2R[k] = 0.f;
    }
    return;
  }
  float xp2 = 1.f;  // x^(p-2)
  for (int i = 0; i < p - 2; ++i) xp2 *= x;
  const float xp1 = xp2 * x, xp = xp1 * x;
  const float u = 1.f - ea * xp + eb * xp * x - ec * xp * x * x;
  const float omx = 1.f - x;
  const float ud = -ed * xp1 * omx * omx * inv_cutoff;
  const float udd = -ed * ((float)(p - 1) * xp2 * omx * omx - 2.f * xp1 * omx) * inv_cutoff * inv_cutoff;
  float s1, c1;
  __sincosf(w * d, &s1, &c1);
  const float inv_d = 1.f / d;
  float sk = s1, ck = c1;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const float kw = (float)(k + 1) * w;
    const float f = sk * inv_d;
    const float f1 = (kw * ck - f) * inv_d;
    const float f2 = (-kw * kw * sk - 2.f * f1) * inv_d;
    R[k] = pref * f * u;
    dR[k] = pref * (f1 * u + f * ud);
    d2R[k] = pref * (f2 * u + 2.f * f1 * ud + f * udd);
    const float sn = sk * c1 + ck * s1;
    const float cn = ck * c1 - sk * s1;
    sk = sn;
    ck = cn;
  }
}

// v * 2^F as a 64-bit two's complement integer modulo 2^64: exact for the
// bits of v at or above 2^-F, the lower ones dropped (toward zero).  Sums of
// such values are exact modulo 2^64, so they do not depend on the order of
// the additions; the result is right when the true sum times 2^F stays
// within +-2^63.
__device__ __forceinline__ unsigned long long to_fixed(float v, int F) {
  const uint32_t bits = __float_as_uint(v);
  const int e = (int)((bits >> 23) & 0xffu);
  if (e == 0) return 0ull;  // zero and subnormals (far below any scale used)
  const unsigned long long m = (unsigned long long)((bits & 0x7fffffu) | 0x800000u);
  const int sh = e - 150 + F;  // v = m * 2^(e - 150)
  unsigned long long q = 0ull;
  if (sh >= 0)
    q = sh < 64 ? m << sh : 0ull;
  else
    q = -sh < 64 ? m >> -sh : 0ull;
  return (bits >> 31) ? 0ull - q : q;
}

// Radial MLP on the basis, in place: the basis values B, B', B'' (from
// radial / radial2) become those of the network's last hidden layer,
//   z_k = sum_j A[k K + j] B_j,  R_k = silu(z_k),  R'_k = silu'(z_k) z'_k,
//   R''_k = silu''(z_k) z'_k^2 + silu'(z_k) z''_k,   silu(z) = z sigmoid(z),
// or, with col = j >= 0, their derivatives with respect to A[k, j] (what the
// weight gradient of the network needs): R_k = silu'(z_k) B_j and
// R'_k = silu''(z_k) z'_k B_j + silu'(z_k) B'_j.  ORDER: how many derivatives
// in d are carried (0: R, 1: R and R', 2: R, R' and R'', col < 0 only).  At
// the cutoff and beyond B = 0, so R = R' = R'' = 0; at d = 0, B' = B'' = 0.
template <int K, int ORDER>
__device__ __forceinline__ void mlp_radial(const float* __restrict__ A, int col, float* R, float* dR, float* d2R) {
  float B[K], B1[ORDER >= 1 ? K : 1], B2[ORDER >= 2 ? K : 1];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    B[j] = R[j];
    if constexpr (ORDER >= 1) B1[j] = dR[j];
    if constexpr (ORDER >= 2) B2[j] = d2R[j];
  }
  // B_col and B'_col by selects (a register array is never indexed at run time)
  float bc = 0.f, bc1 = 0.f;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    bc = j == col ? B[j] : bc;
    if constexpr (ORDER >= 1) bc1 = j == col ? B1[j] : bc1;
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    float z = 0.f, z1 = 0.f, z2 = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float a = A[k * K + j];
      z = __builtin_fmaf(a, B[j], z);
      if constexpr (ORDER >= 1) z1 = __builtin_fmaf(a, B1[j], z1);
      if constexpr (ORDER >= 2) z2 = __builtin_fmaf(a, B2[j], z2);
    }
    const float sg = 1.f / (1.f + __expf(-z));
    const float s1 = sg * (1.f + z * (1.f - sg));
    const float s2 = sg * (1.f - sg) * (2.f + z * (1.f - 2.f * sg));
    if (col < 0) {
      R[k] = z * sg;
      if constexpr (ORDER >= 1) dR[k] = s1 * z1;
      if constexpr (ORDER >= 2) d2R[k] = s2 * z1 * z1 + s1 * z2;
    } else {
      R[k] = s1 * bc;
      if constexpr (ORDER >= 1) dR[k] = s2 * z1 * bc + s1 * bc1;
    }
  }
}

// Real harmonics of a unit vector (x, y, z), component normalised, rows l^2 + l + m.
template <int L>
__device__ __forceinline__ void sh_eval(float x, float y, float z, float* Y) {
  Y[0] = 1.f;
  if (L >= 1) {
    const float s3 = 1.7320508075688772f;
    Y[1] = s3 * y;
    Y[2] = s3 * z;
    Y[3] = s3 * x;
  }
  if (L >= 2) {
    const float s15 = 3.872983346207417f, s5 = 2.23606797749979f;
    Y[4] = s15 * x * y;
    Y[5] = s15 * y * z;
    Y[6] = 0.5f * s5 * (2.f * z * z - x * x - y * y);
    Y[7] = s15 * x * z;
    Y[8] = 0.5f * s15 * (x * x - y * y);
  }
  if (L >= 3) {
    const float a = 0.25f * 8.366600265340756f, b = 0.25f * 6.48074069840786f, s105 = 10.246950765959598f,
                s7 = 2.6457513110645907f;
    Y[9] = a * y * (3.f * x * x - y * y);
    Y[10] = s105 * x * y * z;
    Y[11] = b * y * (4.f * z * z - x * x - y * y);
    Y[12] = 0.5f * s7 * z * (2.f * z * z - 3.f * x * x - 3.f * y * y);
    Y[13] = b * x * (4.f * z * z - x * x - y * y);
    Y[14] = 0.5f * s105 * z * (x * x - y * y);
    Y[15] = a * x * (x * x - 3.f * y * y);
  }
}

// Gradients of the homogeneous polynomials P_lm at the unit vector: G[row][3].
template <int L>
__device__ __forceinline__ void sh_poly_grad(float x, float y, float z, float (*G)[3]) {
  G[0][0] = G[0][1] = G[0][2] = 0.f;
  if (L >= 1) {
    const float s3 = 1.7320508075688772f;
    G[1][0] = 0.f; G[1][1] = s3;  G[1][2] = 0.f;
    G[2][0] = 0.f; G[2][1] = 0.f; G[2][2] = s3;
    G[3][0] = s3;  G[3][1] = 0.f; G[3][2] = 0.f;
  }
  if (L >= 2) {
    const float s15 = 3.872983346207417f, s5 = 2.23606797749979f;
    G[4][0] = s15 * y;  G[4][1] = s15 * x;  G[4][2] = 0.f;
    G[5][0] = 0.f;      G[5][1] = s15 * z;  G[5][2] = s15 * y;
    G[6][0] = -s5 * x;  G[6][1] = -s5 * y;  G[6][2] = 2.f * s5 * z;
    G[7][0] = s15 * z;  G[7][1] = 0.f;      G[7][2] = s15 * x;
    G[8][0] = s15 * x;  G[8][1] = -s15 * y; G[8][2] = 0.f;
  }
  if (L >= 3) {
    const float a = 0.25f * 8.366600265340756f, b = 0.25f * 6.48074069840786f, s105 = 10.246950765959598f,
                h7 = 0.5f * 2.6457513110645907f, h105 = 0.5f * 10.246950765959598f;
    G[9][0] = a * 6.f * x * y;  G[9][1] = a * 3.f * (x * x - y * y);  G[9][2] = 0.f;
    G[10][0] = s105 * y * z;    G[10][1] = s105 * x * z;              G[10][2] = s105 * x * y;
    G[11][0] = -2.f * b * x * y;
    G[11][1] = b * (4.f * z * z - x * x - 3.f * y * y);
    G[11][2] = 8.f * b * y * z;
    G[12][0] = -6.f * h7 * x * z;
    G[12][1] = -6.f * h7 * y * z;
    G[12][2] = h7 * (6.f * z * z - 3.f * x * x - 3.f * y * y);
    G[13][0] = b * (4.f * z * z - 3.f * x * x - y * y);
    G[13][1] = -2.f * b * x * y;
    G[13][2] = 8.f * b * x * z;
    G[14][0] = 2.f * h105 * x * z;  G[14][1] = -2.f * h105 * y * z;  G[14][2] = h105 * (x * x - y * y);
    G[15][0] = a * 3.f * (x * x - y * y);  G[15][1] = -a * 6.f * x * y;  G[15][2] = 0.f;
  }
}

// H_P(u) phi for the Hessians H_P of the homogeneous polynomials P_lm at the
// unit vector u = (x, y, z) (constant for l = 2, linear for l = 3): out[row][3].
template <int L>
__device__ __forceinline__ void sh_poly_hess_dir(float x, float y, float z, float fx, float fy, float fz,
                                                 float (*out)[3]) {
  auto sym = [&](float (&o)[3], float xx, float xy, float xz, float yy, float yz, float zz) {
    o[0] = xx * fx + xy * fy + xz * fz;
    o[1] = xy * fx + yy * fy + yz * fz;
    o[2] = xz * fx + yz * fy + zz * fz;
  };
  for (int r = 0; r < (L < 1 ? 1 : 4); ++r) out[r][0] = out[r][1] = out[r][2] = 0.f;
  if (L >= 2) {
    const float s15 = 3.872983346207417f, s5 = 2.23606797749979f;
    sym(out[4], 0.f, s15, 0.f, 0.f, 0.f, 0.f);
    sym(out[5], 0.f, 0.f, 0.f, 0.f, s15, 0.f);
    sym(out[6], -s5, 0.f, 0.f, -s5, 0.f, 2.f * s5);
    sym(out[7], 0.f, 0.f, s15, 0.f, 0.f, 0.f);
    sym(out[8], s15, 0.f, 0.f, -s15, 0.f, 0.f);
  }
  if (L >= 3) {
    const float a = 0.25f * 8.366600265340756f, b = 0.25f * 6.48074069840786f, s105 = 10.246950765959598f,
                c = 0.5f * 2.6457513110645907f, e = 0.5f * 10.246950765959598f;
    sym(out[9], 6.f * a * y, 6.f * a * x, 0.f, -6.f * a * y, 0.f, 0.f);
    sym(out[10], 0.f, s105 * z, s105 * y, 0.f, s105 * x, 0.f);
    sym(out[11], -2.f * b * y, -2.f * b * x, 0.f, -6.f * b * y, 8.f * b * z, 8.f * b * y);
    sym(out[12], -6.f * c * z, 0.f, -6.f * c * x, -6.f * c * z, -6.f * c * y, 12.f * c * z);
    sym(out[13], -6.f * b * x, -2.f * b * y, 8.f * b * z, -2.f * b * x, 0.f, 8.f * b * x);
    sym(out[14], 2.f * e * z, 0.f, 2.f * e * x, -2.f * e * z, -2.f * e * y, 0.f);
    sym(out[15], 6.f * a * x, -6.f * a * y, 0.f, -6.f * a * x, 0.f, 0.f);
  }
}

constexpr int sh_count(int L) { return (L + 1) * (L + 1); }
constexpr int sh_degree_of_row(int row) {
  return row == 0 ? 0 : row < 4 ? 1 : row < 9 ? 2 : 3;
}

}  // namespace tpconv
