// Device helpers: feature loads, XCD-aware block order, edge geometry
// (radial basis, real harmonics and their derivatives) in fp32.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tpconv {

__device__ __forceinline__ float load_feat(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_feat(const uint16_t* p, int64_t i) {
  return __uint_as_float(((uint32_t)p[i]) << 16);
}
// Gathered features are kept in their stored form until they are used, and
// widened to fp32 only there: a conversion placed at the load would make the
// compiler wait for that load and defeat the prefetch pipelines.
template <typename FT> struct FeatRaw;
template <> struct FeatRaw<float> {
  typedef float type;
  __device__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ static float f32(float v) { return v; }
};
template <> struct FeatRaw<uint16_t> {
  typedef uint32_t type;
  __device__ static uint32_t load(const uint16_t* p, int64_t i) { return p[i]; }
  __device__ static float f32(uint32_t v) { return __uint_as_float(v << 16); }
};

// Four consecutive channels of NIN rows, raw.  `base` indexes the first row's
// first channel; with vec4 (C a multiple of 4, c0 too) each row is one 16-byte
// (fp32) or 8-byte (bf16) load.  Otherwise each channel is read on its own and
// channels past C are zero (that path waits for its loads; it only serves
// channel counts that are not multiples of 4).
template <typename FT, int NIN> struct Quads;
template <int NIN> struct Quads<float, NIN> {
  float v[NIN][4];
  __device__ __forceinline__ void load(const float* p, int64_t base, int C, int c0, bool vec4) {
    if (vec4) {
      typedef float f4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int m = 0; m < NIN; ++m) {
        const f4 x = *reinterpret_cast<const f4*>(p + base + (int64_t)m * C);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[m][i] = x[i];
      }
    } else {
#pragma unroll
      for (int m = 0; m < NIN; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          v[m][i] = c0 + i < C ? p[base + (int64_t)m * C + min(i, C - 1 - c0)] : 0.f;
    }
  }
  // fp32: the raw rows already are the values, [row][channel]
  __device__ __forceinline__ const float (&get(float (&)[NIN][4]) const)[NIN][4] { return v; }
};
template <int NIN> struct Quads<uint16_t, NIN> {
  uint32_t w[NIN][2];  // channels (c0, c0+1) and (c0+2, c0+3), low half first
  __device__ __forceinline__ void load(const uint16_t* p, int64_t base, int C, int c0, bool vec4) {
    if (vec4) {
#pragma unroll
      for (int m = 0; m < NIN; ++m) {
        const uint2 u = *reinterpret_cast<const uint2*>(p + base + (int64_t)m * C);
        w[m][0] = u.x;
        w[m][1] = u.y;
      }
    } else {  // rare: pack four clamped channels
#pragma unroll
      for (int m = 0; m < NIN; ++m) {
        const uint16_t* r = p + base + (int64_t)m * C;
        const int l = C - 1 - c0;
        w[m][0] = (uint32_t)r[0] | (l >= 1 ? (uint32_t)r[1] << 16 : 0u);
        w[m][1] = (l >= 2 ? (uint32_t)r[2] : 0u) | (l >= 3 ? (uint32_t)r[3] << 16 : 0u);
      }
    }
  }
  // bf16: widen into x, [row][channel]
  __device__ __forceinline__ const float (&get(float (&x)[NIN][4]) const)[NIN][4] {
#pragma unroll
    for (int m = 0; m < NIN; ++m) {
      x[m][0] = __uint_as_float(w[m][0] << 16);
      x[m][1] = __uint_as_float(w[m][0] & 0xffff0000u);
      x[m][2] = __uint_as_float(w[m][1] << 16);
      x[m][3] = __uint_as_float(w[m][1] & 0xffff0000u);
    }
    return x;
  }
};

// Four consecutive features p[i..i+3]; i must be a multiple of 4.
__device__ __forceinline__ void load_feat4(const float* p, int64_t i, float (&v)[4]) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4 x = *reinterpret_cast<const f4*>(p + i);
  v[0] = x[0];
  v[1] = x[1];
  v[2] = x[2];
  v[3] = x[3];
}
__device__ __forceinline__ void load_feat4(const uint16_t* p, int64_t i, float (&v)[4]) {
  const uint2 u = *reinterpret_cast<const uint2*>(p + i);
  v[0] = __uint_as_float(u.x << 16);
  v[1] = __uint_as_float(u.x & 0xffff0000u);
  v[2] = __uint_as_float(u.y << 16);
  v[3] = __uint_as_float(u.y & 0xffff0000u);
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

constexpr int sh_count(int L) { return (L + 1) * (L + 1); }
constexpr int sh_degree_of_row(int row) {
  return row == 0 ? 0 : row < 4 ? 1 : row < 9 ? 2 : 3;
}

}  // namespace tpconv
