// Plan construction: irreps parsing, selection rules, real CG tables.
//
// Selection rules ("The Price of Freedom", Approach: interactability as the
// nonzero selection rules of the coupling): a path (l1,p1) x Y_l2 -> (l3,p3)
// exists iff |l1-l2| <= l3 <= l1+l2 and p1 * (-1)^l2 == p3.
//
// CG coefficients: Racah's single-sum closed form in long double, then the
// change of basis to real harmonics (m > 0: (Y^-m + (-1)^m Y^m)/sqrt2,
// m < 0: i (Y^m - (-1)^m Y^-m)/sqrt2).  For even l1+l2+l3 the real table is
// real; for odd it is purely imaginary and its imaginary part is kept.
#include "plan.h"

#include <cctype>
#include <cmath>
#include <complex>

#include "../../include/tpconv.h"

namespace tpconv {

namespace {

long double fact(int n) {
  long double r = 1.0L;
  for (int i = 2; i <= n; ++i) r *= (long double)i;
  return r;
}

// Complex-to-real matrix entry U^l[m][mu] (rows: real m, columns: complex mu).
std::complex<long double> u_entry(int l, int m, int mu) {
  const long double r2 = 1.0L / std::sqrt(2.0L);
  const long double sgn = (std::abs(m) % 2) ? -1.0L : 1.0L;  // (-1)^m
  if (m > 0) {
    if (mu == -m) return {r2, 0.0L};
    if (mu == m) return {sgn * r2, 0.0L};
    return {0.0L, 0.0L};
  }
  if (m < 0) {
    if (mu == m) return {0.0L, r2};
    if (mu == -m) return {0.0L, -sgn * r2};
    return {0.0L, 0.0L};
  }
  return (mu == 0) ? std::complex<long double>(1.0L, 0.0L) : std::complex<long double>(0.0L, 0.0L);
  (void)l;
}

}  // namespace

bool parse_irreps(const std::string& s, std::vector<Irrep>& out) {
  out.clear();
  size_t i = 0;
  const size_t n = s.size();
  auto skip = [&]() { while (i < n && std::isspace((unsigned char)s[i])) ++i; };
  while (true) {
    skip();
    if (i >= n || !std::isdigit((unsigned char)s[i])) return false;
    long v = 0;
    while (i < n && std::isdigit((unsigned char)s[i])) {
      v = v * 10 + (s[i] - '0');
      if (v > 1000000) return false;
      ++i;
    }
    skip();
    long mul = 1, l = v;
    if (i < n && s[i] == 'x') {
      ++i;
      skip();
      if (i >= n || !std::isdigit((unsigned char)s[i])) return false;
      mul = v;
      l = 0;
      while (i < n && std::isdigit((unsigned char)s[i])) {
        l = l * 10 + (s[i] - '0');
        if (l > 1000) return false;
        ++i;
      }
      skip();
    }
    if (i >= n || (s[i] != 'e' && s[i] != 'o')) return false;
    int parity = s[i] == 'e' ? 1 : -1;
    ++i;
    if (mul <= 0) return false;
    out.push_back({(int)mul, (int)l, parity});
    skip();
    if (i >= n) break;
    if (s[i] != '+') return false;
    ++i;
  }
  return !out.empty();
}

long double cg_complex(int j1, int m1, int j2, int m2, int J, int M) {
  if (m1 + m2 != M || std::abs(m1) > j1 || std::abs(m2) > j2 || std::abs(M) > J) return 0.0L;
  if (J < std::abs(j1 - j2) || J > j1 + j2) return 0.0L;
  long double pre = (2 * J + 1) * fact(J + j1 - j2) * fact(J - j1 + j2) * fact(j1 + j2 - J) /
                    fact(j1 + j2 + J + 1);
  pre *= fact(J + M) * fact(J - M) * fact(j1 - m1) * fact(j1 + m1) * fact(j2 - m2) * fact(j2 + m2);
  long double sum = 0.0L;
  for (int k = 0; k <= j1 + j2 - J; ++k) {
    const int a = j1 + j2 - J - k, b = j1 - m1 - k, c = j2 + m2 - k, d = J - j2 + m1 + k,
              e = J - j1 - m2 + k;
    if (a < 0 || b < 0 || c < 0 || d < 0 || e < 0) continue;
    const long double term = 1.0L / (fact(k) * fact(a) * fact(b) * fact(c) * fact(d) * fact(e));
    sum += (k % 2) ? -term : term;
  }
  return std::sqrt(pre) * sum;
}

bool real_cg(int l1, int l2, int l3, std::vector<double>& out) {
  if (l3 < std::abs(l1 - l2) || l3 > l1 + l2) return false;
  const int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
  // complex CG block
  std::vector<long double> cgc((size_t)n1 * n2 * n3, 0.0L);
  for (int a = -l1; a <= l1; ++a)
    for (int b = -l2; b <= l2; ++b) {
      const int c = a + b;
      if (std::abs(c) <= l3) cgc[((a + l1) * n2 + (b + l2)) * n3 + (c + l3)] = cg_complex(l1, a, l2, b, l3, c);
    }
  out.assign((size_t)n1 * n2 * n3, 0.0);
  const bool odd = (l1 + l2 + l3) % 2;
  for (int m1 = -l1; m1 <= l1; ++m1)
    for (int m2 = -l2; m2 <= l2; ++m2)
      for (int m3 = -l3; m3 <= l3; ++m3) {
        std::complex<long double> acc(0.0L, 0.0L);
        for (int a = -l1; a <= l1; ++a) {
          const auto u1 = u_entry(l1, m1, a);
          if (u1 == std::complex<long double>(0.0L, 0.0L)) continue;
          for (int b = -l2; b <= l2; ++b) {
            const auto u2 = u_entry(l2, m2, b);
            if (u2 == std::complex<long double>(0.0L, 0.0L)) continue;
            const int c = a + b;
            if (std::abs(c) > l3) continue;
            const auto u3 = std::conj(u_entry(l3, m3, c));
            acc += u1 * u2 * u3 * cgc[((a + l1) * n2 + (b + l2)) * n3 + (c + l3)];
          }
        }
        long double v = odd ? acc.imag() : acc.real();
        if (std::fabs(v) < 1e-15L) v = 0.0L;
        out[((m1 + l1) * n2 + (m2 + l2)) * n3 + (m3 + l3)] = (double)v;
      }
  return true;
}

std::vector<Path> natural_paths(int L) {
  std::vector<Path> out;
  for (int l1 = 0; l1 <= L; ++l1)
    for (int l2 = 0; l2 <= L; ++l2)
      for (int l3 = 0; l3 <= L; ++l3)
        if (l3 >= std::abs(l1 - l2) && l3 <= l1 + l2 && (l1 + l2 + l3) % 2 == 0)
          out.push_back(Path{l1, l1, l2, l3, l3, 0, 0});
  return out;
}

std::vector<std::vector<int>> natural_bundles(int L, int K, int side) {
  const std::vector<Path> paths = natural_paths(L);
  const bool receiver_side = side != kUnitsSend;
  const int cap = std::max(1, (side == kUnitsPos ? kPosUnitAccumulators : kUnitAccumulators) / K);
  std::vector<std::vector<int>> bundles;
  for (int g = 0; g <= L; ++g) {
    std::vector<int> cur;
    int sum = 0;
    for (int i = 0; i < (int)paths.size(); ++i) {
      const Path& p = paths[i];
      if ((receiver_side ? p.l1 : p.l3) != g) continue;
      const int n = 2 * (receiver_side ? p.l3 : p.l1) + 1;
      if (!cur.empty() && sum + n > cap) {
        bundles.push_back(cur);
        cur.clear();
        sum = 0;
      }
      cur.push_back(i);
      sum += n;
    }
    if (!cur.empty()) bundles.push_back(cur);
  }
  return bundles;
}

int build_plan(const char* irreps_in, const char* irreps_out, int sh_lmax, int K, float cutoff,
               int env_p, int x_dtype, int w_dtype, int connection, Plan& plan) {
  if (connection != TPCONV_FULLY_CONNECTED && connection != TPCONV_CHANNELWISE) return TPCONV_ERROR_INVALID_VALUE;
  if (!irreps_in || !irreps_out) return TPCONV_ERROR_INVALID_VALUE;
  if (K != 8 && K != 16) return TPCONV_ERROR_INVALID_VALUE;
  if (!(cutoff > 0.f) || !std::isfinite(cutoff) || env_p < 2 || env_p > 64) return TPCONV_ERROR_INVALID_VALUE;
  if ((x_dtype != TPCONV_F32 && x_dtype != TPCONV_BF16) || (w_dtype != TPCONV_F32 && w_dtype != TPCONV_BF16))
    return TPCONV_ERROR_INVALID_VALUE;
  if (sh_lmax < 0) return TPCONV_ERROR_INVALID_VALUE;
  Plan p;
  if (!parse_irreps(irreps_in, p.in) || !parse_irreps(irreps_out, p.out)) return TPCONV_ERROR_IRREPS;
  // Ragged multiplicities: keep the caller's layout, pad every irrep of a side
  // to its largest multiplicity (the channel-wise product pads both sides to
  // one count, since it pairs input and output channels).
  for (const auto& ir : p.in) p.rag.mul_in.push_back(ir.mul);
  for (const auto& ir : p.out) p.rag.mul_out.push_back(ir.mul);
  for (const auto& v : {&p.in, &p.out})
    for (const auto& ir : *v)
      if (ir.mul != (*v)[0].mul) p.ragged = true;
  if (p.ragged) {
    int cin = 0, cout = 0;
    for (const auto& ir : p.in) cin = std::max(cin, ir.mul);
    for (const auto& ir : p.out) cout = std::max(cout, ir.mul);
    if (connection == TPCONV_CHANNELWISE) cin = cout = std::max(cin, cout);
    for (auto& ir : p.in) ir.mul = cin;
    for (auto& ir : p.out) ir.mul = cout;
    int64_t o = 0;
    for (size_t i = 0; i < p.in.size(); ++i) {
      p.rag.foff_in.push_back(o);
      o += (int64_t)(2 * p.in[i].l + 1) * p.rag.mul_in[i];
    }
    p.rag.F_in = o;
    o = 0;
    for (size_t i = 0; i < p.out.size(); ++i) {
      p.rag.foff_out.push_back(o);
      o += (int64_t)(2 * p.out[i].l + 1) * p.rag.mul_out[i];
    }
    p.rag.F_out = o;
  }
  int lmax = sh_lmax;
  for (const auto& ir : p.in) lmax = std::max(lmax, ir.l);
  for (const auto& ir : p.out) lmax = std::max(lmax, ir.l);
  if (lmax > kMaxL) return TPCONV_ERROR_UNSUPPORTED;
  if ((int)p.in.size() > kMaxGroups || (int)p.out.size() > kMaxGroups) return TPCONV_ERROR_UNSUPPORTED;
  p.sh_lmax = sh_lmax;
  p.K = K;
  p.cutoff = cutoff;
  p.env_p = env_p;
  p.x_dtype = x_dtype;
  p.w_dtype = w_dtype;
  p.C_in = p.in[0].mul;
  p.C_out = p.out[0].mul;
  p.connection = connection;
  if (connection == TPCONV_CHANNELWISE && p.C_in != p.C_out) return TPCONV_ERROR_IRREPS;
  p.lmax = lmax;
  p.D_in = p.D_out = 0;
  p.in_groups.resize(p.in.size());
  p.out_groups.resize(p.out.size());
  for (size_t i = 0; i < p.in.size(); ++i) {
    p.in_groups[i].irrep = (int)i;
    p.in_groups[i].l = p.in[i].l;
    p.in_groups[i].row_off = p.D_in;
    p.D_in += 2 * p.in[i].l + 1;
  }
  for (size_t i = 0; i < p.out.size(); ++i) {
    p.out_groups[i].irrep = (int)i;
    p.out_groups[i].l = p.out[i].l;
    p.out_groups[i].row_off = p.D_out;
    p.D_out += 2 * p.out[i].l + 1;
  }
  for (size_t i1 = 0; i1 < p.in.size(); ++i1) {
    const int l1 = p.in[i1].l, p1 = p.in[i1].parity;
    for (int l2 = 0; l2 <= sh_lmax; ++l2) {
      const int p2 = (l2 % 2) ? -1 : 1;
      for (size_t i3 = 0; i3 < p.out.size(); ++i3) {
        const int l3 = p.out[i3].l, p3 = p.out[i3].parity;
        if (l3 < std::abs(l1 - l2) || l3 > l1 + l2 || p1 * p2 != p3) continue;
        Path path{(int)i1, l1, l2, (int)i3, l3, 0, 0};
        path.q_out = (int)p.out_groups[i3].paths.size();
        path.q_in = (int)p.in_groups[i1].paths.size();
        p.out_groups[i3].paths.push_back((int)p.paths.size());
        p.in_groups[i1].paths.push_back((int)p.paths.size());
        p.paths.push_back(path);
      }
    }
  }
  p.P = (int)p.paths.size();
  if (p.P > kMaxPaths) return TPCONV_ERROR_UNSUPPORTED;
  if (p.ragged) {
    int64_t o = 0;
    for (const auto& q : p.paths) {
      const int c1 = p.rag.mul_in[q.i1], c3 = p.rag.mul_out[q.i3];
      if (connection == TPCONV_CHANNELWISE && c1 != c3) return TPCONV_ERROR_IRREPS;
      p.rag.woff.push_back(o);
      o += connection == TPCONV_CHANNELWISE ? c1 : (int64_t)c1 * c3;
    }
    p.rag.W_per_k = o;
  }
  p.cg.resize(p.P);
  for (int i = 0; i < p.P; ++i) real_cg(p.paths[i].l1, p.paths[i].l2, p.paths[i].l3, p.cg[i]);
  int64_t off = 0;
  for (auto& g : p.out_groups) {
    g.base_per_node = off;
    off += (int64_t)(2 * g.l + 1) * K * (int64_t)g.paths.size() * p.C_in;
  }
  p.state_in_per_node = off;
  off = 0;
  for (auto& g : p.in_groups) {
    g.base_per_node = off;
    off += (int64_t)(2 * g.l + 1) * K * (int64_t)g.paths.size() * p.C_out;
  }
  p.state_out_per_node = off;
  // natural irreps: irrep i has degree i and parity (-1)^i on both sides, harmonics up to L
  auto is_natural = [&](const std::vector<Irrep>& v) {
    if ((int)v.size() != lmax + 1) return false;
    for (int i = 0; i <= lmax; ++i)
      if (v[i].l != i || v[i].parity != ((i % 2) ? -1 : 1)) return false;
    return true;
  };
  p.natural = is_natural(p.in) && is_natural(p.out) && sh_lmax == lmax;
  if (p.natural) {
    p.recv_units = natural_bundles(lmax, K, kUnitsRecv);
    p.send_units = natural_bundles(lmax, K, kUnitsSend);
    p.pos_units = natural_bundles(lmax, K, kUnitsPos);
    for (const auto* us : {&p.recv_units, &p.send_units, &p.pos_units})
      for (const auto& u : *us)
        if ((int)u.size() > 8) p.natural = false;  // more members than a unit holds
  }
  if (!p.natural) {
    p.recv_units.clear();
    p.send_units.clear();
    p.pos_units.clear();
    for (int i = 0; i < p.P; ++i) {
      p.recv_units.push_back({i});
      p.send_units.push_back({i});
      p.pos_units.push_back({i});
    }
  }
  plan = std::move(p);
  return TPCONV_SUCCESS;
}

}  // namespace tpconv
