// Host-side exercise of the C ABI for an AddressSanitizer / UBSan build of the
// plan builder and the API's argument checks.  It touches no device memory:
// every forward / backward call below must be rejected on the host before any
// launch.  Exit status 0 when every check holds; the sanitizers abort on the
// first memory or undefined-behaviour error.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "tpconv.h"

static int failures = 0;
#define CHECK(cond)                                                    \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "check failed (line %d): %s\n", __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static tpconv_desc desc(const char* in, const char* out, int sh, int K, int conn = 0, int xd = 0, int wd = 0) {
  tpconv_desc d{};
  d.irreps_in = in;
  d.irreps_out = out;
  d.sh_lmax = sh;
  d.num_basis = K;
  d.cutoff = 5.f;
  d.envelope_p = 6;
  d.x_dtype = xd;
  d.w_dtype = wd;
  d.connection = conn;
  return d;
}

// Every query a plan answers on the host, checked for consistency.
static void exercise(tpconv_plan p) {
  int32_t P = 0, ri = 0, ci = 0, ro = 0, co = 0;
  int64_t wn = 0, fi = 0, fo = 0;
  CHECK(tpconv_plan_info(p, &P, &wn, &ri, &ci, &ro, &co) == TPCONV_SUCCESS);
  CHECK(tpconv_plan_features(p, &fi, &fo) == TPCONV_SUCCESS);
  CHECK(P > 0 && wn > 0 && fi > 0 && fo > 0);
  for (int i = 0; i < P; ++i) {
    int32_t l[3], idx[2];
    CHECK(tpconv_plan_path(p, i, l, idx) == TPCONV_SUCCESS);
    std::vector<double> cg((2 * l[0] + 1) * (2 * l[1] + 1) * (2 * l[2] + 1));
    CHECK(tpconv_plan_cg(p, i, cg.data()) == TPCONV_SUCCESS);
    double s = 0;
    for (double v : cg) s += v * v;
    CHECK(s > 0 && std::isfinite(s));
  }
  int32_t l[3], idx[2];
  CHECK(tpconv_plan_path(p, P, l, idx) == TPCONV_ERROR_INVALID_VALUE);
  CHECK(tpconv_plan_path(p, -1, l, idx) == TPCONV_ERROR_INVALID_VALUE);
  for (int op = 0; op <= 5; ++op)
    for (int64_t N : {0, 1, 1000, 100000}) {
      size_t b = 1;
      CHECK(tpconv_workspace_size(p, op, N, 4 * N, &b) == TPCONV_SUCCESS);
    }
  size_t b = 0;
  CHECK(tpconv_workspace_size(p, 99, 10, 10, &b) == TPCONV_ERROR_INVALID_VALUE);
  CHECK(tpconv_workspace_size(p, 0, -1, 10, &b) == TPCONV_ERROR_INVALID_VALUE);
  CHECK(tpconv_state_size(p, 77, &b) == TPCONV_SUCCESS);

  // argument errors caught before any device work
  tpconv_graph g{};
  g.num_nodes = 4;
  g.num_edges = 4;
  float dummy[4];
  CHECK(tpconv_forward(p, nullptr, dummy, dummy, dummy, dummy, nullptr, nullptr, 0, nullptr) != TPCONV_SUCCESS);
  CHECK(tpconv_forward(p, &g, nullptr, dummy, dummy, dummy, nullptr, nullptr, 0, nullptr) != TPCONV_SUCCESS);
  CHECK(tpconv_backward(p, &g, dummy, dummy, dummy, dummy, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                        nullptr) != TPCONV_SUCCESS);
  CHECK(tpconv_double_backward(p, &g, dummy, dummy, dummy, dummy, dummy, nullptr, nullptr, nullptr, nullptr,
                               nullptr, 0, nullptr) != TPCONV_SUCCESS);
  g.num_nodes = -1;
  CHECK(tpconv_graph_prepare(p, &g, nullptr, nullptr, 0, nullptr, 0, nullptr) != TPCONV_SUCCESS);
  CHECK(tpconv_graph_order(p, &g, dummy, nullptr, nullptr, 0, nullptr) != TPCONV_SUCCESS);
}

int main() {
  struct Case {
    const char *in, *out;
    int sh, K, conn, xd, wd;
  };
  const Case good[] = {
      {"8x0e+8x1o", "8x0e+8x1o", 1, 8, 0, 0, 0},
      {"32x0e+32x1o+32x2e", "32x0e+32x1o+32x2e", 2, 8, 0, 0, 0},
      {"64x0e+64x1o+64x2e+64x3o", "64x0e+64x1o+64x2e+64x3o", 3, 8, 0, 1, 1},
      {"128x0e+128x1o+128x2e", "128x0e+128x1o+128x2e", 2, 16, 0, 0, 0},
      {"32x0e+32x1o+32x2e", "32x0e+32x1o+32x2e", 2, 8, 1, 0, 0},
      {"64x0e+32x1o+16x2e", "16x0e+24x1o+40x2e", 2, 8, 0, 0, 1},
      {"4x0e+4x1o+4x1e+4x2e", "4x0e+4x0o+4x1o+4x1e+4x2e+4x3o", 2, 8, 0, 1, 0},
      {"8x0e", "8x0e+8x1e", 1, 8, 0, 0, 0},
      {"1x3o", "1x0e+1x0o+1x1e+1x1o+1x2e+1x2o+1x3e+1x3o", 3, 16, 0, 0, 0},
  };
  for (const Case& c : good) {
    tpconv_desc d = desc(c.in, c.out, c.sh, c.K, c.conn, c.xd, c.wd);
    tpconv_plan p = nullptr;
    const tpconv_status st = tpconv_plan_create(&p, &d);
    CHECK(st == TPCONV_SUCCESS);
    if (st == TPCONV_SUCCESS) {
      exercise(p);
      CHECK(tpconv_plan_destroy(p) == TPCONV_SUCCESS);
    }
  }
  // malformed or unsupported descriptors: rejected, no plan leaked
  const char* bad_irreps[] = {"", "x", "8x", "8x0", "8x0q", "8x4e", "0x0e", "-1x0e", "8x0e+", "+8x0e",
                              "8x0e++8x1o", "99999999999x0e", "8x0e 8x1o", "8x1o+8x0e+8x1o+8x2e+8x3o+8x0o+8x1e+8x2o+"
                              "8x3e+8x0e+8x1o+8x2e+8x3o+8x0o+8x1e+8x2o+8x3e"};
  for (const char* s : bad_irreps) {
    tpconv_desc d = desc(s, "8x0e", 1, 8);
    tpconv_plan p = nullptr;
    const tpconv_status st = tpconv_plan_create(&p, &d);
    CHECK(st != TPCONV_SUCCESS);
    if (st == TPCONV_SUCCESS) tpconv_plan_destroy(p);
  }
  tpconv_desc d = desc("8x0e", "8x0e", 1, 8);
  tpconv_plan p = nullptr;
  CHECK(tpconv_plan_create(nullptr, &d) == TPCONV_ERROR_INVALID_VALUE);
  CHECK(tpconv_plan_create(&p, nullptr) == TPCONV_ERROR_INVALID_VALUE);
  d.num_basis = 12;
  CHECK(tpconv_plan_create(&p, &d) == TPCONV_ERROR_INVALID_VALUE);
  d = desc("8x0e", "8x0e", 4, 8);
  CHECK(tpconv_plan_create(&p, &d) != TPCONV_SUCCESS);
  d = desc("8x0e", "8x0e", 1, 8);
  d.cutoff = -1.f;
  CHECK(tpconv_plan_create(&p, &d) == TPCONV_ERROR_INVALID_VALUE);
  d = desc("8x0e", "8x0e", 1, 8);
  d.envelope_p = 1;
  CHECK(tpconv_plan_create(&p, &d) == TPCONV_ERROR_INVALID_VALUE);
  d = desc("8x0e", "8x0e", 1, 8, 7);
  CHECK(tpconv_plan_create(&p, &d) == TPCONV_ERROR_INVALID_VALUE);
  // radial MLP plans: the MLP entry points need radial_w, the plain ones refuse the plan
  {
    tpconv_desc dm = desc("8x0e+8x1o+8x2e", "8x0e+8x1o+8x2e", 2, 8);
    dm.radial_mlp = 1;
    tpconv_plan pm = nullptr;
    CHECK(tpconv_plan_create(&pm, &dm) == TPCONV_SUCCESS);
    if (pm) {
      exercise(pm);
      tpconv_graph g{};
      g.num_nodes = 4;
      g.num_edges = 0;
      float dummy[4];
      CHECK(tpconv_forward(pm, &g, dummy, dummy, dummy, dummy, nullptr, nullptr, 0, nullptr) ==
            TPCONV_ERROR_INVALID_VALUE);
      CHECK(tpconv_forward_mlp(pm, &g, dummy, dummy, dummy, nullptr, dummy, nullptr, nullptr, 0, nullptr) ==
            TPCONV_ERROR_INVALID_VALUE);
      CHECK(tpconv_backward_mlp(pm, &g, dummy, dummy, dummy, dummy, dummy, nullptr, nullptr, nullptr, nullptr,
                                nullptr, nullptr, 0, nullptr) == TPCONV_ERROR_INVALID_VALUE);
      CHECK(tpconv_double_backward_mlp(pm, &g, dummy, dummy, dummy, nullptr, dummy, dummy, nullptr, nullptr,
                                       nullptr, nullptr, dummy, nullptr, 0, nullptr) == TPCONV_ERROR_INVALID_VALUE);
      size_t plain = 0, mlp = 0;
      tpconv_plan pp = nullptr;
      tpconv_desc dp = desc("8x0e+8x1o+8x2e", "8x0e+8x1o+8x2e", 2, 8);
      CHECK(tpconv_plan_create(&pp, &dp) == TPCONV_SUCCESS);
      if (pp) {
        CHECK(tpconv_workspace_size(pp, TPCONV_OP_BACKWARD, 1000, 5000, &plain) == TPCONV_SUCCESS);
        CHECK(tpconv_workspace_size(pm, TPCONV_OP_BACKWARD, 1000, 5000, &mlp) == TPCONV_SUCCESS);
        CHECK(mlp > plain);
        CHECK(tpconv_forward_mlp(pp, &g, dummy, dummy, dummy, dummy, dummy, nullptr, nullptr, 0, nullptr) ==
              TPCONV_ERROR_INVALID_VALUE);
        tpconv_plan_destroy(pp);
      }
      tpconv_plan_destroy(pm);
    }
    // deterministic position gradients: more workspace (the fixed-point sums), invalid flags rejected
    tpconv_desc dd = desc("8x0e+8x1o+8x2e", "8x0e+8x1o+8x2e", 2, 8);
    dd.deterministic = 1;
    tpconv_plan pd = nullptr;
    CHECK(tpconv_plan_create(&pd, &dd) == TPCONV_SUCCESS);
    if (pd) {
      exercise(pd);
      size_t det = 0, plain = 0;
      tpconv_desc dp = desc("8x0e+8x1o+8x2e", "8x0e+8x1o+8x2e", 2, 8);
      tpconv_plan pp = nullptr;
      CHECK(tpconv_plan_create(&pp, &dp) == TPCONV_SUCCESS);
      if (pp) {
        CHECK(tpconv_workspace_size(pd, TPCONV_OP_DOUBLE_BACKWARD, 1000, 5000, &det) == TPCONV_SUCCESS);
        CHECK(tpconv_workspace_size(pp, TPCONV_OP_DOUBLE_BACKWARD, 1000, 5000, &plain) == TPCONV_SUCCESS);
        CHECK(det >= plain + 1000 * 3 * 8);
        tpconv_plan_destroy(pp);
      }
      tpconv_plan_destroy(pd);
    }
    dd.deterministic = -1;
    CHECK(tpconv_plan_create(&pd, &dd) == TPCONV_ERROR_INVALID_VALUE);
    dm.connection = TPCONV_CHANNELWISE;
    CHECK(tpconv_plan_create(&pm, &dm) == TPCONV_ERROR_UNSUPPORTED);
    dm.connection = 0;
    dm.radial_mlp = 2;
    CHECK(tpconv_plan_create(&pm, &dm) == TPCONV_ERROR_INVALID_VALUE);
  }
  for (int s = 0; s <= 7; ++s) CHECK(tpconv_status_string((tpconv_status)s) != nullptr);
  CHECK(tpconv_status_string((tpconv_status)1234) != nullptr);
  CHECK(tpconv_plan_destroy(nullptr) != TPCONV_SUCCESS || true);
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("host sanitizer checks passed\n");
  return 0;
}
