// Host-side plan: irreps, parity-allowed paths, real CG tables and the layout
// of the node-sized receiver / sender states.  Pure C++ (no device calls).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace tpconv {

constexpr int kMaxL = 3;        // largest degree of any irrep or harmonic
constexpr int kMaxPaths = 64;   // paths per plan (kernel argument tables)
constexpr int kMaxGroups = 16;  // irreps per side
constexpr int kUnitAccumulators = 128;    // state accumulators per lane in a stream work unit
constexpr int kPosUnitAccumulators = 96;  // state cotangents per lane in a position-gradient unit

// Which stream a list of work units is for.
enum UnitSide { kUnitsRecv = 0, kUnitsSend = 1, kUnitsPos = 2 };

struct Irrep {
  int mul;
  int l;
  int parity;  // +1 even, -1 odd
};

// One parity-allowed coupling (input irrep i1 of degree l1) x (harmonic of
// degree l2) -> (output irrep i3 of degree l3).
struct Path {
  int i1, l1, l2, i3, l3;
  int q_out;  // index of the path among the paths of output irrep i3
  int q_in;   // index of the path among the paths of input irrep i1
};

// Paths that write one output irrep (receiver state S) or read one input
// irrep (sender state T).  The state of group g is a row-major matrix with
// rows (node, m) and columns (k, q, channel):
//   element (node, m, k, q, c) at base + ((node * n + m) * K + k) * cols_per_k + q * C + c
// with n = 2l+1 and cols_per_k = (#paths in the group) * C.
struct Group {
  int irrep;                // irrep index on its side
  int l;                    // its degree
  int row_off;              // row offset of the irrep in the feature layout
  std::vector<int> paths;   // plan path indices, in plan order
  int64_t base_per_node;    // element offset of this group's state = N * base_per_node
};

// Ragged multiplicities run on the uniform kernels with every irrep padded by
// zero channels to the largest multiplicity of its side (C_in / C_out below);
// the caller's tensors use the ragged layout: per node, irrep i's block
// [2l_i+1][mul_i] at feature offset foff[i]; per k, path p's weight block
// [mul(i1_p)][mul(i3_p)] (channel-wise: [mul_p]) at woff[p].
struct RaggedLayout {
  std::vector<int> mul_in, mul_out;     // caller's multiplicity per irrep
  std::vector<int64_t> foff_in, foff_out;
  int64_t F_in = 0, F_out = 0;          // caller's features per node
  std::vector<int64_t> woff;            // per path, within one k
  int64_t W_per_k = 0;
};

struct Plan {
  std::vector<Irrep> in, out;
  bool ragged = false;  // the caller's multiplicities differ between irreps (layout in `rag`)
  RaggedLayout rag;
  int sh_lmax = 0, K = 0, env_p = 6;
  float cutoff = 5.f;
  int x_dtype = 0, w_dtype = 0;
  int connection = 0;  // tpconv_connection
  int radial_mlp = 0;  // 1: the radial basis feeds a K x K SiLU layer whose outputs are the radial functions
  int deterministic = 0;  // 1: position gradients summed in exact fixed point (bitwise reproducible)
  int C_in = 0, C_out = 0, D_in = 0, D_out = 0, P = 0;
  int lmax = 0;  // max degree over irreps and harmonics
  std::vector<Path> paths;
  std::vector<std::vector<double>> cg;  // dense [2l1+1][2l2+1][2l3+1] per path
  std::vector<Group> out_groups;        // indexed by output irrep
  std::vector<Group> in_groups;         // indexed by input irrep
  int64_t state_in_per_node = 0;        // K * C_in * sum_p (2l3+1)
  int64_t state_out_per_node = 0;       // K * C_out * sum_p (2l1+1)
  // Work units of the edge streams.  With the natural irreps (one irrep per
  // degree 0..L on both sides, harmonics up to L) paths that gather the same
  // feature block are packed into bundles; otherwise every path is its own unit.
  bool natural = false;
  std::vector<std::vector<int>> recv_units;  // path indices per unit, receiver-side streams
  std::vector<std::vector<int>> send_units;  // path indices per unit, sender-side streams
  std::vector<std::vector<int>> pos_units;   // path indices per unit, position-gradient stream
};

// Paths (l1, l2, l3) of the natural irreps of degree <= L, in plan order.
std::vector<Path> natural_paths(int L);

// Bundles over natural_paths(L): paths grouped by the degree of the gathered
// block (l1 on the receiver side and in the position gradient, l3 on the
// sender side), packed in order so that K * (sum of output degrees 2l+1) stays
// within kUnitAccumulators (kPosUnitAccumulators for the position gradient).
std::vector<std::vector<int>> natural_bundles(int L, int K, int side);

// Parse "32x0e+32x1o"; returns false on a malformed string.
bool parse_irreps(const std::string& s, std::vector<Irrep>& out);

// <j1 m1 j2 m2 | J M> (Racah closed form, long double).
long double cg_complex(int j1, int m1, int j2, int m2, int J, int M);

// Real-basis table C[m1][m2][m3] (dense, row-major); false if the triangle rule fails.
bool real_cg(int l1, int l2, int l3, std::vector<double>& out);

// Returns 0 on success or a tpconv_status code.
int build_plan(const char* irreps_in, const char* irreps_out, int sh_lmax, int K, float cutoff,
               int env_p, int x_dtype, int w_dtype, int connection, Plan& plan);

}  // namespace tpconv
