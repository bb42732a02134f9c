// Kernel argument blocks and host launchers shared by the C-ABI layer and the
// kernel translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"

namespace tpconv {

// Edge-stream kernel modes.  Receiver-side modes walk the receiver-sorted CSR
// (self = receiver v, neighbour = sender s, gathered features = x[s]);
// sender-side modes walk the sender-sorted view (self = s, neighbour = v,
// gathered features = grad_out[v]).
enum StreamMode : int {
  kFwd = 0,      // S_v   += R (x) CG(x_s, Y)                      (receiver)
  kJvp = 1,      // Sd_v  += Rd (x) CG(x_s, Y) + R (x) CG(x_s, Yd)  (receiver)
  kSnd = 2,      // T_s   += R (x) CG'(g_v, Y)                      (sender)
  kSndT = 3,     // Td_s  += R (x) CG'(g_v, Yd) + Rd (x) CG'(g_v, Y) (sender)
  kBwdPos = 4,   // grad_pos from gS_v and the edge geometry        (receiver)
  kBwdHess = 5,  // d(force loss)/dpos: H_e phi_e from gS_v          (receiver)
};

struct StreamPath {
  int32_t l1, l2, l3;
  int32_t feat_row;     // first row of the gathered block (x rows of l1, or grad_out rows of l3)
  int64_t state_base;   // element offset of the group's state block
  int32_t cols_per_k;   // (#paths of the group) * channels
  int32_t q;            // path index inside its group
  int32_t path;         // plan path index (row k * P + path of W)
  int32_t out_row;      // first row of the path's output irrep in grad_out (channel-wise cotangent)
};

constexpr int kMaxUnitPaths = 8;  // member paths per stream work unit
constexpr int kPosMaxBlockWaves = 8;  // waves per block of the position streams
constexpr int kMaxPosPairs = 256;     // (slice, unit) pairs of a position-stream launch

struct StreamArgs {
  int32_t num_nodes;
  int32_t npaths;
  int32_t nunits;       // work units per (node, tile)
  int32_t bundled;      // units are the compile-time bundles of the natural path list
  int32_t nslices;      // 32-channel slices of the gathered planes (one wave, or one pair of a block, each)
  int32_t feat_rows;    // rows per node of the gathered feature tensor
  int32_t C;            // channels of the gathered features and of the state
  int32_t feat_cs;      // channel stride of the gathered planes (>= C; a multiple of 32 except bf16 used in place)
  int32_t env_p;
  float cutoff, inv_cutoff, pref;          // pref = sqrt(2 / cutoff)
  float env_a, env_b, env_c, env_d;        // u = 1 - a x^p + b x^(p+1) - c x^(p+2); u' = -d x^(p-1) (1-x)^2
  const int32_t* order; // [N] visiting order of the self nodes (NULL: 0..N-1)
  const int32_t* ptr;   // [N+1] segment offsets of self
  const int32_t* nbr;   // [E] neighbour of each edge
  const float* pos;     // [N][3]
  const float* ggpos;   // [N][3] tangent (kJvp, kSndT)
  const float* mlp;     // [K][K] weights of the radial MLP (NULL: the fixed basis feeds W directly)
  int32_t mlp_col;      // -1: the MLP's radial functions; j >= 0: their derivatives w.r.t. A[k][j]
  // kFwd / kJvp: with dot_state set, each work item writes, instead of its
  // state tile, the tile's dot with the same elements of dot_state per k to
  // dot_part[item][k] (the radial MLP's weight gradient, one column at a time)
  const float* dot_state;
  float* dot_part;
  // position streams, deterministic mode: per-edge shares added as 64-bit
  // fixed point (to_fixed with shift *fx_shift) to gpos_fx [N][3] instead of
  // fp32 atomics to gpos
  unsigned long long* gpos_fx;
  const int32_t* fx_shift;
  const void* feat;     // gathered features as bf16 [N][feat_rows][feat_cs]: the hi plane of split fp32, or bf16
  const void* feat_lo;  // lo bf16 plane of fp32 features split into hi + lo (NULL: bf16 features)
  float* state;         // output state (kFwd, kJvp, kSnd, kSndT)
  const float* gstate;  // receiver-state cotangent gS (kBwdPos, fully connected)
  float* gpos;          // position gradient (kBwdPos) or force-loss position derivative (kBwdHess), accumulated
  // kBwdPos with channel-wise weights: the cotangent gS[k, p, c, m3] =
  // W[k, p, c] grad_out[v][out_row + m3][c] is formed in registers
  int32_t cw;           // 1: channel-wise cotangent from W and grad_out
  int32_t w_bf16;
  int32_t gout_rows;    // rows per node of grad_out
  const void* W;        // [K][P][C], fp32 or bf16
  const float* gout;    // [N][gout_rows][C]
  // position streams: the block's waves (pos_waves) and the (slice, unit)
  // pairs of each wave w, pair_order[pair_begin[w] .. pair_begin[w + 1])
  int32_t pos_waves;
  int16_t pair_begin[kPosMaxBlockWaves + 1];
  uint8_t pair_order[kMaxPosPairs];
  StreamPath paths[kMaxPaths];
  int8_t unit_paths[kMaxPaths][kMaxUnitPaths];  // plan path indices of each unit's members
};

// Dense contractions with W, one group per launch slice.
enum GemmKind : int {
  kGemmOut = 0,  // out[(v,m3), co]   = sum_j S_g[(v,m3), j] W[j -> (k,p,ci), co]
  kGemmGs = 1,   // gS_g[(v,m3), j]   = sum_co g_out[(v,m3), co] W[j -> (k,p,ci), co]
  kGemmGx = 2,   // g_x[(s,m1), ci]   = sum_j T_g[(s,m1), j] W[j -> (k,p,co), ci]
  kGemmGw = 3,   // part[(k,p,ci), co] = sum_(v,m3) S_g[(v,m3), j] g_out[(v,m3), co]  (split over rows)
};

struct GemmGroup {
  int32_t M, N, Kr;          // C[M][N] = sum_r A[M][r] B[r][N]
  int32_t n;                 // 2l+1 of the group's irrep (rows per node)
  int32_t row_off;           // row offset of the irrep in the feature tensor it touches
  int32_t npg;               // paths in the group
  int32_t plist;             // first entry of the group's path list in GemmArgs::path_list
  int32_t tiles_n;           // column tiles
  int32_t tiles;             // total tiles (row tiles * column tiles)
  int32_t tile_begin;        // first block of the group in the flattened launch
  int64_t state_off;         // element offset of the group's state block
  int64_t part_off;          // element offset of the group's split-K partials (kGemmGw)
};

struct GemmArgs {
  int32_t ngroups;
  int32_t P, K, C_in, C_out, D_feat;  // D_feat: rows per node of the feature tensor touched
  int32_t splits;                     // kGemmGw: reduction splits
  int32_t vec;                        // channel counts allow 16-byte operand loads
  int32_t feat_cs;                    // channel stride of the g_out planes
  const float* state;                 // S_g / T_g blocks (A for Out, Gx, Gw)
  const uint16_t* feat_hi;            // bf16 planes of g_out [N][D_out][feat_cs] (A for Gs, B for Gw)
  const uint16_t* feat_lo;
  const uint16_t* w_hi;               // bf16 planes of W in its layout [K][P][C_in][C_out] (B for Gs, Gx)
  const uint16_t* w_lo;               // (NULL for bf16 weights: W is exact in bf16)
  const uint16_t* wt_hi;              // the same transposed per (k, p): [K][P][C_out][C_in] (B for Out)
  const uint16_t* wt_lo;
  float* out;                         // out / gS / g_x / partials
  float* part;                        // out, g_x split over blocks (splits > 1): their partial sums
  int32_t path_list[kMaxPaths];
  GemmGroup g[kMaxGroups];
};

// Channel-wise (diagonal) contractions over one side's irrep groups:
//   contract: dst[node][row_off + m][c] = sum_{q, k} W[k][path q][c] state_g[(node, m)][(k, q, c)]
//   gw:       part[split][elem_off + (k, q, c)] = sum_{(v, m) in split} state_g[(v, m)][(k, q, c)] gout[v][row_off + m][c]
//   reduce:   gW[k][path q][c] = sum over splits of part (fixed order)
struct CwGroup {
  int32_t n;         // 2l+1 rows per node
  int32_t row_off;   // row offset of the irrep in the feature tensor
  int32_t npg;       // paths in the group
  int32_t plist;     // first entry in CwArgs::path_list
  int64_t state_off; // element offset of the group's state block
  int64_t first;     // first flattened work index of the group
  int64_t elem_off;  // offset of the group's (k, q, c) block in the partials
};

struct CwArgs {
  int32_t ngroups, K, P, C, D_feat, splits, w_bf16;
  int64_t N;
  int64_t total;      // flattened work items (contract: rows x C; gw/reduce: elements)
  int64_t elems;      // sum over groups of K * npg * C
  const float* state;
  const float* gout;
  const void* W;
  float* dst;         // contract output, gw partials, or reduced gW
  const float* part;  // reduce input
  int32_t path_list[kMaxPaths];
  CwGroup g[kMaxGroups];
};

struct ReduceArgs {
  int32_t ngroups, splits, P, C_in, C_out;
  const float* part;
  float* gw;
  int32_t path_list[kMaxPaths];
  GemmGroup g[kMaxGroups];
};

// Ragged multiplicities: maps between the caller's layout and the padded one.
constexpr int kMaxRows = kMaxGroups * (2 * kMaxL + 1);
struct RaggedNodeMap {
  int32_t D, C;             // padded rows per node, padded channels
  int64_t F;                // caller's features per node
  int32_t off[kMaxRows];    // caller's feature offset of padded row r within a node
  int32_t mul[kMaxRows];    // channels of row r in the caller's layout
};
struct RaggedWeightMap {
  int32_t K, P, Ci, Co, cw;  // padded shape [K][P][Ci][Co] (channel-wise [K][P][Ci])
  int64_t W_per_k;           // caller's weights per k
  int64_t woff[kMaxPaths];   // caller's offset of path p's block within one k
  int32_t c1[kMaxPaths], c3[kMaxPaths];
};

// Host launchers (return a hipError_t).
hipError_t launch_ragged_nodes(const RaggedNodeMap& m, const void* src, void* dst, int64_t N, int elem_bytes,
                               bool pack, hipStream_t s);
hipError_t launch_ragged_weights(const RaggedWeightMap& m, const void* src, void* dst, int elem_bytes, bool pack,
                                 hipStream_t s);
hipError_t launch_stream(int mode, int lmax, int K, bool feat_bf16, const StreamArgs& a, int64_t items,
                         hipStream_t s);
// Fills the tiling fields of a.g[] (tiles, tiles_n, tile_begin) and launches.
hipError_t launch_gemm(int kind, GemmArgs& a, hipStream_t s);
// bf16 planes of W [KP][C_in][C_out] (fp32 split into hi + lo; bf16 copied into
// hi, lo unused): in its own layout and transposed per (k, p) to [KP][C_out][C_in].
hipError_t launch_w_planes(const void* W, bool w_bf16, int64_t kp, int C_in, int C_out, uint16_t* hi, uint16_t* lo,
                           uint16_t* thi, uint16_t* tlo, hipStream_t s);
// Wave tiles of a C[M][N] product of the given kind (the tile shape launch_gemm uses).
int64_t gemm_wave_tiles(int kind, int M, int N, int max_cols);
// Reduction splits of an out or g_x contraction (1: none), for the groups of
// `a` (set up with one split) and its vec flag; splits > 1 need partial sums
// of splits * sum_g M * N floats in a.part and launch_rows_reduce afterwards.
int gemm_rows_splits(int kind, const GemmArgs& a);
hipError_t launch_rows_reduce(int kind, const GemmArgs& a, hipStream_t s);
hipError_t launch_gw_reduce(const ReduceArgs& a, int64_t total, hipStream_t s);
// Zeroes rows [row_off, row_off + nrows) of every node of a [N][D][C] tensor.
hipError_t launch_zero_rows(float* base, int64_t N, int D, int C, int row_off, int nrows, hipStream_t s);
hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s);

// out[k * stride + j] = sum over b < nitems of part[(j * nitems + b) * K + k]
// for the columns j < ncols, in a fixed order: the per-item sums of the
// dot-out streams, one slab per column.
// Deterministic position gradients: the fixed-point shift from the largest
// |g| of a first fp32 pass (F = 58 - ceil(log2 max|g|), five bits of headroom
// for the exact sums), and the conversion of the fixed-point sums back.
hipError_t launch_fixed_shift(const float* g, int64_t n, uint32_t* maxbits, int32_t* shift, hipStream_t s);
hipError_t launch_fixed_to_float(const unsigned long long* acc, const int32_t* shift, float* out, int64_t n,
                                 hipStream_t s);
hipError_t launch_dot_reduce(const float* part, int64_t nitems, int K, int ncols, float* out, int stride,
                             hipStream_t s);
// hi[i] = bf16(x[i]), lo[i] = bf16(x[i] - hi[i]) (round to nearest even), as raw bf16 bits.
// bf16 planes of rows x C features with channel stride CS >= C, zero-padded:
// fp32 features split into hi + lo, bf16 features copied into hi (lo unused).
hipError_t launch_planes(const void* x, bool x_bf16, int64_t rows, int C, int CS, uint16_t* hi, uint16_t* lo,
                         hipStream_t s);
hipError_t launch_cw_contract(const CwArgs& a, hipStream_t s);
hipError_t launch_cw_gw(const CwArgs& a, hipStream_t s);
hipError_t launch_cw_reduce(const CwArgs& a, hipStream_t s);
hipError_t launch_graph_validate(const int32_t* rowptr, const int32_t* senders, int64_t N, int64_t E,
                                 int32_t* flag, hipStream_t s);
hipError_t graph_csc(const int32_t* rowptr, const int32_t* senders, int64_t N, int64_t E, int32_t* colptr,
                     int32_t* receivers_out, void* ws, size_t ws_bytes, hipStream_t s);
size_t graph_csc_workspace(int64_t N, int64_t E);
// Morton order of the node positions (a permutation of 0..N-1, deterministic).
hipError_t graph_order(const float* pos, int64_t N, int32_t* order, void* ws, size_t ws_bytes, hipStream_t s);
size_t graph_order_workspace(int64_t N);

}  // namespace tpconv
