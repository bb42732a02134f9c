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

struct StreamArgs {
  int32_t num_nodes;
  int32_t npaths;
  int32_t nunits;       // work units per (node, tile)
  int32_t bundled;      // units are the compile-time bundles of the natural path list
  int32_t share_geometry;  // kBwdPos: the units of a (node, tile) share one block and its batch geometry
  int32_t ct_log2;      // channel tile = 1 << ct_log2 (<= 64); edge slots per wave = 64 / tile
  int32_t ntiles;       // channels / tile
  int32_t feat_rows;    // rows per node of the gathered feature tensor
  int32_t C;            // channels of the gathered features and of the state
  int32_t env_p;
  float cutoff, inv_cutoff, pref;          // pref = sqrt(2 / cutoff)
  float env_a, env_b, env_c, env_d;        // u = 1 - a x^p + b x^(p+1) - c x^(p+2); u' = -d x^(p-1) (1-x)^2
  const int32_t* ptr;   // [N+1] segment offsets of self
  const int32_t* nbr;   // [E] neighbour of each edge
  const float* pos;     // [N][3]
  const float* ggpos;   // [N][3] tangent (kJvp, kSndT)
  const void* feat;     // [N][feat_rows][C], fp32 or bf16
  float* state;         // output state (kFwd, kJvp, kSnd, kSndT)
  const float* gstate;  // receiver-state cotangent gS (kBwdPos, fully connected)
  float* gpos;          // position gradient, accumulated (kBwdPos)
  // kBwdPos with channel-wise weights: the cotangent gS[k, p, c, m3] =
  // W[k, p, c] grad_out[v][out_row + m3][c] is formed in registers
  int32_t cw;           // 1: channel-wise cotangent from W and grad_out
  int32_t w_bf16;
  int32_t gout_rows;    // rows per node of grad_out
  const void* W;        // [K][P][C], fp32 or bf16
  const float* gout;    // [N][gout_rows][C]
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
  int32_t w_bf16;
  int32_t vec;                        // channel counts allow float4 operand loads
  const float* state;                 // S_g / T_g blocks (A for Out, Gx, Gw)
  const float* feat;                  // g_out (A for Gs, B for Gw)
  const void* W;                      // fp32 or bf16
  float* out;                         // out / gS / g_x / partials
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

// Host launchers (return a hipError_t).
hipError_t launch_stream(int mode, int lmax, int K, bool feat_bf16, const StreamArgs& a, int64_t items,
                         hipStream_t s);
// Fills the tiling fields of a.g[] (tiles, tiles_n, tile_begin) and launches.
hipError_t launch_gemm(int kind, GemmArgs& a, hipStream_t s);
// Wave tiles of a C[M][N] product of the given kind (the tile shape launch_gemm uses).
int64_t gemm_wave_tiles(int kind, int M, int N, int max_cols);
hipError_t launch_gw_reduce(const ReduceArgs& a, int64_t total, hipStream_t s);
hipError_t launch_zero_rows(float* base, int64_t N, int rows, int C, int row_off, int nrows, hipStream_t s);
hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t s);
hipError_t launch_cw_contract(const CwArgs& a, hipStream_t s);
hipError_t launch_cw_gw(const CwArgs& a, hipStream_t s);
hipError_t launch_cw_reduce(const CwArgs& a, hipStream_t s);
hipError_t launch_graph_validate(const int32_t* rowptr, const int32_t* senders, int64_t N, int64_t E,
                                 int32_t* flag, hipStream_t s);
hipError_t graph_csc(const int32_t* rowptr, const int32_t* senders, int64_t N, int64_t E, int32_t* colptr,
                     int32_t* receivers_out, void* ws, size_t ws_bytes, hipStream_t s);
size_t graph_csc_workspace(int64_t N, int64_t E);

}  // namespace tpconv
