// C ABI of the streaming CG tensor-product convolution (declared in include/tpconv.h).
//
// Pass structure (each step is one kernel launch on the caller's stream):
//   forward          : receiver stream S_v = sum_e R_e (x) U_e  ->  out = S . W
//   backward         : gS = g_out . W^T  ->  receiver stream for grad_pos
//                      S^T . g_out (split, ordered sum) -> grad_W
//                      sender stream T_s = sum_e R_e (x) CG'(g_out_v, Y_e)  ->  grad_x = T . W^T
//   double backward  : receiver tangent stream S_dot (along phi_e = gg[s] - gg[v])
//                      -> d_W = S_dot^T . g_out, d_grad_out = S_dot . W
//                      sender tangent stream T_dot -> d_x = T_dot . W^T
// Every intermediate is node-sized; nothing per edge is stored.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <numeric>
#include <new>
#include <vector>

#include "../../include/tpconv.h"
#include "kernels.h"
#include "plan.h"
#include "timing.h"

struct tpconv_plan_s {
  tpconv::Plan plan;
};

namespace tpconv {
namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t b) { return (b + kAlign - 1) / kAlign * kAlign; }

// Carves aligned sub-buffers out of the caller's workspace.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* p) : base(static_cast<char*>(p)) {}
  float* take(size_t count) {
    float* p = reinterpret_cast<float*>(base ? base + used : nullptr);
    used += align_up(count * sizeof(float));
    return p;
  }
};


// Reduction splits of the gW product over blocks: enough waves to fill the
// chip (with up to 4 waves per block; with channel counts that are multiples
// of 16, about 4096 waves of the LDS-staged kernel, which shares each chunk
// of g_out among four row tiles) while each split of the largest group keeps
// >= 512 reductions (smaller groups get shorter splits).
int gw_splits(const Plan& p, int64_t N) {
  int64_t tiles = 0, max_kr = 0;
  for (const auto& g : p.out_groups) {
    if (g.paths.empty()) continue;
    const int64_t M = (int64_t)p.K * g.paths.size() * p.C_in;
    tiles += gemm_wave_tiles(kGemmGw, (int)M, p.C_out, p.C_out);
    max_kr = std::max<int64_t>(max_kr, N * (2 * g.l + 1));
  }
  if (tiles == 0) return 1;
  int64_t s = (1024 + tiles - 1) / tiles;
  if (p.C_in % 16 == 0 && p.C_out % 16 == 0) {
    // waves of the LDS-staged kernel (32-row tiles, up to 128 columns per block)
    const int nt = p.C_out <= 32 ? 1 : (p.C_out <= 64 ? 2 : 4);
    int64_t lw = 0;
    for (const auto& g : p.out_groups)
      if (!g.paths.empty())
        lw += (((int64_t)p.K * g.paths.size() * p.C_in + 31) / 32) * ((p.C_out + 32 * nt - 1) / (32 * nt));
    if (lw > 0) s = std::max<int64_t>(s, (4096 + lw - 1) / lw);
  }
  s = std::min<int64_t>(s, 64);
  s = std::min<int64_t>(s, std::max<int64_t>(1, max_kr / 512));
  return (int)std::max<int64_t>(1, s);
}

size_t state_in_elems(const Plan& p, int64_t N) { return (size_t)(N * p.state_in_per_node); }
size_t state_out_elems(const Plan& p, int64_t N) { return (size_t)(N * p.state_out_per_node); }
bool channelwise(const Plan& p) { return p.connection == TPCONV_CHANNELWISE; }
size_t w_elems(const Plan& p) { return (size_t)p.K * p.P * p.C_in * (channelwise(p) ? 1 : p.C_out); }

// Row splits of the channel-wise weight gradient: about 256k threads, each
// summing at least 16 rows of the smallest group.
int cw_splits(const Plan& p, int64_t N) {
  const int64_t elems = (int64_t)w_elems(p);
  int64_t min_rows = INT64_MAX;
  for (const auto& g : p.out_groups)
    if (!g.paths.empty()) min_rows = std::min<int64_t>(min_rows, N * (2 * g.l + 1));
  if (elems == 0 || min_rows == INT64_MAX) return 1;
  int64_t s = (262144 + elems - 1) / elems;
  s = std::min<int64_t>(s, 1024);
  s = std::min<int64_t>(s, std::max<int64_t>(1, min_rows / 16));
  return (int)std::max<int64_t>(1, s);
}

// Partial sums of the weight gradient (either connection).
size_t part_elems(const Plan& p, int64_t N) {
  return (size_t)(channelwise(p) ? cw_splits(p, N) : gw_splits(p, N)) * w_elems(p);
}

// Weights in the caller's layout (ragged plans: the per-path blocks).
size_t w_elems_caller(const Plan& p) { return p.ragged ? (size_t)(p.K * p.rag.W_per_k) : w_elems(p); }

// Padded copies of a ragged plan's inputs and outputs (placed in front of the
// uniform passes' workspace): x, W and for each pass its node / weight outputs.
size_t pad_bytes(const Plan& p, int64_t N, int op) {
  if (!p.ragged) return 0;
  const size_t xin = (size_t)N * p.D_in * p.C_in, xout = (size_t)N * p.D_out * p.C_out;
  const size_t xb = p.x_dtype == TPCONV_BF16 ? 2 : 4, wb = p.w_dtype == TPCONV_BF16 ? 2 : 4;
  size_t b = align_up(xin * xb) + align_up(w_elems(p) * wb);
  if (op == TPCONV_OP_FORWARD) return b + align_up(xout * 4);  // out
  b += align_up(xout * 4) + align_up(xin * 4) + align_up(w_elems(p) * 4);  // grad_out, grad_x / d_x, grad_W / d_W
  if (op == TPCONV_OP_DOUBLE_BACKWARD) b += align_up(xout * 4);              // d_grad_out
  return b;
}

tpconv_status dev(hipError_t e) { return e == hipSuccess ? TPCONV_SUCCESS : TPCONV_ERROR_DEVICE; }

// bf16 planes of the features the edge streams gather, rows padded to a
// multiple of 32 channels: fp32 features split into hi and lo, bf16 features
// used in place when C is a multiple of 32 and copied otherwise.
int plane_cs(int C) { return (C + 31) / 32 * 32; }
size_t plane_bytes(int64_t N, int rows, int C, bool bf16) {
  if (bf16 && C % 32 == 0) return 0;
  const size_t one = align_up((size_t)N * rows * plane_cs(C) * 2);
  return bf16 ? one : 2 * one;
}
size_t x_planes(const Plan& p, int64_t N) { return plane_bytes(N, p.D_in, p.C_in, p.x_dtype == TPCONV_BF16); }
size_t g_planes(const Plan& p, int64_t N) { return plane_bytes(N, p.D_out, p.C_out, false); }
// The streams address the planes with 32-bit byte offsets.
bool planes_addressable(const Plan& p, int64_t N) {
  return (uint64_t)N * p.D_in * plane_cs(p.C_in) * 2 < (uint64_t(1) << 32) &&
         (uint64_t)N * p.D_out * plane_cs(p.C_out) * 2 < (uint64_t(1) << 32);
}

struct Planes {
  const void* hi = nullptr;
  const void* lo = nullptr;
  int cs = 0;
};

// The planes of rows x C features, carved from the workspace (none for bf16
// features already padded).
tpconv_status make_planes(const void* x, bool bf16, int64_t N, int rows, int C, Carver& c, Planes& out,
                          hipStream_t s) {
  out.cs = plane_cs(C);
  if (bf16 && C % 32 == 0) {
    out.hi = x;
    out.lo = nullptr;
    return TPCONV_SUCCESS;
  }
  const size_t n = (size_t)N * rows * out.cs;
  uint16_t* hi = reinterpret_cast<uint16_t*>(c.take((n + 1) / 2));
  uint16_t* lo = bf16 ? nullptr : reinterpret_cast<uint16_t*>(c.take((n + 1) / 2));
  out.hi = hi;
  out.lo = lo;
  return dev(launch_planes(x, bf16, N * rows, C, out.cs, hi, lo, s));
}

// bf16 planes of W for the contractions (fully connected only): hi and, for
// fp32 weights, lo, each in W's layout and transposed per (k, p).
size_t w_planes(const Plan& p) {
  if (channelwise(p)) return 0;
  return (p.w_dtype == TPCONV_BF16 ? 2 : 4) * align_up(w_elems(p) * 2);
}

struct WPlanes {
  const uint16_t* hi = nullptr;
  const uint16_t* lo = nullptr;
  const uint16_t* thi = nullptr;
  const uint16_t* tlo = nullptr;
};

tpconv_status make_w_planes(const Plan& p, const void* W, Carver& c, WPlanes& out, hipStream_t s) {
  if (channelwise(p)) return TPCONV_SUCCESS;
  const size_t n = w_elems(p);
  const bool bf16 = p.w_dtype == TPCONV_BF16;
  uint16_t* hi = reinterpret_cast<uint16_t*>(c.take((n + 1) / 2));
  uint16_t* thi = reinterpret_cast<uint16_t*>(c.take((n + 1) / 2));
  uint16_t* lo = bf16 ? nullptr : reinterpret_cast<uint16_t*>(c.take((n + 1) / 2));
  uint16_t* tlo = bf16 ? nullptr : reinterpret_cast<uint16_t*>(c.take((n + 1) / 2));
  out.hi = hi;
  out.lo = lo;
  out.thi = thi;
  out.tlo = tlo;
  return dev(launch_w_planes(W, bf16, (int64_t)p.K * p.P, p.C_in, p.C_out, hi, lo, thi, tlo, s));
}

size_t rows_part_elems(const Plan& p, int kind, int64_t N);

// Per-item sums of the radial MLP's weight gradient: the receiver stream in
// its dot-out mode writes K values per work item (node, unit, slice).
size_t dot_part_elems(const Plan& p, int64_t N) {
  if (!p.radial_mlp) return 0;  // one slab of per-item sums per column of A
  return (size_t)N * p.recv_units.size() * ((p.C_in + 31) / 32) * p.K * p.K;
}

// Deterministic position gradients: 64-bit fixed-point sums [N][3] and two
// scalars (the largest magnitude's bits and the shift).
struct FixedBufs {
  unsigned long long* acc = nullptr;
  int32_t* tmp = nullptr;
};
size_t fixed_bytes(const Plan& p, int64_t N) {
  return p.deterministic ? align_up((size_t)N * 3 * 8) + align_up(2 * 4) : 0;
}
FixedBufs take_fixed(const Plan& p, int64_t N, Carver& c) {
  FixedBufs f;
  if (!p.deterministic) return f;
  f.acc = reinterpret_cast<unsigned long long*>(c.take((size_t)N * 6));
  f.tmp = reinterpret_cast<int32_t*>(c.take(2));
  return f;
}

size_t ws_forward(const Plan& p, int64_t N, bool have_saved) {
  return (have_saved ? 0 : align_up(state_in_elems(p, N) * 4)) + align_up(rows_part_elems(p, kGemmOut, N) * 4) +
         x_planes(p, N) + w_planes(p) + pad_bytes(p, N, TPCONV_OP_FORWARD);
}

size_t ws_backward(const Plan& p, int64_t N) {
  // S (recomputed when not saved) and T share one buffer: the weight gradient
  // reads S before the sender stream writes T, both on the side stream.
  // Then gS (fully connected only), gW partials, planes of x and g_out.
  return align_up(std::max(state_in_elems(p, N), state_out_elems(p, N)) * 4) +
         (channelwise(p) ? 0 : align_up(state_in_elems(p, N) * 4)) + align_up(part_elems(p, N) * 4) +
         align_up(rows_part_elems(p, kGemmGx, N) * 4) + x_planes(p, N) + g_planes(p, N) + w_planes(p) +
         pad_bytes(p, N, TPCONV_OP_BACKWARD) +
         align_up(dot_part_elems(p, N) * 4) +  // radial MLP: per-item sums of dL/dA
         fixed_bytes(p, N);
}

size_t ws_double_backward(const Plan& p, int64_t N) {
  // S_dot (gS, fully connected, reuses it once its contractions are done; one
  // stream), T_dot, weight partials, planes of x and g_out
  return align_up(state_in_elems(p, N) * 4) + align_up(state_out_elems(p, N) * 4) +
         align_up(part_elems(p, N) * 4) + align_up(rows_part_elems(p, kGemmGx, N) * 4) +
         align_up(rows_part_elems(p, kGemmOut, N) * 4) + x_planes(p, N) + g_planes(p, N) + w_planes(p) +
         pad_bytes(p, N, TPCONV_OP_DOUBLE_BACKWARD) + align_up(dot_part_elems(p, N) * 4) + fixed_bytes(p, N);
}

// Independent chains of one call (the position gradient, the input gradient
// and the weight gradient) run concurrently: a second stream per device,
// created on first use with the default priority, is forked from the
// caller's stream with an event and joined back before the call returns.
// The mutex keeps the record/wait pairs of concurrent callers on one device
// from interleaving.  While kernel timing is on, or with TPCONV_OVERLAP=0 in
// the environment, everything stays on the caller's stream.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};

SideStream* side_stream() {
  static std::mutex mu;
  static std::map<int, SideStream*> per_device;
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  auto it = per_device.find(d);
  if (it != per_device.end()) return it->second;
  SideStream* ss = new (std::nothrow) SideStream();
  if (!ss) return nullptr;
  if (hipStreamCreateWithFlags(&ss->s, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&ss->fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&ss->join, hipEventDisableTiming) != hipSuccess) {
    delete ss;  // (a failed creation leaves the call on one stream)
    return nullptr;
  }
  per_device[d] = ss;
  return ss;
}

bool overlap_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("TPCONV_OVERLAP");
    return !(e && e[0] == '0');
  }();
  return on && !timing_enabled();
}

class Fork {
 public:
  explicit Fork(hipStream_t main) : main_(main), side_(main) {
    if (!overlap_enabled()) return;
    ss_ = side_stream();
    if (!ss_) return;
    ss_->mu.lock();
    if (hipEventRecord(ss_->fork, main_) != hipSuccess || hipStreamWaitEvent(ss_->s, ss_->fork, 0) != hipSuccess) {
      ss_->mu.unlock();
      ss_ = nullptr;
      return;
    }
    side_ = ss_->s;
  }
  hipStream_t side() const { return side_; }
  // Makes the caller's stream wait for the side stream; idempotent.
  tpconv_status join() {
    if (!ss_) return TPCONV_SUCCESS;
    hipError_t e = hipEventRecord(ss_->join, side_);
    if (e == hipSuccess) e = hipStreamWaitEvent(main_, ss_->join, 0);
    ss_->mu.unlock();
    ss_ = nullptr;
    return dev(e);
  }
  ~Fork() { join(); }
  Fork(const Fork&) = delete;
  Fork& operator=(const Fork&) = delete;

 private:
  hipStream_t main_, side_;
  SideStream* ss_ = nullptr;
};

tpconv_status check_graph(const tpconv_graph* g, bool need_csc) {
  if (!g) return TPCONV_ERROR_INVALID_VALUE;
  if (g->num_nodes < 0 || g->num_edges < 0 || g->num_nodes >= INT32_MAX || g->num_edges >= INT32_MAX)
    return TPCONV_ERROR_INVALID_VALUE;
  if (g->num_nodes > 0 && !g->rowptr) return TPCONV_ERROR_INVALID_VALUE;
  if (g->num_edges > 0 && (!g->senders || g->num_nodes == 0)) return TPCONV_ERROR_INVALID_VALUE;
  if (need_csc && g->num_nodes > 0 && (!g->csc_colptr || (g->num_edges > 0 && !g->csc_receivers)))
    return TPCONV_ERROR_INVALID_VALUE;
  return TPCONV_SUCCESS;
}

void fill_common(const Plan& p, StreamArgs& a, const tpconv_graph* g, const float* pos) {
  const int64_t N = g->num_nodes;
  std::memset(&a, 0, sizeof(a));
  a.order = g->node_order;
  a.num_nodes = (int32_t)N;
  a.npaths = p.P;
  a.env_p = p.env_p;
  a.cutoff = p.cutoff;
  a.inv_cutoff = 1.0f / p.cutoff;
  a.pref = (float)std::sqrt(2.0 / p.cutoff);
  const double e = p.env_p;
  a.env_a = (float)((e + 1) * (e + 2) / 2);
  a.env_b = (float)(e * (e + 2));
  a.env_c = (float)(e * (e + 1) / 2);
  a.env_d = (float)(e * (e + 1) * (e + 2) / 2);
  a.pos = pos;
  a.mlp = nullptr;
  a.mlp_col = -1;
}

void set_units(const Plan& p, StreamArgs& a, const std::vector<std::vector<int>>& units) {
  a.nunits = (int32_t)units.size();
  a.bundled = p.natural ? 1 : 0;
  for (size_t u = 0; u < units.size(); ++u)
    for (size_t i = 0; i < units[u].size(); ++i) a.unit_paths[u][i] = (int8_t)units[u][i];
}

// Receiver-side stream over the CSR: gathered features x [N][D_in][C_in],
// state S (or S_dot) in the output-group layout.
void recv_args(const Plan& p, StreamArgs& a, const tpconv_graph* g, const float* pos, const void* x,
               const float* rw) {
  const int64_t N = g->num_nodes;
  fill_common(p, a, g, pos);
  a.mlp = rw;
  a.ptr = g->rowptr;
  a.nbr = g->senders;
  a.feat = x;
  a.feat_rows = p.D_in;
  a.C = p.C_in;
  for (int i = 0; i < p.P; ++i) {
    const Path& q = p.paths[i];
    const Group& og = p.out_groups[q.i3];
    a.paths[i] = StreamPath{q.l1, q.l2, q.l3, p.in_groups[q.i1].row_off, N * og.base_per_node,
                            (int32_t)og.paths.size() * p.C_in, q.q_out, i, og.row_off};
  }
  set_units(p, a, p.recv_units);
}

// Sender-side stream over the CSC view: gathered features grad_out [N][D_out][C_out],
// state T (or T_dot) in the input-group layout.
void send_args(const Plan& p, StreamArgs& a, const tpconv_graph* g, const float* pos, const float* gout,
               const float* rw) {
  const int64_t N = g->num_nodes;
  fill_common(p, a, g, pos);
  a.mlp = rw;
  a.ptr = g->csc_colptr;
  a.nbr = g->csc_receivers;
  a.feat = gout;
  a.feat_rows = p.D_out;
  a.C = p.C_out;
  for (int i = 0; i < p.P; ++i) {
    const Path& q = p.paths[i];
    const Group& ig = p.in_groups[q.i1];
    a.paths[i] = StreamPath{q.l1, q.l2, q.l3, p.out_groups[q.i3].row_off, N * ig.base_per_node,
                            (int32_t)ig.paths.size() * p.C_out, q.q_in, i, p.in_groups[q.i1].row_off};
  }
  set_units(p, a, p.send_units);
}

// The gathered features of a stream as bf16 planes; the streams take their
// 32-channel slices.
void use_planes(StreamArgs& a, const Planes& pl) {
  a.feat = pl.hi;
  a.feat_lo = pl.lo;
  a.feat_cs = pl.cs;
  a.nslices = pl.cs / 32;
}

// Work items of a stream launch: one wave (or block) per (node, unit, slice).
int64_t stream_items(const StreamArgs& a) { return (int64_t)a.num_nodes * a.nunits * a.nslices; }

// Groups of a GEMM over the output irreps (Out, Gs, Gw) or input irreps (Gx).
int gemm_setup(const Plan& p, int kind, int64_t N, GemmArgs& a, int splits) {
  std::memset(&a, 0, sizeof(a));
  a.P = p.P;
  a.K = p.K;
  a.C_in = p.C_in;
  a.C_out = p.C_out;
  a.splits = splits;
  const bool in_side = kind == kGemmGx;
  const auto& groups = in_side ? p.in_groups : p.out_groups;
  a.D_feat = in_side ? p.D_in : p.D_out;
  int npl = 0, ng = 0;
  int64_t part = 0;
  for (const auto& g : groups) {
    const int npg = (int)g.paths.size();
    // A group that no path reaches has an empty reduction (out, g_x: its rows
    // are zero-filled by run_gemm) or no columns (gS, gW): never launched.
    if (npg == 0) continue;
    GemmGroup G{};
    const int n = 2 * g.l + 1;
    G.n = n;
    G.row_off = g.row_off;
    G.npg = npg;
    G.plist = npl;
    for (int q : g.paths) a.path_list[npl++] = q;
    G.state_off = N * g.base_per_node;
    switch (kind) {
      case kGemmOut: G.M = (int)(N * n); G.N = p.C_out; G.Kr = p.K * npg * p.C_in; break;
      case kGemmGs: G.M = (int)(N * n); G.N = p.K * npg * p.C_in; G.Kr = p.C_out; break;
      case kGemmGx: G.M = (int)(N * n); G.N = p.C_in; G.Kr = p.K * npg * p.C_out; break;
      case kGemmGw: G.M = p.K * npg * p.C_in; G.N = p.C_out; G.Kr = (int)(N * n); break;
    }
    G.part_off = part;
    part += (int64_t)splits * G.M * G.N;
    a.g[ng++] = G;
  }
  a.ngroups = ng;
  return ng;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Partial sums of an out or g_x contraction split over blocks (floats; 0 when
// it runs unsplit), for workspace sizing: the 16-byte load path is assumed.
size_t rows_part_elems(const Plan& p, int kind, int64_t N) {
  if (channelwise(p)) return 0;
  GemmArgs a;
  gemm_setup(p, kind, N, a, 1);
  a.vec = (p.C_in % 16 == 0) && (p.C_out % 16 == 0);
  const int sp = gemm_rows_splits(kind, a);
  if (sp <= 1) return 0;
  size_t n = 0;
  for (int g = 0; g < a.ngroups; ++g) n += (size_t)a.g[g].M * a.g[g].N;
  return n * sp;
}

// 16-byte operand loads need channel counts that are multiples of 16 and
// 16-byte aligned states (the planes come from the workspace, 256-aligned).
void set_vec(const Plan& p, GemmArgs& a) {
  a.vec = (p.C_in % 16 == 0) && (p.C_out % 16 == 0) && aligned16(a.state);
}

void set_planes(GemmArgs& a, const Planes* gp, const WPlanes& wp) {
  if (gp) {
    a.feat_hi = static_cast<const uint16_t*>(gp->hi);
    a.feat_lo = static_cast<const uint16_t*>(gp->lo);
    a.feat_cs = gp->cs;
  }
  a.w_hi = wp.hi;
  a.w_lo = wp.lo;
  a.wt_hi = wp.thi;
  a.wt_lo = wp.tlo;
}

// gp: the g_out planes (gS); wp: the W planes; rows_part: room for the
// partial sums of a split out or g_x (rows_part_elems floats).
tpconv_status run_gemm(const Plan& p, int kind, int64_t N, const float* state, const Planes* gp, const WPlanes& wp,
                       float* out, float* rows_part, hipStream_t s) {
  if (kind == kGemmOut || kind == kGemmGx) {  // rows of irreps that no path reaches are zero
    const bool in_side = kind == kGemmGx;
    for (const auto& g : in_side ? p.in_groups : p.out_groups) {
      if (!g.paths.empty()) continue;
      const hipError_t e = launch_zero_rows(out, N, in_side ? p.D_in : p.D_out, in_side ? p.C_in : p.C_out,
                                            g.row_off, 2 * g.l + 1, s);
      if (e != hipSuccess) return dev(e);
    }
  }
  GemmArgs a;
  gemm_setup(p, kind, N, a, 1);
  a.state = state;
  set_planes(a, gp, wp);
  a.out = out;
  set_vec(p, a);
  const int sp = gemm_rows_splits(kind, a);
  if (sp > 1) {  // reduction split over blocks: partial sums, then their ordered sum
    if (!rows_part) return TPCONV_ERROR_WORKSPACE;
    gemm_setup(p, kind, N, a, sp);
    a.state = state;
    set_planes(a, gp, wp);
    a.out = out;
    set_vec(p, a);
    a.part = rows_part;
    tpconv_status st = dev(launch_gemm(kind, a, s));
    if (st != TPCONV_SUCCESS) return st;
    return dev(launch_rows_reduce(kind, a, s));
  }
  return dev(launch_gemm(kind, a, s));
}

// gW = S^T g_out from the g_out planes gp.
tpconv_status run_gw(const Plan& p, int64_t N, const float* state, const Planes& gp, float* part, float* gW,
                     hipStream_t s) {
  const int splits = gw_splits(p, N);
  GemmArgs a;
  gemm_setup(p, kGemmGw, N, a, splits);
  a.state = state;
  set_planes(a, &gp, WPlanes{});
  a.out = part;
  set_vec(p, a);
  tpconv_status st = dev(launch_gemm(kGemmGw, a, s));
  if (st != TPCONV_SUCCESS) return st;
  ReduceArgs r;
  std::memset(&r, 0, sizeof(r));
  r.ngroups = a.ngroups;
  r.splits = splits;
  r.P = p.P;
  r.C_in = p.C_in;
  r.C_out = p.C_out;
  r.part = part;
  r.gw = gW;
  std::memcpy(r.path_list, a.path_list, sizeof(r.path_list));
  std::memcpy(r.g, a.g, sizeof(r.g));
  int64_t total = 0;
  for (int i = 0; i < a.ngroups; ++i) total += (int64_t)a.g[i].M * a.g[i].N;
  if (total == 0) return dev(launch_fill(gW, (int64_t)w_elems(p), 0.f, s));
  return dev(launch_gw_reduce(r, total, s));
}

// Channel-wise contraction of a state over one side's groups into a feature
// tensor: out / d_grad_out from S or S_dot (output side), g_x / d_x from T or
// T_dot (input side).
tpconv_status run_cw_contract(const Plan& p, bool out_side, int64_t N, const float* state, const void* W,
                              float* dst, hipStream_t s) {
  CwArgs a;
  std::memset(&a, 0, sizeof(a));
  const auto& groups = out_side ? p.out_groups : p.in_groups;
  a.K = p.K;
  a.P = p.P;
  a.C = p.C_in;
  a.N = N;
  a.D_feat = out_side ? p.D_out : p.D_in;
  a.w_bf16 = p.w_dtype == TPCONV_BF16;
  a.state = state;
  a.W = W;
  a.dst = dst;
  int npl = 0;
  int64_t total = 0;
  for (const auto& g : groups) {
    CwGroup G{};
    G.n = 2 * g.l + 1;
    G.row_off = g.row_off;
    G.npg = (int)g.paths.size();
    G.plist = npl;
    for (int q : g.paths) a.path_list[npl++] = q;
    G.state_off = N * g.base_per_node;
    G.first = total;
    total += N * G.n * p.C_in;
    a.g[a.ngroups++] = G;
  }
  a.total = total;
  return dev(launch_cw_contract(a, s));
}

// Channel-wise weight gradient dW[k, p, c] = sum_{v, m3} state * grad_out over
// the output groups (S for grad_W, S_dot for d_W), split over rows and summed
// in a fixed order.
tpconv_status run_cw_gw(const Plan& p, int64_t N, const float* state, const float* gout, float* part, float* gW,
                        hipStream_t s) {
  CwArgs a;
  std::memset(&a, 0, sizeof(a));
  a.K = p.K;
  a.P = p.P;
  a.C = p.C_in;
  a.N = N;
  a.D_feat = p.D_out;
  a.splits = cw_splits(p, N);
  a.state = state;
  a.gout = gout;
  a.dst = part;
  int npl = 0;
  int64_t elems = 0;
  for (const auto& g : p.out_groups) {
    if (g.paths.empty()) continue;
    CwGroup G{};
    G.n = 2 * g.l + 1;
    G.row_off = g.row_off;
    G.npg = (int)g.paths.size();
    G.plist = npl;
    for (int q : g.paths) a.path_list[npl++] = q;
    G.state_off = N * g.base_per_node;
    G.elem_off = elems;
    elems += (int64_t)p.K * G.npg * p.C_in;
    a.g[a.ngroups++] = G;
  }
  a.elems = elems;
  if (elems == 0) return dev(launch_fill(gW, (int64_t)w_elems(p), 0.f, s));
  tpconv_status st = dev(launch_cw_gw(a, s));
  if (st != TPCONV_SUCCESS) return st;
  a.part = part;
  a.dst = gW;
  return dev(launch_cw_reduce(a, s));
}

// Waves per block of the position streams and each wave's (slice, unit)
// pairs.  The waves of a block meet at every 64-edge batch, so a block takes
// as long as its most loaded wave: the pairs (cost: row tiles times gathered
// rows, the per-batch count of matrix-core steps) are packed longest first
// onto the least loaded wave, for the wave count (2..8) that wastes the
// least wave time.
bool assign_pos_pairs(const Plan& p, StreamArgs& a) {
  const int npairs = a.nunits * a.nslices;
  if (npairs <= 0 || npairs > kMaxPosPairs) return false;
  std::vector<int> cost(npairs);
  for (int pr = 0; pr < npairs; ++pr) {
    const auto& u = p.pos_units[pr % a.nunits];
    int tot = 0;
    for (int q : u) tot += 2 * p.paths[q].l3 + 1;
    cost[pr] = ((p.K * tot + 15) / 16) * (2 * p.paths[u[0]].l1 + 1) + 1;
  }
  std::vector<int> idx(npairs);
  for (int i = 0; i < npairs; ++i) idx[i] = i;
  std::stable_sort(idx.begin(), idx.end(), [&](int x, int y) { return cost[x] > cost[y]; });
  double best = -1.0;
  std::vector<std::vector<int>> best_lists;
  for (int nw = 1; nw <= std::min(kPosMaxBlockWaves, npairs); ++nw) {
    std::vector<std::vector<int>> lists(nw);
    std::vector<int> load(nw, 0);
    for (int i : idx) {
      const int w = (int)(std::min_element(load.begin(), load.end()) - load.begin());
      lists[w].push_back(i);
      load[w] += cost[i];
    }
    const int total = std::accumulate(load.begin(), load.end(), 0);
    const double eff = (double)total / ((double)nw * *std::max_element(load.begin(), load.end()));
    // at least two waves (a one-wave block leaves too little room for
    // others in the LDS of a compute unit), otherwise the best balance
    if ((nw >= 2 || npairs == 1) && eff > best + 1e-9) {
      best = eff;
      best_lists = lists;
    }
  }
  a.pos_waves = (int32_t)best_lists.size();
  int k = 0;
  for (int w = 0; w < a.pos_waves; ++w) {
    a.pair_begin[w] = (int16_t)k;
    for (int pr : best_lists[w]) a.pair_order[k++] = (uint8_t)pr;
  }
  a.pair_begin[a.pos_waves] = (int16_t)k;
  return true;
}

// The receiver-side position streams (kBwdPos: grad_pos; kBwdHess: the
// position derivative of the force loss along gg_pos) into out [N][3]:
// gS = g_out W^T first unless gs_ready (formed in registers when
// channel-wise); xp, gp, wp: the bf16 planes of x, g_out and W; rw: the
// radial MLP's weights or NULL.
tpconv_status run_pos_stream(const Plan& p, int mode, const tpconv_graph* g, const float* pos, const void* x,
                             const Planes& xp, const Planes& gp, const WPlanes& wp, const void* W,
                             const float* grad_out, const float* gg_pos, float* gS, bool gs_ready, const float* rw,
                             const FixedBufs& fx, float* out, hipStream_t s) {
  const int64_t N = g->num_nodes;
  const bool cw = channelwise(p);
  tpconv_status st;
  if (!cw && !gs_ready && (st = run_gemm(p, kGemmGs, N, nullptr, &gp, wp, gS, nullptr, s)) != TPCONV_SUCCESS)
    return st;
  if ((st = dev(launch_fill(out, 3 * N, 0.f, s))) != TPCONV_SUCCESS) return st;
  StreamArgs a;
  recv_args(p, a, g, pos, x, rw);
  set_units(p, a, p.pos_units);
  use_planes(a, xp);
  if (!assign_pos_pairs(p, a)) return TPCONV_ERROR_INVALID_VALUE;
  a.gstate = gS;
  a.gpos = out;
  a.ggpos = gg_pos;
  if (cw) {
    a.cw = 1;
    a.W = W;
    a.w_bf16 = p.w_dtype == TPCONV_BF16;
    a.gout = grad_out;
    a.gout_rows = p.D_out;
  }
  if ((st = dev(launch_stream(mode, p.lmax, p.K, p.x_dtype == TPCONV_BF16, a, stream_items(a), s))) !=
          TPCONV_SUCCESS ||
      !fx.acc)
    return st;
  // deterministic: the fp32 result sets the fixed-point shift, then the same
  // stream again with exact 64-bit sums
  uint32_t* maxbits = reinterpret_cast<uint32_t*>(fx.tmp);
  int32_t* shift = fx.tmp + 1;
  if ((st = dev(launch_fill(reinterpret_cast<float*>(maxbits), 1, 0.f, s))) != TPCONV_SUCCESS) return st;
  if ((st = dev(launch_fixed_shift(out, 3 * N, maxbits, shift, s))) != TPCONV_SUCCESS) return st;
  if ((st = dev(launch_fill(reinterpret_cast<float*>(fx.acc), 6 * N, 0.f, s))) != TPCONV_SUCCESS) return st;
  a.gpos_fx = fx.acc;
  a.fx_shift = shift;
  if ((st = dev(launch_stream(mode, p.lmax, p.K, p.x_dtype == TPCONV_BF16, a, stream_items(a), s))) !=
      TPCONV_SUCCESS)
    return st;
  return dev(launch_fixed_to_float(fx.acc, shift, out, 3 * N, s));
}

RaggedNodeMap node_map(const Plan& p, bool in_side) {
  RaggedNodeMap m;
  std::memset(&m, 0, sizeof(m));
  const auto& irs = in_side ? p.in : p.out;
  const auto& mul = in_side ? p.rag.mul_in : p.rag.mul_out;
  const auto& foff = in_side ? p.rag.foff_in : p.rag.foff_out;
  m.D = in_side ? p.D_in : p.D_out;
  m.C = in_side ? p.C_in : p.C_out;
  m.F = in_side ? p.rag.F_in : p.rag.F_out;
  int r = 0;
  for (size_t i = 0; i < irs.size(); ++i)
    for (int k = 0; k < 2 * irs[i].l + 1; ++k, ++r) {
      m.off[r] = (int32_t)(foff[i] + (int64_t)k * mul[i]);
      m.mul[r] = mul[i];
    }
  return m;
}

RaggedWeightMap weight_map(const Plan& p) {
  RaggedWeightMap m;
  std::memset(&m, 0, sizeof(m));
  m.K = p.K;
  m.P = p.P;
  m.Ci = p.C_in;
  m.Co = p.C_out;
  m.cw = channelwise(p) ? 1 : 0;
  m.W_per_k = p.rag.W_per_k;
  for (int i = 0; i < p.P; ++i) {
    m.woff[i] = p.rag.woff[i];
    m.c1[i] = p.rag.mul_in[p.paths[i].i1];
    m.c3[i] = p.rag.mul_out[p.paths[i].i3];
  }
  return m;
}

// The passes on uniform (for ragged plans: padded) tensors.
tpconv_status forward_core(const Plan& p, const tpconv_graph* g, const float* pos, const void* x, const void* W,
                           const float* rw, float* out, float* saved_state, void* ws, hipStream_t s) {
  const int64_t N = g->num_nodes;
  Carver c(ws);
  float* S = saved_state ? saved_state : c.take(state_in_elems(p, N));
  float* rpart = c.take(rows_part_elems(p, kGemmOut, N));
  tpconv_status st;
  Planes xp;
  if ((st = make_planes(x, p.x_dtype == TPCONV_BF16, N, p.D_in, p.C_in, c, xp, s)) != TPCONV_SUCCESS) return st;
  WPlanes wp;
  if ((st = make_w_planes(p, W, c, wp, s)) != TPCONV_SUCCESS) return st;
  StreamArgs a;
  recv_args(p, a, g, pos, x, rw);
  use_planes(a, xp);
  a.state = S;
  if ((st = dev(launch_stream(kFwd, p.lmax, p.K, p.x_dtype == TPCONV_BF16, a, stream_items(a), s))) !=
      TPCONV_SUCCESS)
    return st;
  if (channelwise(p)) return run_cw_contract(p, true, N, S, W, out, s);
  return run_gemm(p, kGemmOut, N, S, nullptr, wp, out, rpart, s);
}

tpconv_status backward_core(const Plan& p, const tpconv_graph* g, const float* pos, const void* x, const void* W,
                            const float* rw, const float* grad_out, const float* saved_state, float* grad_x,
                            float* grad_W, float* grad_pos, float* grad_rw, void* ws, hipStream_t s) {
  const int64_t N = g->num_nodes;
  const bool cw = channelwise(p);
  tpconv_status st;
  Carver c(ws);
  float* S_ws = c.take(std::max(state_in_elems(p, N), state_out_elems(p, N)));
  float* T = S_ws;  // written only after the weight gradient has read S (same stream)
  float* gS = cw ? nullptr : c.take(state_in_elems(p, N));
  float* part = c.take(part_elems(p, N));
  float* xpart = c.take(rows_part_elems(p, kGemmGx, N));
  float* dpart = c.take(dot_part_elems(p, N));
  const FixedBufs fx = take_fixed(p, N, c);

  const float* S = saved_state;
  Planes xp;
  if ((grad_W && !S) || grad_pos || grad_rw) {
    if ((st = make_planes(x, p.x_dtype == TPCONV_BF16, N, p.D_in, p.C_in, c, xp, s)) != TPCONV_SUCCESS) return st;
  }
  if (grad_W && !S) {  // recompute the receiver state for the weight gradient
    StreamArgs a;
    recv_args(p, a, g, pos, x, rw);
    use_planes(a, xp);
    a.state = S_ws;
    if ((st = dev(launch_stream(kFwd, p.lmax, p.K, p.x_dtype == TPCONV_BF16, a, stream_items(a), s))) !=
        TPCONV_SUCCESS)
      return st;
    S = S_ws;
  }
  // planes of g_out (sender stream, gS, gW) and of W, before the fork
  Planes gp;
  if ((st = make_planes(grad_out, false, N, p.D_out, p.C_out, c, gp, s)) != TPCONV_SUCCESS) return st;
  WPlanes wp;
  if ((grad_x || grad_pos || grad_rw) && (st = make_w_planes(p, W, c, wp, s)) != TPCONV_SUCCESS) return st;
  Fork fork(s);
  const hipStream_t s2 = fork.side();
  if (grad_W) {  // side stream: gW = S^T g_out, first (T reuses the buffer of a recomputed S)
    st = cw ? run_cw_gw(p, N, S, grad_out, part, grad_W, s2) : run_gw(p, N, S, gp, part, grad_W, s2);
    if (st != TPCONV_SUCCESS) return st;
  }
  if (grad_x) {  // side stream: sender stream, then g_x = T W^T
    StreamArgs a;
    send_args(p, a, g, pos, grad_out, rw);
    use_planes(a, gp);
    a.state = T;
    if ((st = dev(launch_stream(kSnd, p.lmax, p.K, false, a, stream_items(a), s2))) != TPCONV_SUCCESS) return st;
    st = cw ? run_cw_contract(p, false, N, T, W, grad_x, s2)
            : run_gemm(p, kGemmGx, N, T, nullptr, wp, grad_x, xpart, s2);
    if (st != TPCONV_SUCCESS) return st;
  }
  // caller's stream: gS, the position gradient, and dL/dA of the radial MLP
  // one column at a time, dL/dA[k, j] = <gS[k], S^(j)[k]>: the receiver
  // stream forms S^(j) and writes only its dots with gS
  if (grad_rw && (st = run_gemm(p, kGemmGs, N, nullptr, &gp, wp, gS, nullptr, s)) != TPCONV_SUCCESS) return st;
  if (grad_pos) {
    st = run_pos_stream(p, kBwdPos, g, pos, x, xp, gp, wp, W, grad_out, nullptr, gS, grad_rw != nullptr, rw, fx,
                        grad_pos, s);
    if (st != TPCONV_SUCCESS) return st;
  }
  int64_t dot_items = 0;
  for (int j = 0; grad_rw && j < p.K; ++j) {
    StreamArgs a;
    recv_args(p, a, g, pos, x, rw);
    a.mlp_col = j;
    use_planes(a, xp);
    dot_items = stream_items(a);
    if ((size_t)dot_items * p.K * p.K > dot_part_elems(p, N)) return TPCONV_ERROR_INVALID_VALUE;
    a.dot_state = gS;
    a.dot_part = dpart + (size_t)j * dot_items * p.K;
    if ((st = dev(launch_stream(kFwd, p.lmax, p.K, p.x_dtype == TPCONV_BF16, a, dot_items, s))) != TPCONV_SUCCESS)
      return st;
  }
  if (grad_rw && (st = dev(launch_dot_reduce(dpart, dot_items, p.K, p.K, grad_rw, p.K, s))) != TPCONV_SUCCESS)
    return st;
  return fork.join();
}

tpconv_status double_backward_core(const Plan& p, const tpconv_graph* g, const float* pos, const void* x,
                                   const void* W, const float* rw, const float* grad_out, const float* gg_pos,
                                   float* d_W, float* d_x, float* d_grad_out, float* d_pos, float* d_rw, void* ws,
                                   hipStream_t s) {
  const int64_t N = g->num_nodes;
  const bool cw = channelwise(p);
  tpconv_status st;
  Carver c(ws);
  float* Sd = c.take(state_in_elems(p, N));
  float* Td = c.take(state_out_elems(p, N));
  float* part = c.take(part_elems(p, N));
  // gS is written on the caller's stream after d_W and d_grad_out have read
  // S_dot there, and nothing reads S_dot after it: the two share one buffer
  float* gS = cw ? nullptr : Sd;
  float* xpart = c.take(rows_part_elems(p, kGemmGx, N));  // d_x (side stream)
  float* opart = c.take(rows_part_elems(p, kGemmOut, N));  // d_grad_out (caller's stream)
  float* dpart = c.take(dot_part_elems(p, N));
  const FixedBufs fx = take_fixed(p, N, c);
  Planes xp;
  if (d_W || d_grad_out || d_pos || d_rw) {
    if ((st = make_planes(x, p.x_dtype == TPCONV_BF16, N, p.D_in, p.C_in, c, xp, s)) != TPCONV_SUCCESS) return st;
  }
  // planes of g_out (sender tangent stream, d_W, gS) and of W, before the fork
  Planes gp;
  if ((st = make_planes(grad_out, false, N, p.D_out, p.C_out, c, gp, s)) != TPCONV_SUCCESS) return st;
  WPlanes wp;
  if ((d_x || d_grad_out || d_pos || d_rw) && (st = make_w_planes(p, W, c, wp, s)) != TPCONV_SUCCESS) return st;
  Fork fork(s);
  const hipStream_t s2 = fork.side();
  if (d_x) {  // side stream: sender tangent stream, then d_x = T_dot W^T
    StreamArgs a;
    send_args(p, a, g, pos, grad_out, rw);
    use_planes(a, gp);
    a.ggpos = gg_pos;
    a.state = Td;
    if ((st = dev(launch_stream(kSndT, p.lmax, p.K, false, a, stream_items(a), s2))) != TPCONV_SUCCESS) return st;
    st = cw ? run_cw_contract(p, false, N, Td, W, d_x, s2) : run_gemm(p, kGemmGx, N, Td, nullptr, wp, d_x, xpart, s2);
    if (st != TPCONV_SUCCESS) return st;
  }
  if (d_W || d_grad_out) {  // caller's stream: tangent state, then its two contractions
    StreamArgs a;
    recv_args(p, a, g, pos, x, rw);
    use_planes(a, xp);
    a.ggpos = gg_pos;
    a.state = Sd;
    if ((st = dev(launch_stream(kJvp, p.lmax, p.K, p.x_dtype == TPCONV_BF16, a, stream_items(a), s))) !=
        TPCONV_SUCCESS)
      return st;
    if (d_W) {
      st = cw ? run_cw_gw(p, N, Sd, grad_out, part, d_W, s) : run_gw(p, N, Sd, gp, part, d_W, s);
      if (st != TPCONV_SUCCESS) return st;
    }
    if (d_grad_out) {
      st = cw ? run_cw_contract(p, true, N, Sd, W, d_grad_out, s)
              : run_gemm(p, kGemmOut, N, Sd, nullptr, wp, d_grad_out, opart, s);
      if (st != TPCONV_SUCCESS) return st;
    }
  }
  // caller's stream: gS, the Hessian term, and dL/dA of the radial MLP one
  // column at a time, dL/dA[k, j] = <gS[k], S_dot^(j)[k]> with the tangent
  // state formed in the mlp_col = j mode and dotted with gS in the stream
  if (d_rw && (st = run_gemm(p, kGemmGs, N, nullptr, &gp, wp, gS, nullptr, s)) != TPCONV_SUCCESS) return st;
  if (d_pos) {
    st = run_pos_stream(p, kBwdHess, g, pos, x, xp, gp, wp, W, grad_out, gg_pos, gS, d_rw != nullptr, rw, fx, d_pos,
                        s);
    if (st != TPCONV_SUCCESS) return st;
  }
  int64_t dot_items = 0;
  for (int j = 0; d_rw && j < p.K; ++j) {
    StreamArgs a;
    recv_args(p, a, g, pos, x, rw);
    a.mlp_col = j;
    use_planes(a, xp);
    a.ggpos = gg_pos;
    dot_items = stream_items(a);
    if ((size_t)dot_items * p.K * p.K > dot_part_elems(p, N)) return TPCONV_ERROR_INVALID_VALUE;
    a.dot_state = gS;
    a.dot_part = dpart + (size_t)j * dot_items * p.K;
    if ((st = dev(launch_stream(kJvp, p.lmax, p.K, p.x_dtype == TPCONV_BF16, a, dot_items, s))) != TPCONV_SUCCESS)
      return st;
  }
  if (d_rw && (st = dev(launch_dot_reduce(dpart, dot_items, p.K, p.K, d_rw, p.K, s))) != TPCONV_SUCCESS)
    return st;
  return fork.join();
}

// A ragged plan's inputs in the padded layout, carved from the front of the
// workspace; `rest` is where the uniform passes' workspace begins.
struct Padded {
  const Plan& p;
  Carver c;
  hipStream_t s;
  RaggedNodeMap in_map, out_map;
  tpconv_status st = TPCONV_SUCCESS;
  Padded(const Plan& plan, void* ws, hipStream_t stream)
      : p(plan), c(ws), s(stream), in_map(node_map(plan, true)), out_map(node_map(plan, false)) {}
  void* take_bytes(size_t b) { return c.take((b + 3) / 4); }
  const void* pack_nodes(const void* src, bool in_side, int elem, int64_t N) {
    const RaggedNodeMap& m = in_side ? in_map : out_map;
    void* dst = take_bytes((size_t)N * m.D * m.C * elem);
    if (st == TPCONV_SUCCESS) st = dev(launch_ragged_nodes(m, src, dst, N, elem, true, s));
    return dst;
  }
  const void* pack_w(const void* src, int elem) {
    void* dst = take_bytes(w_elems(p) * elem);
    if (st == TPCONV_SUCCESS) st = dev(launch_ragged_weights(weight_map(p), src, dst, elem, true, s));
    return dst;
  }
  float* out_nodes(bool in_side, int64_t N) {
    const RaggedNodeMap& m = in_side ? in_map : out_map;
    return static_cast<float*>(take_bytes((size_t)N * m.D * m.C * 4));
  }
  float* out_w() { return static_cast<float*>(take_bytes(w_elems(p) * 4)); }
  void unpack_nodes(const float* src, float* dst, bool in_side, int64_t N) {
    if (dst && st == TPCONV_SUCCESS) st = dev(launch_ragged_nodes(in_side ? in_map : out_map, src, dst, N, 4, false, s));
  }
  void unpack_w(const float* src, float* dst) {
    if (dst && st == TPCONV_SUCCESS) st = dev(launch_ragged_weights(weight_map(p), src, dst, 4, false, s));
  }
  void* rest() { return c.base + c.used; }
};

int xbytes(const Plan& p) { return p.x_dtype == TPCONV_BF16 ? 2 : 4; }
int wbytes(const Plan& p) { return p.w_dtype == TPCONV_BF16 ? 2 : 4; }

}  // namespace
}  // namespace tpconv

using namespace tpconv;

extern "C" {

const char* tpconv_status_string(tpconv_status st) {
  switch (st) {
    case TPCONV_SUCCESS: return "success";
    case TPCONV_ERROR_INVALID_VALUE: return "invalid value";
    case TPCONV_ERROR_IRREPS: return "invalid irreps";
    case TPCONV_ERROR_GRAPH: return "invalid graph";
    case TPCONV_ERROR_WORKSPACE: return "workspace missing or too small";
    case TPCONV_ERROR_UNSUPPORTED: return "unsupported configuration";
    case TPCONV_ERROR_DEVICE: return "device error";
    case TPCONV_ERROR_SCRATCH: return "problem needs more than the library's static scratch (64 MiB)";
  }
  return "unknown status";
}

tpconv_status tpconv_plan_create(tpconv_plan* out, const tpconv_desc* d) {
  if (!out || !d) return TPCONV_ERROR_INVALID_VALUE;
  *out = nullptr;
  try {
    auto* h = new (std::nothrow) tpconv_plan_s;
    if (!h) return TPCONV_ERROR_INVALID_VALUE;
    int st = build_plan(d->irreps_in, d->irreps_out, d->sh_lmax, d->num_basis, d->cutoff, d->envelope_p,
                        d->x_dtype, d->w_dtype, d->connection, h->plan);
    if (st == TPCONV_SUCCESS && (d->radial_mlp < 0 || d->radial_mlp > 1)) st = TPCONV_ERROR_INVALID_VALUE;
    if (st == TPCONV_SUCCESS && (d->deterministic < 0 || d->deterministic > 1)) st = TPCONV_ERROR_INVALID_VALUE;
    // the MLP's weight gradient contracts the state cotangent, which the
    // channel-wise passes never form
    if (st == TPCONV_SUCCESS && d->radial_mlp && d->connection == TPCONV_CHANNELWISE) st = TPCONV_ERROR_UNSUPPORTED;
    if (st != TPCONV_SUCCESS) {
      delete h;
      return (tpconv_status)st;
    }
    h->plan.radial_mlp = d->radial_mlp;
    h->plan.deterministic = d->deterministic;
    *out = h;
    return TPCONV_SUCCESS;
  } catch (...) {
    return TPCONV_ERROR_INVALID_VALUE;
  }
}

tpconv_status tpconv_plan_destroy(tpconv_plan plan) {
  delete plan;
  return TPCONV_SUCCESS;
}

tpconv_status tpconv_plan_info(tpconv_plan plan, int32_t* num_paths, int64_t* w_numel, int32_t* rows_in,
                               int32_t* ch_in, int32_t* rows_out, int32_t* ch_out) {
  if (!plan) return TPCONV_ERROR_INVALID_VALUE;
  const Plan& p = plan->plan;
  if (num_paths) *num_paths = p.P;
  if (w_numel) *w_numel = (int64_t)w_elems_caller(p);
  if (rows_in) *rows_in = p.D_in;
  if (ch_in) *ch_in = p.ragged ? 0 : p.C_in;
  if (rows_out) *rows_out = p.D_out;
  if (ch_out) *ch_out = p.ragged ? 0 : p.C_out;
  return TPCONV_SUCCESS;
}

tpconv_status tpconv_plan_path(tpconv_plan plan, int32_t path, int32_t* l123, int32_t* idx) {
  if (!plan || path < 0 || path >= plan->plan.P) return TPCONV_ERROR_INVALID_VALUE;
  const Path& q = plan->plan.paths[path];
  if (l123) {
    l123[0] = q.l1;
    l123[1] = q.l2;
    l123[2] = q.l3;
  }
  if (idx) {
    idx[0] = q.i1;
    idx[1] = q.i3;
  }
  return TPCONV_SUCCESS;
}

tpconv_status tpconv_plan_cg(tpconv_plan plan, int32_t path, double* out) {
  if (!plan || !out || path < 0 || path >= plan->plan.P) return TPCONV_ERROR_INVALID_VALUE;
  const auto& t = plan->plan.cg[path];
  std::memcpy(out, t.data(), t.size() * sizeof(double));
  return TPCONV_SUCCESS;
}

tpconv_status tpconv_state_size(tpconv_plan plan, int64_t N, size_t* bytes) {
  if (!plan || !bytes || N < 0) return TPCONV_ERROR_INVALID_VALUE;
  *bytes = state_in_elems(plan->plan, N) * sizeof(float);
  return TPCONV_SUCCESS;
}

tpconv_status tpconv_workspace_size(tpconv_plan plan, int32_t op, int64_t N, int64_t E, size_t* bytes) {
  if (!plan || !bytes || N < 0 || E < 0) return TPCONV_ERROR_INVALID_VALUE;
  const Plan& p = plan->plan;
  switch (op) {
    case TPCONV_OP_FORWARD: *bytes = ws_forward(p, N, false); break;
    case TPCONV_OP_FORWARD_SAVED: *bytes = ws_forward(p, N, true); break;
    case TPCONV_OP_BACKWARD: *bytes = ws_backward(p, N); break;
    case TPCONV_OP_DOUBLE_BACKWARD: *bytes = ws_double_backward(p, N); break;
    case TPCONV_OP_GRAPH_PREPARE: *bytes = graph_csc_workspace(N, E) + kAlign; break;
    case TPCONV_OP_GRAPH_ORDER: *bytes = graph_order_workspace(N); break;
    default: return TPCONV_ERROR_INVALID_VALUE;
  }
  return TPCONV_SUCCESS;
}

tpconv_status tpconv_graph_prepare(tpconv_plan plan, const tpconv_graph* g, int32_t* csc_colptr,
                                   int32_t* csc_receivers, int32_t validate, void* ws, size_t ws_bytes,
                                   void* stream) {
  if (!plan) return TPCONV_ERROR_INVALID_VALUE;
  tpconv_status st = check_graph(g, false);
  if (st != TPCONV_SUCCESS) return st;
  const int64_t N = g->num_nodes, E = g->num_edges;
  if (!csc_colptr || (E > 0 && !csc_receivers)) return TPCONV_ERROR_INVALID_VALUE;
  const size_t need = graph_csc_workspace(N, E) + kAlign;
  if (!ws || ws_bytes < need) return TPCONV_ERROR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (validate && N > 0) {
    int32_t* flag = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + graph_csc_workspace(N, E));
    if ((st = dev(launch_graph_validate(g->rowptr, g->senders, N, E, flag, s))) != TPCONV_SUCCESS) return st;
    int32_t host_flag = 0;
    if (hipMemcpyAsync(&host_flag, flag, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return TPCONV_ERROR_DEVICE;
    if (host_flag) return TPCONV_ERROR_GRAPH;
  }
  if (N == 0) return TPCONV_SUCCESS;
  return dev(graph_csc(g->rowptr, g->senders, N, E, csc_colptr, csc_receivers, ws, ws_bytes, s));
}

tpconv_status tpconv_graph_order(tpconv_plan plan, const tpconv_graph* g, const float* pos, int32_t* node_order,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (!plan) return TPCONV_ERROR_INVALID_VALUE;
  tpconv_status st = check_graph(g, false);
  if (st != TPCONV_SUCCESS) return st;
  const int64_t N = g->num_nodes;
  if (N == 0) return TPCONV_SUCCESS;
  if (!pos || !node_order) return TPCONV_ERROR_INVALID_VALUE;
  if (!ws || ws_bytes < graph_order_workspace(N)) return TPCONV_ERROR_WORKSPACE;
  return dev(graph_order(pos, N, node_order, ws, ws_bytes, static_cast<hipStream_t>(stream)));
}

tpconv_status tpconv_forward(tpconv_plan plan, const tpconv_graph* g, const float* pos, const void* x,
                             const void* W, float* out, float* saved_state, void* ws, size_t ws_bytes,
                             void* stream) {
  return tpconv_forward_mlp(plan, g, pos, x, W, nullptr, out, saved_state, ws, ws_bytes, stream);
}

tpconv_status tpconv_forward_mlp(tpconv_plan plan, const tpconv_graph* g, const float* pos, const void* x,
                                 const void* W, const float* radial_w, float* out, float* saved_state, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (!plan || (plan->plan.radial_mlp != 0) != (radial_w != nullptr)) return TPCONV_ERROR_INVALID_VALUE;
  tpconv_status st = check_graph(g, false);
  if (st != TPCONV_SUCCESS) return st;
  const Plan& p = plan->plan;
  const int64_t N = g->num_nodes;
  if (N > 0 && (!pos || !x || !W || !out)) return TPCONV_ERROR_INVALID_VALUE;
  if (!planes_addressable(p, N)) return TPCONV_ERROR_INVALID_VALUE;
  const size_t need = ws_forward(p, N, saved_state != nullptr);
  if (need > 0 && (!ws || ws_bytes < need)) return TPCONV_ERROR_WORKSPACE;
  if (N == 0) return TPCONV_SUCCESS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!p.ragged) return forward_core(p, g, pos, x, W, radial_w, out, saved_state, ws, s);
  Padded pd(p, ws, s);
  const void* xp = pd.pack_nodes(x, true, xbytes(p), N);
  const void* Wp = pd.pack_w(W, wbytes(p));
  float* outp = pd.out_nodes(false, N);
  if (pd.st != TPCONV_SUCCESS) return pd.st;
  if ((st = forward_core(p, g, pos, xp, Wp, radial_w, outp, saved_state, pd.rest(), s)) != TPCONV_SUCCESS) return st;
  pd.unpack_nodes(outp, out, false, N);
  return pd.st;
}

tpconv_status tpconv_backward(tpconv_plan plan, const tpconv_graph* g, const float* pos, const void* x,
                              const void* W, const float* grad_out, const float* saved_state, float* grad_x,
                              float* grad_W, float* grad_pos, void* ws, size_t ws_bytes, void* stream) {
  return tpconv_backward_mlp(plan, g, pos, x, W, nullptr, grad_out, saved_state, grad_x, grad_W, grad_pos, nullptr,
                             ws, ws_bytes, stream);
}

tpconv_status tpconv_backward_mlp(tpconv_plan plan, const tpconv_graph* g, const float* pos, const void* x,
                                  const void* W, const float* radial_w, const float* grad_out,
                                  const float* saved_state, float* grad_x, float* grad_W, float* grad_pos,
                                  float* grad_radial_w, void* ws, size_t ws_bytes, void* stream) {
  if (!plan || (plan->plan.radial_mlp != 0) != (radial_w != nullptr)) return TPCONV_ERROR_INVALID_VALUE;
  if (grad_radial_w && !radial_w) return TPCONV_ERROR_INVALID_VALUE;
  tpconv_status st = check_graph(g, grad_x != nullptr);
  if (st != TPCONV_SUCCESS) return st;
  if (!grad_x && !grad_W && !grad_pos && !grad_radial_w) return TPCONV_ERROR_INVALID_VALUE;
  const Plan& p = plan->plan;
  const int64_t N = g->num_nodes;
  if (N > 0 && (!pos || !x || !W || !grad_out)) return TPCONV_ERROR_INVALID_VALUE;
  if (!planes_addressable(p, N)) return TPCONV_ERROR_INVALID_VALUE;
  const size_t need = ws_backward(p, N);
  if (need > 0 && (!ws || ws_bytes < need)) return TPCONV_ERROR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0) {
    if (grad_W && (st = dev(launch_fill(grad_W, (int64_t)w_elems_caller(p), 0.f, s))) != TPCONV_SUCCESS) return st;
    if (grad_radial_w) return dev(launch_fill(grad_radial_w, (int64_t)p.K * p.K, 0.f, s));
    return TPCONV_SUCCESS;
  }
  if (!p.ragged)
    return backward_core(p, g, pos, x, W, radial_w, grad_out, saved_state, grad_x, grad_W, grad_pos, grad_radial_w,
                         ws, s);
  Padded pd(p, ws, s);
  const void* xp = pd.pack_nodes(x, true, xbytes(p), N);
  const void* Wp = pd.pack_w(W, wbytes(p));
  const float* gop = static_cast<const float*>(pd.pack_nodes(grad_out, false, 4, N));
  float* gxp = pd.out_nodes(true, N);
  float* gWp = pd.out_w();
  if (pd.st != TPCONV_SUCCESS) return pd.st;
  if ((st = backward_core(p, g, pos, xp, Wp, radial_w, gop, saved_state, grad_x ? gxp : nullptr,
                          grad_W ? gWp : nullptr, grad_pos, grad_radial_w, pd.rest(), s)) != TPCONV_SUCCESS)
    return st;
  pd.unpack_nodes(gxp, grad_x, true, N);
  pd.unpack_w(gWp, grad_W);
  return pd.st;
}

tpconv_status tpconv_double_backward(tpconv_plan plan, const tpconv_graph* g, const float* pos, const void* x,
                                     const void* W, const float* grad_out, const float* gg_pos, float* d_W,
                                     float* d_x, float* d_grad_out, float* d_pos, void* ws, size_t ws_bytes,
                                     void* stream) {
  return tpconv_double_backward_mlp(plan, g, pos, x, W, nullptr, grad_out, gg_pos, d_W, d_x, d_grad_out, d_pos,
                                    nullptr, ws, ws_bytes, stream);
}

tpconv_status tpconv_double_backward_mlp(tpconv_plan plan, const tpconv_graph* g, const float* pos, const void* x,
                                         const void* W, const float* radial_w, const float* grad_out,
                                         const float* gg_pos, float* d_W, float* d_x, float* d_grad_out,
                                         float* d_pos, float* d_radial_w, void* ws, size_t ws_bytes, void* stream) {
  if (!plan || (plan->plan.radial_mlp != 0) != (radial_w != nullptr)) return TPCONV_ERROR_INVALID_VALUE;
  if (d_radial_w && !radial_w) return TPCONV_ERROR_INVALID_VALUE;
  tpconv_status st = check_graph(g, d_x != nullptr);
  if (st != TPCONV_SUCCESS) return st;
  if (!d_W && !d_x && !d_grad_out && !d_pos && !d_radial_w) return TPCONV_ERROR_INVALID_VALUE;
  const Plan& p = plan->plan;
  const int64_t N = g->num_nodes;
  if (N > 0 && (!pos || !x || !W || !grad_out || !gg_pos)) return TPCONV_ERROR_INVALID_VALUE;
  if (!planes_addressable(p, N)) return TPCONV_ERROR_INVALID_VALUE;
  const size_t need = ws_double_backward(p, N);
  if (need > 0 && (!ws || ws_bytes < need)) return TPCONV_ERROR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0) {
    if (d_W && (st = dev(launch_fill(d_W, (int64_t)w_elems_caller(p), 0.f, s))) != TPCONV_SUCCESS) return st;
    if (d_radial_w) return dev(launch_fill(d_radial_w, (int64_t)p.K * p.K, 0.f, s));
    return TPCONV_SUCCESS;
  }
  if (!p.ragged)
    return double_backward_core(p, g, pos, x, W, radial_w, grad_out, gg_pos, d_W, d_x, d_grad_out, d_pos,
                                d_radial_w, ws, s);
  Padded pd(p, ws, s);
  const void* xp = pd.pack_nodes(x, true, xbytes(p), N);
  const void* Wp = pd.pack_w(W, wbytes(p));
  const float* gop = static_cast<const float*>(pd.pack_nodes(grad_out, false, 4, N));
  float* dxp = pd.out_nodes(true, N);
  float* dWp = pd.out_w();
  float* dgp = pd.out_nodes(false, N);
  if (pd.st != TPCONV_SUCCESS) return pd.st;
  if ((st = double_backward_core(p, g, pos, xp, Wp, radial_w, gop, gg_pos, d_W ? dWp : nullptr,
                                 d_x ? dxp : nullptr, d_grad_out ? dgp : nullptr, d_pos, d_radial_w, pd.rest(),
                                 s)) != TPCONV_SUCCESS)
    return st;
  pd.unpack_w(dWp, d_W);
  pd.unpack_nodes(dxp, d_x, true, N);
  pd.unpack_nodes(dgp, d_grad_out, false, N);
  return pd.st;
}

tpconv_status tpconv_plan_features(tpconv_plan plan, int64_t* feat_in, int64_t* feat_out) {
  if (!plan) return TPCONV_ERROR_INVALID_VALUE;
  const Plan& p = plan->plan;
  if (feat_in) *feat_in = p.ragged ? p.rag.F_in : (int64_t)p.D_in * p.C_in;
  if (feat_out) *feat_out = p.ragged ? p.rag.F_out : (int64_t)p.D_out * p.C_out;
  return TPCONV_SUCCESS;
}

tpconv_status tpconv_kernel_timing(int32_t enable) {
  return timing_set(enable != 0) ? TPCONV_SUCCESS : TPCONV_ERROR_DEVICE;
}

tpconv_status tpconv_kernel_timing_read(int32_t kernel, int64_t* launches, double* total_ms) {
  if (kernel < 0 || kernel >= kcCount || !launches || !total_ms) return TPCONV_ERROR_INVALID_VALUE;
  long long n = 0;
  double ms = 0.0;
  if (!timing_read(kernel, &n, &ms)) return TPCONV_ERROR_DEVICE;
  *launches = n;
  *total_ms = ms;
  return TPCONV_SUCCESS;
}

}  // extern "C"
