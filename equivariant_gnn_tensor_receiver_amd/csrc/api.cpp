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

// log2 of the channel tile of the edge streams: the largest power of two
// dividing C, at most 64 and at least 4 (lanes are paired in fours by the
// 4x4 outer products; a tile past C is masked).
int ct_log2_of(int C) {
  int t = 0;
  while (t < 6 && (C % (2 << t)) == 0) ++t;
  return t < 2 ? 2 : t;
}

// Reduction splits of the gW product over blocks: enough waves to fill the
// chip (with up to 4 waves per block) while each split of the largest group
// keeps >= 512 reductions (smaller groups get shorter splits).
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

size_t ws_forward(const Plan& p, int64_t N, bool have_saved) {
  return have_saved ? 0 : align_up(state_in_elems(p, N) * 4);
}

size_t ws_backward(const Plan& p, int64_t N) {
  // S (recomputed when not saved), gS (fully connected only), T, gW partials
  return align_up(state_in_elems(p, N) * 4) * (channelwise(p) ? 1 : 2) + align_up(state_out_elems(p, N) * 4) +
         align_up(part_elems(p, N) * 4);
}

size_t ws_double_backward(const Plan& p, int64_t N) {
  return align_up(state_in_elems(p, N) * 4) + align_up(state_out_elems(p, N) * 4) +
         align_up(part_elems(p, N) * 4);
}

tpconv_status dev(hipError_t e) { return e == hipSuccess ? TPCONV_SUCCESS : TPCONV_ERROR_DEVICE; }

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

void fill_common(const Plan& p, StreamArgs& a, int64_t N, const float* pos) {
  std::memset(&a, 0, sizeof(a));
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
}

void set_units(const Plan& p, StreamArgs& a, const std::vector<std::vector<int>>& units) {
  a.nunits = (int32_t)units.size();
  a.bundled = p.natural ? 1 : 0;
  for (size_t u = 0; u < units.size(); ++u)
    for (size_t i = 0; i < units[u].size(); ++i) a.unit_paths[u][i] = (int8_t)units[u][i];
}

// Receiver-side stream over the CSR: gathered features x [N][D_in][C_in],
// state S (or S_dot) in the output-group layout.
// Low mean degree (nearly every node one 64-edge batch): the units of a node
// may share one block and its batch geometry (the launcher decides per mode).
// With more batches per node the block waits for its slowest unit at every
// batch boundary, which measured slower than recomputing the geometry per unit.
bool share_geometry(const tpconv_graph* g) { return g->num_edges <= 48 * g->num_nodes; }

void recv_args(const Plan& p, StreamArgs& a, const tpconv_graph* g, const float* pos, const void* x) {
  const int64_t N = g->num_nodes;
  fill_common(p, a, N, pos);
  a.share_geometry = share_geometry(g);
  a.ptr = g->rowptr;
  a.nbr = g->senders;
  a.feat = x;
  a.feat_rows = p.D_in;
  a.C = p.C_in;
  a.ct_log2 = ct_log2_of(p.C_in);
  a.ntiles = (p.C_in + (1 << a.ct_log2) - 1) >> a.ct_log2;
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
void send_args(const Plan& p, StreamArgs& a, const tpconv_graph* g, const float* pos, const float* gout) {
  const int64_t N = g->num_nodes;
  fill_common(p, a, N, pos);
  a.share_geometry = share_geometry(g);
  a.ptr = g->csc_colptr;
  a.nbr = g->csc_receivers;
  a.feat = gout;
  a.feat_rows = p.D_out;
  a.C = p.C_out;
  a.ct_log2 = ct_log2_of(p.C_out);
  a.ntiles = (p.C_out + (1 << a.ct_log2) - 1) >> a.ct_log2;
  for (int i = 0; i < p.P; ++i) {
    const Path& q = p.paths[i];
    const Group& ig = p.in_groups[q.i1];
    a.paths[i] = StreamPath{q.l1, q.l2, q.l3, p.out_groups[q.i3].row_off, N * ig.base_per_node,
                            (int32_t)ig.paths.size() * p.C_out, q.q_in, i, p.in_groups[q.i1].row_off};
  }
  set_units(p, a, p.send_units);
}

// Work items of a stream launch: one wave per (node, channel tile, unit).
int64_t stream_items(const StreamArgs& a) { return (int64_t)a.num_nodes * a.ntiles * a.nunits; }

// Groups of a GEMM over the output irreps (Out, Gs, Gw) or input irreps (Gx).
int gemm_setup(const Plan& p, int kind, int64_t N, GemmArgs& a, int splits) {
  std::memset(&a, 0, sizeof(a));
  a.P = p.P;
  a.K = p.K;
  a.C_in = p.C_in;
  a.C_out = p.C_out;
  a.splits = splits;
  a.w_bf16 = p.w_dtype == TPCONV_BF16;
  const bool in_side = kind == kGemmGx;
  const auto& groups = in_side ? p.in_groups : p.out_groups;
  a.D_feat = in_side ? p.D_in : p.D_out;
  int npl = 0, ng = 0;
  int64_t part = 0;
  for (const auto& g : groups) {
    const int npg = (int)g.paths.size();
    if (npg == 0 && (kind == kGemmGs || kind == kGemmGw)) continue;
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

// 16-byte operand loads need channel counts that are multiples of 16 and
// 16-byte aligned base pointers.
void set_vec(const Plan& p, GemmArgs& a) {
  a.vec = (p.C_in % 16 == 0) && (p.C_out % 16 == 0) && aligned16(a.state) && aligned16(a.feat) && aligned16(a.W);
}

tpconv_status run_gemm(const Plan& p, int kind, int64_t N, const float* state, const float* feat,
                       const void* W, float* out, int splits, hipStream_t s) {
  GemmArgs a;
  gemm_setup(p, kind, N, a, splits);
  a.state = state;
  a.feat = feat;
  a.W = W;
  a.out = out;
  set_vec(p, a);
  return dev(launch_gemm(kind, a, s));
}

tpconv_status run_gw(const Plan& p, int64_t N, const float* state, const float* gout, float* part, float* gW,
                     hipStream_t s) {
  const int splits = gw_splits(p, N);
  GemmArgs a;
  gemm_setup(p, kGemmGw, N, a, splits);
  a.state = state;
  a.feat = gout;
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
  }
  return "unknown status";
}

tpconv_status tpconv_plan_create(tpconv_plan* out, const tpconv_desc* d) {
  if (!out || !d) return TPCONV_ERROR_INVALID_VALUE;
  *out = nullptr;
  try {
    auto* h = new (std::nothrow) tpconv_plan_s;
    if (!h) return TPCONV_ERROR_INVALID_VALUE;
    const int st = build_plan(d->irreps_in, d->irreps_out, d->sh_lmax, d->num_basis, d->cutoff, d->envelope_p,
                              d->x_dtype, d->w_dtype, d->connection, h->plan);
    if (st != TPCONV_SUCCESS) {
      delete h;
      return (tpconv_status)st;
    }
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
  if (w_numel) *w_numel = (int64_t)w_elems(p);
  if (rows_in) *rows_in = p.D_in;
  if (ch_in) *ch_in = p.C_in;
  if (rows_out) *rows_out = p.D_out;
  if (ch_out) *ch_out = p.C_out;
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
    case TPCONV_OP_BACKWARD: *bytes = ws_backward(p, N); break;
    case TPCONV_OP_DOUBLE_BACKWARD: *bytes = ws_double_backward(p, N); break;
    case TPCONV_OP_GRAPH_PREPARE: *bytes = graph_csc_workspace(N, E) + kAlign; break;
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

tpconv_status tpconv_forward(tpconv_plan plan, const tpconv_graph* g, const float* pos, const void* x,
                             const void* W, float* out, float* saved_state, void* ws, size_t ws_bytes,
                             void* stream) {
  if (!plan) return TPCONV_ERROR_INVALID_VALUE;
  tpconv_status st = check_graph(g, false);
  if (st != TPCONV_SUCCESS) return st;
  const Plan& p = plan->plan;
  const int64_t N = g->num_nodes;
  if (N > 0 && (!pos || !x || !W || !out)) return TPCONV_ERROR_INVALID_VALUE;
  const size_t need = ws_forward(p, N, saved_state != nullptr);
  if (need > 0 && (!ws || ws_bytes < need)) return TPCONV_ERROR_WORKSPACE;
  if (N == 0) return TPCONV_SUCCESS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* S = saved_state ? saved_state : static_cast<float*>(ws);
  StreamArgs a;
  recv_args(p, a, g, pos, x);
  a.state = S;
  if ((st = dev(launch_stream(kFwd, p.lmax, p.K, p.x_dtype == TPCONV_BF16, a, stream_items(a), s))) !=
      TPCONV_SUCCESS)
    return st;
  if (channelwise(p)) return run_cw_contract(p, true, N, S, W, out, s);
  return run_gemm(p, kGemmOut, N, S, nullptr, W, out, 1, s);
}

tpconv_status tpconv_backward(tpconv_plan plan, const tpconv_graph* g, const float* pos, const void* x,
                              const void* W, const float* grad_out, const float* saved_state, float* grad_x,
                              float* grad_W, float* grad_pos, void* ws, size_t ws_bytes, void* stream) {
  if (!plan) return TPCONV_ERROR_INVALID_VALUE;
  tpconv_status st = check_graph(g, grad_x != nullptr);
  if (st != TPCONV_SUCCESS) return st;
  if (!grad_x && !grad_W && !grad_pos) return TPCONV_ERROR_INVALID_VALUE;
  const Plan& p = plan->plan;
  const int64_t N = g->num_nodes;
  if (N > 0 && (!pos || !x || !W || !grad_out)) return TPCONV_ERROR_INVALID_VALUE;
  const size_t need = ws_backward(p, N);
  if (need > 0 && (!ws || ws_bytes < need)) return TPCONV_ERROR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0) {
    if (grad_W) return dev(launch_fill(grad_W, (int64_t)w_elems(p), 0.f, s));
    return TPCONV_SUCCESS;
  }
  const bool cw = channelwise(p);
  Carver c(ws);
  float* S_ws = c.take(state_in_elems(p, N));
  float* gS = cw ? nullptr : c.take(state_in_elems(p, N));
  float* T = c.take(state_out_elems(p, N));
  float* part = c.take(part_elems(p, N));

  const float* S = saved_state;
  if (grad_W && !S) {  // recompute the receiver state for the weight gradient
    StreamArgs a;
    recv_args(p, a, g, pos, x);
    a.state = S_ws;
    if ((st = dev(launch_stream(kFwd, p.lmax, p.K, p.x_dtype == TPCONV_BF16, a, stream_items(a), s))) !=
        TPCONV_SUCCESS)
      return st;
    S = S_ws;
  }
  Fork fork(s);
  const hipStream_t s2 = fork.side();
  if (grad_x) {  // side stream: sender stream, then g_x = T W^T
    StreamArgs a;
    send_args(p, a, g, pos, grad_out);
    a.state = T;
    if ((st = dev(launch_stream(kSnd, p.lmax, p.K, false, a, stream_items(a), s2))) != TPCONV_SUCCESS) return st;
    st = cw ? run_cw_contract(p, false, N, T, W, grad_x, s2) : run_gemm(p, kGemmGx, N, T, nullptr, W, grad_x, 1, s2);
    if (st != TPCONV_SUCCESS) return st;
  }
  if (grad_W) {  // side stream: gW = S^T g_out
    st = cw ? run_cw_gw(p, N, S, grad_out, part, grad_W, s2) : run_gw(p, N, S, grad_out, part, grad_W, s2);
    if (st != TPCONV_SUCCESS) return st;
  }
  if (grad_pos) {  // caller's stream: gS = g_out W^T (formed in registers when channel-wise), then the stream
    if (!cw && (st = run_gemm(p, kGemmGs, N, nullptr, grad_out, W, gS, 1, s)) != TPCONV_SUCCESS) return st;
    if ((st = dev(launch_fill(grad_pos, 3 * N, 0.f, s))) != TPCONV_SUCCESS) return st;
    StreamArgs a;
    recv_args(p, a, g, pos, x);
    set_units(p, a, p.pos_units);
    a.gstate = gS;
    a.gpos = grad_pos;
    if (cw) {
      a.cw = 1;
      a.W = W;
      a.w_bf16 = p.w_dtype == TPCONV_BF16;
      a.gout = grad_out;
      a.gout_rows = p.D_out;
    }
    if ((st = dev(launch_stream(kBwdPos, p.lmax, p.K, p.x_dtype == TPCONV_BF16, a, stream_items(a), s))) !=
        TPCONV_SUCCESS)
      return st;
  }
  return fork.join();
}

tpconv_status tpconv_double_backward(tpconv_plan plan, const tpconv_graph* g, const float* pos, const void* x,
                                     const void* W, const float* grad_out, const float* gg_pos, float* d_W,
                                     float* d_x, float* d_grad_out, void* ws, size_t ws_bytes, void* stream) {
  if (!plan) return TPCONV_ERROR_INVALID_VALUE;
  tpconv_status st = check_graph(g, d_x != nullptr);
  if (st != TPCONV_SUCCESS) return st;
  if (!d_W && !d_x && !d_grad_out) return TPCONV_ERROR_INVALID_VALUE;
  const Plan& p = plan->plan;
  const int64_t N = g->num_nodes;
  if (N > 0 && (!pos || !x || !W || !grad_out || !gg_pos)) return TPCONV_ERROR_INVALID_VALUE;
  const size_t need = ws_double_backward(p, N);
  if (need > 0 && (!ws || ws_bytes < need)) return TPCONV_ERROR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0) {
    if (d_W) return dev(launch_fill(d_W, (int64_t)w_elems(p), 0.f, s));
    return TPCONV_SUCCESS;
  }
  const bool cw = channelwise(p);
  Carver c(ws);
  float* Sd = c.take(state_in_elems(p, N));
  float* Td = c.take(state_out_elems(p, N));
  float* part = c.take(part_elems(p, N));
  Fork fork(s);
  const hipStream_t s2 = fork.side();
  if (d_x) {  // side stream: sender tangent stream, then d_x = T_dot W^T
    StreamArgs a;
    send_args(p, a, g, pos, grad_out);
    a.ggpos = gg_pos;
    a.state = Td;
    if ((st = dev(launch_stream(kSndT, p.lmax, p.K, false, a, stream_items(a), s2))) != TPCONV_SUCCESS) return st;
    st = cw ? run_cw_contract(p, false, N, Td, W, d_x, s2) : run_gemm(p, kGemmGx, N, Td, nullptr, W, d_x, 1, s2);
    if (st != TPCONV_SUCCESS) return st;
  }
  if (d_W || d_grad_out) {  // caller's stream: tangent state, then its two contractions
    StreamArgs a;
    recv_args(p, a, g, pos, x);
    a.ggpos = gg_pos;
    a.state = Sd;
    if ((st = dev(launch_stream(kJvp, p.lmax, p.K, p.x_dtype == TPCONV_BF16, a, stream_items(a), s))) !=
        TPCONV_SUCCESS)
      return st;
    if (d_W) {
      st = cw ? run_cw_gw(p, N, Sd, grad_out, part, d_W, s) : run_gw(p, N, Sd, grad_out, part, d_W, s);
      if (st != TPCONV_SUCCESS) return st;
    }
    if (d_grad_out) {
      st = cw ? run_cw_contract(p, true, N, Sd, W, d_grad_out, s)
              : run_gemm(p, kGemmOut, N, Sd, nullptr, W, d_grad_out, 1, s);
      if (st != TPCONV_SUCCESS) return st;
    }
  }
  return fork.join();
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
