/*
 * tpconv.h — streaming Clebsch–Gordan tensor-product convolution on AMD MI355X (gfx950).
 *
 * The operation ("Sobek: streaming equivariant tensor-product convolution",
 * abstract): for every directed edge e = (s -> v) of a receiver-sorted graph,
 *
 *     r_e = pos[s] - pos[v],  d = |r_e|,  r_hat = r_e / d
 *     R_e[k]        = sqrt(2/c) sin(k pi d / c) / d * u_p(d / c),   k = 1..K
 *     Y_e[l2,m2]    = real spherical harmonics of r_hat (component normalised)
 *     U_e[p,ci,m3]  = sum_{m1,m2} C^p[m1,m2,m3] x[s][l1,ci,m1] Y_e[l2,m2]
 *     out[v][l3,co,m3] = sum_{e->v} sum_{p->l3} sum_{k,ci} R_e[k] W[k,p,ci,co] U_e[p,ci,m3]
 *
 * where p runs over the parity-allowed paths (l1, l2, l3) ("The Price of
 * Freedom", Approach: selection rules) and W mixes all input channels into all
 * output channels per (k, path) (the abstract's fully connected multiplicity
 * mixing).  The library evaluates it in the reassociated streaming form the
 * Sobek abstract describes: edge-local products are consumed directly into a
 * bounded per-receiver state S_v[k,p,ci,m3] = sum_{e->v} R_e[k] U_e[p,ci,m3],
 * followed by one dense contraction with W.  No per-edge weight, message or
 * adjoint is ever written to memory; every workspace is O(num_nodes).
 *
 * Conventions fixed by this library (the pages fix none of them):
 *   real harmonics: Y_00 = 1, l = 1 is sqrt(3) (y, z, x); order m = -l..l;
 *   CG tables: Racah complex CG taken to the real basis of the harmonics; for
 *   odd l1+l2+l3 the (purely imaginary) table's imaginary part; orthonormal;
 *   u_p(x) = 1 - (p+1)(p+2)/2 x^p + p(p+2) x^(p+1) - p(p+1)/2 x^(p+2) (x < 1).
 *   An edge with d = 0 uses r_hat := 0 and R at its d -> 0 limit and
 *   contributes no position gradient; an edge with d >= c contributes nothing.
 *
 * Layouts (row-major, all device memory owned by the caller):
 *   x, out, grad_out, grad_x, d_x, d_grad_out : [N][rows][C]   rows ordered by the
 *       irreps string, row of (irrep i, m) = offset(i) + l_i + m; channels innermost
 *   W, grad_W, d_W : [K][P][C_in][C_out], paths in tpconv_plan_path order
 *   Ragged multiplicities (irreps of one side with different channel counts,
 *   the abstract's varied feature structures): node tensors are [N][F], irrep
 *   i's block [2l_i+1][mul_i] following the blocks of irreps 0..i-1 (F from
 *   tpconv_plan_features); weights are [K][sum_p mul(l1 irrep of p) *
 *   mul(l3 irrep of p)], path p's block [mul_in][mul_out] following those of
 *   paths 0..p-1 (channel-wise: [K][sum_p mul_p]).  With one multiplicity per
 *   side these are exactly the layouts above.  Ragged plans pad every irrep of
 *   a side to the side's largest multiplicity inside the workspace (zero
 *   channels add nothing), so they cost what the padded uniform problem costs.
 *   pos, grad_pos, gg_pos : [N][3] fp32
 *   graph: rowptr[N+1], senders[E] int32, edges sorted by receiver;
 *          csc_colptr[N+1], csc_receivers[E] int32: the same edges sorted by
 *          sender (stable), built by tpconv_graph_prepare.
 * x and W are fp32 or bf16 (desc.x_dtype / desc.w_dtype); every output is fp32.
 *
 * Semantics: outputs are overwritten (never accumulated).  Calls are
 * asynchronous and ordered on the given HIP stream (a hipStream_t passed as
 * void*, NULL = the default stream).  Arguments are checked synchronously
 * before any launch; on an error nothing is launched and no output is written.
 * A plan is immutable after creation and may be used from several streams,
 * but concurrent calls must not share a workspace.
 *
 * Errors: every entry point returns a tpconv_status; no C++ exception crosses
 * the ABI.  TPCONV_ERROR_DEVICE reports a failed launch or a HIP runtime error
 * (asynchronous device faults surface at the caller's next synchronisation).
 */
#ifndef TPCONV_H_
#define TPCONV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tpconv_plan_s* tpconv_plan;

typedef enum {
  TPCONV_SUCCESS = 0,
  TPCONV_ERROR_INVALID_VALUE = 1, /* null pointer, negative size, bad enum */
  TPCONV_ERROR_IRREPS = 2,        /* unparsable irreps, channel-wise path with unequal multiplicities */
  TPCONV_ERROR_GRAPH = 3,         /* CSR fails validation (tpconv_graph_prepare, validate=1) */
  TPCONV_ERROR_WORKSPACE = 4,     /* workspace pointer null or smaller than required */
  TPCONV_ERROR_UNSUPPORTED = 5,   /* valid request the library does not implement */
  TPCONV_ERROR_DEVICE = 6,        /* HIP runtime or launch failure */
  TPCONV_ERROR_SCRATCH = 7        /* tpconv_forward_static: the problem needs more than the static scratch */
} tpconv_status;

/* Size of the per-device static scratch array behind tpconv_forward_static. */
#define TPCONV_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

typedef enum { TPCONV_F32 = 0, TPCONV_BF16 = 1 } tpconv_dtype;

/* How the shared weights mix channels (the Sobek page's abstract names two
 * operator families of the edge-conditioned tensor-product convolution).
 *   FULLY_CONNECTED ("uvw"): W[K][P][C_in][C_out], one C_in x C_out matrix per
 *                            (radial function, path).
 *   CHANNELWISE     ("uvu"): W[K][P][C], C_in = C_out = C, one weight per
 *                            (radial function, path, channel). */
typedef enum { TPCONV_FULLY_CONNECTED = 0, TPCONV_CHANNELWISE = 1 } tpconv_connection;

typedef enum {
  TPCONV_OP_FORWARD = 0,
  TPCONV_OP_BACKWARD = 1,
  TPCONV_OP_DOUBLE_BACKWARD = 2,
  TPCONV_OP_GRAPH_PREPARE = 3,
  TPCONV_OP_GRAPH_ORDER = 4,
  TPCONV_OP_FORWARD_SAVED = 5     /* tpconv_forward with a saved_state */
} tpconv_op;

typedef struct {
  const char* irreps_in;  /* e.g. "32x0e+32x1o+32x2e" or "64x0e+32x1o+16x2e"; l <= 3 */
  const char* irreps_out; /* same rules; may differ from irreps_in */
  int32_t sh_lmax;        /* degree of the edge harmonics, 0..3 */
  int32_t num_basis;      /* K radial functions: 8 or 16 */
  float cutoff;           /* c > 0 (Angstrom in the workloads) */
  int32_t envelope_p;     /* polynomial envelope exponent p >= 2 (6 in the workloads) */
  int32_t x_dtype;        /* tpconv_dtype of x */
  int32_t w_dtype;        /* tpconv_dtype of W */
  int32_t connection;     /* tpconv_connection; 0 (fully connected) when zero-initialised */
  int32_t radial_mlp;     /* 0: the K Bessel x envelope functions are the radial functions R_e[k];
                             1: a radial MLP in front of them (the _mlp entry points below) */
  int32_t deterministic;  /* 1: grad_pos and d_pos bitwise reproducible: every per-edge share is
                             added as an exact 64-bit fixed-point integer (shift from a first fp32
                             pass over the same stream, so the position stream runs twice);
                             0: fp32 atomic additions, last bits may vary between runs */
} tpconv_desc;

typedef struct {
  int64_t num_nodes;            /* N >= 0 */
  int64_t num_edges;            /* E >= 0, < 2^31 */
  const int32_t* rowptr;        /* device [N+1], receiver-sorted CSR */
  const int32_t* senders;       /* device [E] */
  const int32_t* csc_colptr;    /* device [N+1] or NULL (needed by backward passes) */
  const int32_t* csc_receivers; /* device [E] or NULL (needed by backward passes) */
  const int32_t* node_order;    /* device [N] permutation of 0..N-1, or NULL (identity): the order
                                   in which the edge streams visit nodes (tpconv_graph_order) */
} tpconv_graph;

/* Build a plan from the descriptor: parses the irreps, enumerates the
 * parity-allowed paths (input irrep, then l2, then output irrep) and computes
 * the real CG tables ("The Price of Freedom", Approach: selection rules;
 * Key results: the CG product is the fully expressive coupling).  Host only;
 * touches no device.  *out receives an owning handle (free with
 * tpconv_plan_destroy).  Errors: INVALID_VALUE (null pointers, K not in {8,16},
 * cutoff <= 0, p < 2, bad dtype or connection), IRREPS (bad strings, or for
 * the channel-wise connection a path whose input and output multiplicities
 * differ), UNSUPPORTED (l > 3). */
tpconv_status tpconv_plan_create(tpconv_plan* out, const tpconv_desc* desc);

/* Release a plan (NULL is accepted). */
tpconv_status tpconv_plan_destroy(tpconv_plan plan);

/* Sizes of a plan; any output pointer may be NULL.
 * rows_* = sum of (2l+1) over the irreps, ch_* = the multiplicity (0 when the
 * multiplicities of that side differ), w_numel = K * P * C_in * C_out (fully
 * connected) or K * P * C (channel-wise), or the ragged layout's count. */
tpconv_status tpconv_plan_info(tpconv_plan plan, int32_t* num_paths, int64_t* w_numel,
                               int32_t* rows_in, int32_t* ch_in, int32_t* rows_out, int32_t* ch_out);

/* Features per node of the input and output tensors in the caller's layout
 * (rows * C, or the ragged block sizes summed).  Either pointer may be NULL. */
tpconv_status tpconv_plan_features(tpconv_plan plan, int64_t* feat_in, int64_t* feat_out);

/* Path `path` (0 <= path < P): l123[3] = (l1, l2, l3), irrep_idx[2] = (input
 * irrep index, output irrep index).  Either pointer may be NULL. */
tpconv_status tpconv_plan_path(tpconv_plan plan, int32_t path, int32_t* l123, int32_t* irrep_idx);

/* The real CG table of a path as fp64, row-major [2l1+1][2l2+1][2l3+1]
 * (host memory, caller-owned).  These are the values the kernels use (rounded
 * to fp32 there). */
tpconv_status tpconv_plan_cg(tpconv_plan plan, int32_t path, double* out);

/* Bytes of caller-provided device workspace an operation needs for N nodes and
 * E edges ("Sobek" page, abstract: edge-local products go straight into a
 * receiver-side state of bounded size, so the tensor-product workspace does
 * not grow with the edge count).  For FORWARD, BACKWARD and DOUBLE_BACKWARD the
 * size does not depend on E: it holds node-sized states (S, its cotangent, the
 * sender state T) and the fixed-count partial sums of the weight gradient.
 * GRAPH_PREPARE needs O(N) int32 scratch for the sender sort (index
 * metadata, not tensor-product workspace), GRAPH_ORDER O(N) for the sort of
 * the nodes.  FORWARD's figure is for saved_state == NULL,
 * FORWARD_SAVED's for a forward that writes a saved state (it holds no S).
 * The passes also hold bf16 copies of the gathered features and of W for the
 * matrix cores (fp32 split into hi and lo planes; feature rows padded to a
 * multiple of 32 channels, W also transposed per (k, p); bf16 features with
 * 32-channel rows are used in place).
 * Errors: INVALID_VALUE (null plan or bytes, negative sizes, unknown op). */
tpconv_status tpconv_workspace_size(tpconv_plan plan, int32_t op, int64_t num_nodes,
                                    int64_t num_edges, size_t* bytes);

/* Bytes of the per-receiver state S (K * C_in * sum_p(2l3+1) fp32 per node)
 * that tpconv_forward can save for tpconv_backward. */
tpconv_status tpconv_state_size(tpconv_plan plan, int64_t num_nodes, size_t* bytes);

/* Build the sender-sorted view of the receiver-sorted graph (stable: for each
 * sender, receivers in increasing edge order).  The pages say nothing about how
 * the backward reaches the senders; the reading taken here is that the
 * sender-side passes (grad_x, and d_x of the double backward) stream the same
 * edges grouped by sender, the mirror of the receiver-side schedule ("Sobek"
 * page, abstract: the streaming form extends through the backward and double
 * backward), so they too accumulate into node-sized state without atomics.
 * g->rowptr, g->senders are read;
 * csc_colptr [N+1] and csc_receivers [E] are written (device).  With
 * validate != 0 the CSR is first checked on the device (rowptr[0] = 0,
 * non-decreasing, rowptr[N] = E, 0 <= sender < N); this synchronises the
 * stream and returns TPCONV_ERROR_GRAPH without writing the outputs when the
 * check fails.  Workspace: tpconv_workspace_size(GRAPH_PREPARE). */
tpconv_status tpconv_graph_prepare(tpconv_plan plan, const tpconv_graph* g, int32_t* csc_colptr,
                                   int32_t* csc_receivers, int32_t validate, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* A spatial visiting order of the nodes for g->node_order: the nodes sorted
 * by the Morton code of their positions (30 bits over the bounding cube; ties,
 * which only coincident quantised positions produce, by node id), so the
 * deterministic permutation does not depend on the graph's node numbering.  The
 * pages say nothing about the order in which receivers are processed; every
 * receiver's result is independent of it (grad_pos only up to the rounding
 * of its atomic additions).  Streams that visit spatially close receivers one
 * after another gather mostly the same sender rows, so those gathers hit the
 * L2 cache of the XCD that runs them.  pos: device [N][3]; node_order: device
 * [N] (written).  Workspace: tpconv_workspace_size(GRAPH_ORDER), O(N).
 * Errors: INVALID_VALUE (null pointers), WORKSPACE, DEVICE. */
tpconv_status tpconv_graph_order(tpconv_plan plan, const tpconv_graph* g, const float* pos, int32_t* node_order,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Forward: out = conv(pos, x, W) as defined at the top of this header.
 * saved_state: NULL, or device memory of tpconv_state_size bytes that receives
 * the receiver state S for a later tpconv_backward (then the workspace needs
 * tpconv_workspace_size(FORWARD_SAVED) bytes, which may be 0 and then allows
 * NULL).  Device pointers: pos, x, W, out (and saved_state).
 * Limit of every pass: the bf16 planes of x and of grad_out
 * (N * rows * roundup(C, 32) * 2 bytes each) stay below 4 GiB, or the call
 * returns INVALID_VALUE. */
tpconv_status tpconv_forward(tpconv_plan plan, const tpconv_graph* g, const float* pos,
                             const void* x, const void* W, float* out, float* saved_state,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Backward ("Sobek" page, abstract: the streaming formulation covers the
 * backward pass; the same receiver-side schedule, with no per-edge adjoint
 * stored).  Gradients of <grad_out, out>: grad_x [N][rows_in][C_in],
 * grad_W [K][P][C_in][C_out],
 * grad_pos [N][3]; each may be NULL to skip it (at least one must be given).
 * saved_state: S from tpconv_forward with the same inputs, or NULL to recompute it.
 * Needs g->csc_colptr / csc_receivers when grad_x is requested.  grad_pos sums
 * per-edge contributions with fp32 atomics, so its last bits may vary between
 * runs unless the plan was created with desc.deterministic = 1; grad_x and
 * grad_W are deterministic. */
tpconv_status tpconv_backward(tpconv_plan plan, const tpconv_graph* g, const float* pos,
                              const void* x, const void* W, const float* grad_out,
                              const float* saved_state, float* grad_x, float* grad_W,
                              float* grad_pos, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Double backward ("Sobek" page, abstract: the streaming formulation covers the
 * double backward; tangent states are node-sized like S and T) of the scalar
 * force loss L = sum_n <gg_pos[n], grad_pos[n]>, where grad_pos is the
 * backward above for the given grad_out:
 *   d_W = dL/dW, d_x = dL/dx, d_grad_out = dL/dgrad_out, d_pos = dL/dpos
 *   (each may be NULL; at least one must be given).
 * With phi_e = gg_pos[s] - gg_pos[v], L = sum_e <phi_e, grad_r eps_e> for the
 * edge energies eps_e = <grad_out[v], message_e>; L is linear in W, x and
 * grad_out, and its position derivative is the Hessian term
 * dL/dpos[s] += H_e phi_e, dL/dpos[v] -= H_e phi_e (H_e the Hessian of eps_e
 * w.r.t. r_e, from R'' and the second derivatives of the harmonics), summed
 * like grad_pos (fp32 atomics, or exact fixed point for deterministic plans).
 * Needs the CSC view when d_x is requested.
 * Errors as tpconv_backward. */
tpconv_status tpconv_double_backward(tpconv_plan plan, const tpconv_graph* g, const float* pos,
                                     const void* x, const void* W, const float* grad_out,
                                     const float* gg_pos, float* d_W, float* d_x,
                                     float* d_grad_out, float* d_pos, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* tpconv_forward without workspace and without any allocation, for callers
 * that cannot allocate device memory (code under HIP stream capture, tight
 * serving loops, harnesses that forbid hipMalloc).  The receiver state S is
 * kept in a file-scope device array of TPCONV_STATIC_SCRATCH_BYTES (64 MiB)
 * that every GPU the library runs on holds until the process ends; it fits
 * problems whose tpconv_workspace_size(FORWARD) is at most that size (the
 * state S and the bf16 planes of x and W: for example N <= 1794 nodes at 32
 * channels of 0e+1o+2e with K = 8, 35 KiB of state and 1.1 KiB of planes per
 * node, or N <= 26208 at 8 channels of 0e+1o, 2.5 KiB).  Larger problems
 * return TPCONV_ERROR_SCRATCH before any launch.  The array is looked
 * up on the first call on each device (the call then needs that device
 * current).  Same arguments, results and errors as tpconv_forward otherwise.
 * All calls on one GPU share the array: calls that overlap in time on one GPU
 * (several streams or threads) race and must be serialised by the caller. */
tpconv_status tpconv_forward_static(tpconv_plan plan, const tpconv_graph* g, const float* pos, const void* x,
                                    const void* W, float* out, void* stream);

/* Radial MLP front end.  The pages name learned radial networks only as the
 * usual setting of the layer; the reading taken keeps the reassociation of
 * the Sobek page's abstract intact: the network's last hidden layer is the K
 * radial functions the node-sized state is built from, and its output layer
 * folds into W.  For a plan created with desc.radial_mlp = 1,
 *   R_e[k] = silu(z_ek),  z_ek = sum_j radial_w[k][j] B_j(d_e),  silu(z) = z / (1 + exp(-z)),
 * with B the K Bessel x envelope functions (no bias: R vanishes with B at the
 * cutoff).  radial_w: device fp32 [K][K], row k = output function k.  These
 * entry points are tpconv_forward / _backward / _double_backward with the
 * network in front; the plain ones reject such a plan, and these reject a
 * plan without it (INVALID_VALUE).  The backward also returns
 * grad_radial_w = dL/dradial_w [K][K] and the double backward
 * d_radial_w = dL_F/dradial_w (each may be NULL), formed one column j at a
 * time as <gS[k], S^(j)[k]>: S^(j) is the state (tangent state) with R_e[k]
 * replaced by dR_e[k]/dradial_w[k][j], formed tile by tile in the receiver
 * stream and dotted with gS there (never stored), so a requested weight
 * gradient costs K more passes of the receiver stream.  Deterministic.
 * Channel-wise plans do not take the network (UNSUPPORTED at plan creation).
 * Workspace: tpconv_workspace_size of the same op (for such plans also K
 * floats per stream work item: N x units x 32-channel slices). */
tpconv_status tpconv_forward_mlp(tpconv_plan plan, const tpconv_graph* g, const float* pos, const void* x,
                                 const void* W, const float* radial_w, float* out, float* saved_state,
                                 void* workspace, size_t workspace_bytes, void* stream);
tpconv_status tpconv_backward_mlp(tpconv_plan plan, const tpconv_graph* g, const float* pos, const void* x,
                                  const void* W, const float* radial_w, const float* grad_out,
                                  const float* saved_state, float* grad_x, float* grad_W, float* grad_pos,
                                  float* grad_radial_w, void* workspace, size_t workspace_bytes, void* stream);
tpconv_status tpconv_double_backward_mlp(tpconv_plan plan, const tpconv_graph* g, const float* pos,
                                         const void* x, const void* W, const float* radial_w,
                                         const float* grad_out, const float* gg_pos, float* d_W, float* d_x,
                                         float* d_grad_out, float* d_pos, float* d_radial_w, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* Kernel classes for tpconv_kernel_timing_read. */
typedef enum {
  TPCONV_KERNEL_STREAM_FWD = 0,    /* receiver stream: S */
  TPCONV_KERNEL_STREAM_JVP = 1,    /* receiver stream: S_dot */
  TPCONV_KERNEL_STREAM_SND = 2,    /* sender stream: T */
  TPCONV_KERNEL_STREAM_SNDT = 3,   /* sender stream: T_dot */
  TPCONV_KERNEL_STREAM_BWDPOS = 4, /* receiver stream: grad_pos */
  TPCONV_KERNEL_GEMM_OUT = 5,      /* out = S . W  (also d_grad_out) */
  TPCONV_KERNEL_GEMM_GS = 6,       /* gS = grad_out . W^T */
  TPCONV_KERNEL_GEMM_GX = 7,       /* grad_x = T . W^T  (also d_x) */
  TPCONV_KERNEL_GEMM_GW = 8,       /* grad_W partials = S^T . grad_out  (also d_W) */
  TPCONV_KERNEL_GW_REDUCE = 9,     /* ordered sums of split partials (grad_W; out and grad_x when split) */
  TPCONV_KERNEL_FILL = 10,         /* zero fills */
  TPCONV_KERNEL_GRAPH = 11,        /* sender-sorted view construction */
  TPCONV_KERNEL_CW_CONTRACT = 12,  /* channel-wise: out, grad_x, d_grad_out, d_x from S / T */
  TPCONV_KERNEL_CW_GW = 13,        /* channel-wise: grad_W partials (also d_W) */
  TPCONV_KERNEL_CW_REDUCE = 14,    /* channel-wise: ordered sum of the partials */
  TPCONV_KERNEL_STREAM_HESS = 15,  /* receiver stream: position derivative of the force loss */
  TPCONV_KERNEL_STATE_DOT = 16,    /* per-k dot products of two states (radial MLP weight gradient) */
  TPCONV_KERNEL_COUNT = 17
} tpconv_kernel;

/* Diagnostics for roofline measurements (not needed for computing).
 * tpconv_kernel_timing(1) clears the table and starts bracketing every
 * library launch with two HIP events recorded on the launch's own stream;
 * tpconv_kernel_timing(0) stops (and clears).  Timing adds event packets
 * between launches, so time end-to-end throughput with it disabled.
 * tpconv_kernel_timing_read waits for the recorded events of one kernel class
 * and returns the number of launches and their summed duration (ms).
 * Process-global; not meant for concurrent use from several threads. */
tpconv_status tpconv_kernel_timing(int32_t enable);
tpconv_status tpconv_kernel_timing_read(int32_t kernel, int64_t* launches, double* total_ms);

/* Static description of a status code. */
const char* tpconv_status_string(tpconv_status status);

#ifdef __cplusplus
}
#endif

#endif /* TPCONV_H_ */
