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
  TPCONV_ERROR_IRREPS = 2,        /* unparsable irreps, non-uniform multiplicity, l > 3 */
  TPCONV_ERROR_GRAPH = 3,         /* CSR fails validation (tpconv_graph_prepare, validate=1) */
  TPCONV_ERROR_WORKSPACE = 4,     /* workspace pointer null or smaller than required */
  TPCONV_ERROR_UNSUPPORTED = 5,   /* valid request the library does not implement */
  TPCONV_ERROR_DEVICE = 6         /* HIP runtime or launch failure */
} tpconv_status;

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
  TPCONV_OP_GRAPH_PREPARE = 3
} tpconv_op;

typedef struct {
  const char* irreps_in;  /* e.g. "32x0e+32x1o+32x2e"; one multiplicity, l <= 3 */
  const char* irreps_out; /* same rules; may differ from irreps_in */
  int32_t sh_lmax;        /* degree of the edge harmonics, 0..3 */
  int32_t num_basis;      /* K radial functions: 8 or 16 */
  float cutoff;           /* c > 0 (Angstrom in the workloads) */
  int32_t envelope_p;     /* polynomial envelope exponent p >= 2 (6 in the workloads) */
  int32_t x_dtype;        /* tpconv_dtype of x */
  int32_t w_dtype;        /* tpconv_dtype of W */
  int32_t connection;     /* tpconv_connection; 0 (fully connected) when zero-initialised */
} tpconv_desc;

typedef struct {
  int64_t num_nodes;            /* N >= 0 */
  int64_t num_edges;            /* E >= 0, < 2^31 */
  const int32_t* rowptr;        /* device [N+1], receiver-sorted CSR */
  const int32_t* senders;       /* device [E] */
  const int32_t* csc_colptr;    /* device [N+1] or NULL (needed by backward passes) */
  const int32_t* csc_receivers; /* device [E] or NULL (needed by backward passes) */
} tpconv_graph;

/* Build a plan from the descriptor: parses the irreps, enumerates the
 * parity-allowed paths (input irrep, then l2, then output irrep) and computes
 * the real CG tables ("The Price of Freedom", Approach: selection rules;
 * Key results: the CG product is the fully expressive coupling).  Host only;
 * touches no device.  *out receives an owning handle (free with
 * tpconv_plan_destroy).  Errors: INVALID_VALUE (null pointers, K not in {8,16},
 * cutoff <= 0, p < 2, bad dtype or connection), IRREPS (bad strings, or
 * C_in != C_out for the channel-wise connection), UNSUPPORTED (l > 3). */
tpconv_status tpconv_plan_create(tpconv_plan* out, const tpconv_desc* desc);

/* Release a plan (NULL is accepted). */
tpconv_status tpconv_plan_destroy(tpconv_plan plan);

/* Sizes of a plan; any output pointer may be NULL.
 * rows_* = sum of (2l+1) over the irreps, ch_* = the multiplicity,
 * w_numel = K * P * C_in * C_out (fully connected) or K * P * C (channel-wise). */
tpconv_status tpconv_plan_info(tpconv_plan plan, int32_t* num_paths, int64_t* w_numel,
                               int32_t* rows_in, int32_t* ch_in, int32_t* rows_out, int32_t* ch_out);

/* Path `path` (0 <= path < P): l123[3] = (l1, l2, l3), irrep_idx[2] = (input
 * irrep index, output irrep index).  Either pointer may be NULL. */
tpconv_status tpconv_plan_path(tpconv_plan plan, int32_t path, int32_t* l123, int32_t* irrep_idx);

/* The real CG table of a path as fp64, row-major [2l1+1][2l2+1][2l3+1]
 * (host memory, caller-owned).  These are the values the kernels use (rounded
 * to fp32 there). */
tpconv_status tpconv_plan_cg(tpconv_plan plan, int32_t path, double* out);

/* Bytes of caller-provided device workspace an operation needs for N nodes and
 * E edges.  For FORWARD, BACKWARD and DOUBLE_BACKWARD the size does not depend
 * on E (bounded receiver state, O(N)); GRAPH_PREPARE needs O(E) int32 scratch
 * for the sender sort.  FORWARD's figure assumes saved_state == NULL (0 is
 * returned for the in-place-state case via tpconv_state_size). */
tpconv_status tpconv_workspace_size(tpconv_plan plan, int32_t op, int64_t num_nodes,
                                    int64_t num_edges, size_t* bytes);

/* Bytes of the per-receiver state S (K * C_in * sum_p(2l3+1) fp32 per node)
 * that tpconv_forward can save for tpconv_backward. */
tpconv_status tpconv_state_size(tpconv_plan plan, int64_t num_nodes, size_t* bytes);

/* Build the sender-sorted view of the receiver-sorted graph (stable: for each
 * sender, receivers in increasing edge order).  g->rowptr, g->senders are read;
 * csc_colptr [N+1] and csc_receivers [E] are written (device).  With
 * validate != 0 the CSR is first checked on the device (rowptr[0] = 0,
 * non-decreasing, rowptr[N] = E, 0 <= sender < N); this synchronises the
 * stream and returns TPCONV_ERROR_GRAPH without writing the outputs when the
 * check fails.  Workspace: tpconv_workspace_size(GRAPH_PREPARE). */
tpconv_status tpconv_graph_prepare(tpconv_plan plan, const tpconv_graph* g, int32_t* csc_colptr,
                                   int32_t* csc_receivers, int32_t validate, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Forward: out = conv(pos, x, W) as defined at the top of this header.
 * saved_state: NULL, or device memory of tpconv_state_size bytes that receives
 * the receiver state S for a later tpconv_backward (then the workspace may be
 * NULL/0).  Device pointers: pos, x, W, out (and saved_state). */
tpconv_status tpconv_forward(tpconv_plan plan, const tpconv_graph* g, const float* pos,
                             const void* x, const void* W, float* out, float* saved_state,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Backward of <grad_out, out>: grad_x [N][rows_in][C_in], grad_W [K][P][C_in][C_out],
 * grad_pos [N][3]; each may be NULL to skip it (at least one must be given).
 * saved_state: S from tpconv_forward with the same inputs, or NULL to recompute it.
 * Needs g->csc_colptr / csc_receivers when grad_x is requested.  grad_pos sums
 * per-edge contributions with fp32 atomics, so its last bits may vary between
 * runs; grad_x and grad_W are deterministic. */
tpconv_status tpconv_backward(tpconv_plan plan, const tpconv_graph* g, const float* pos,
                              const void* x, const void* W, const float* grad_out,
                              const float* saved_state, float* grad_x, float* grad_W,
                              float* grad_pos, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Double backward of the scalar force loss L = sum_n <gg_pos[n], grad_pos[n]>,
 * where grad_pos is the backward above for the given grad_out:
 *   d_W = dL/dW, d_x = dL/dx, d_grad_out = dL/dgrad_out (each may be NULL).
 * With phi_e = gg_pos[s] - gg_pos[v], L is the derivative of the edge
 * energies along phi, so it is linear in W, x and grad_out; dL/dpos (the
 * Hessian term) is not computed.  Needs the CSC view when d_x is requested. */
tpconv_status tpconv_double_backward(tpconv_plan plan, const tpconv_graph* g, const float* pos,
                                     const void* x, const void* W, const float* grad_out,
                                     const float* gg_pos, float* d_W, float* d_x,
                                     float* d_grad_out, void* workspace, size_t workspace_bytes,
                                     void* stream);

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
  TPCONV_KERNEL_GW_REDUCE = 9,     /* ordered sum of the grad_W partials */
  TPCONV_KERNEL_FILL = 10,         /* zero fills */
  TPCONV_KERNEL_GRAPH = 11,        /* sender-sorted view construction */
  TPCONV_KERNEL_CW_CONTRACT = 12,  /* channel-wise: out, grad_x, d_grad_out, d_x from S / T */
  TPCONV_KERNEL_CW_GW = 13,        /* channel-wise: grad_W partials (also d_W) */
  TPCONV_KERNEL_CW_REDUCE = 14,    /* channel-wise: ordered sum of the partials */
  TPCONV_KERNEL_COUNT = 15
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
