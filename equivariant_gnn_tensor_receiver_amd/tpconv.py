"""Thin Python binding over libtpconv.so (the C ABI in include/tpconv.h).

Argument marshalling only: every step of the convolution runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and the current HIP
stream; tensors are passed as raw pointers.  The library is loaded from this
package directory on first use; if it is missing, every call raises.

Functions carry the C names (``tpconv_plan_create``, ``tpconv_forward``, ...).
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_void_p

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpconv.so")

TPCONV_F32, TPCONV_BF16 = 0, 1
FULLY_CONNECTED, CHANNELWISE = 0, 1  # tpconv_connection
OP_FORWARD, OP_BACKWARD, OP_DOUBLE_BACKWARD, OP_GRAPH_PREPARE, OP_GRAPH_ORDER, OP_FORWARD_SAVED = 0, 1, 2, 3, 4, 5
STATUS = {0: "SUCCESS", 1: "INVALID_VALUE", 2: "IRREPS", 3: "GRAPH", 4: "WORKSPACE", 5: "UNSUPPORTED",
          6: "DEVICE", 7: "SCRATCH"}
STATIC_SCRATCH_BYTES = 64 << 20

EXPORTS = ("tpconv_plan_create", "tpconv_plan_destroy", "tpconv_plan_info", "tpconv_plan_path",
           "tpconv_plan_cg", "tpconv_workspace_size", "tpconv_state_size", "tpconv_graph_prepare",
           "tpconv_forward", "tpconv_backward", "tpconv_double_backward", "tpconv_status_string",
           "tpconv_kernel_timing", "tpconv_kernel_timing_read", "tpconv_forward_static", "tpconv_graph_order",
           "tpconv_plan_features", "tpconv_forward_mlp", "tpconv_backward_mlp", "tpconv_double_backward_mlp")
KERNELS = ("stream_fwd", "stream_jvp", "stream_snd", "stream_sndt", "stream_bwdpos", "gemm_out", "gemm_gs",
           "gemm_gx", "gemm_gw", "gw_reduce", "fill", "graph", "cw_contract", "cw_gw", "cw_reduce", "stream_hess",
           "state_dot")


class TpconvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: TPCONV_ERROR_{STATUS.get(status, status)} ({_lib().tpconv_status_string(status).decode()})")


class TpconvDesc(ctypes.Structure):
    _fields_ = [("irreps_in", c_char_p), ("irreps_out", c_char_p), ("sh_lmax", c_int32), ("num_basis", c_int32),
                ("cutoff", c_float), ("envelope_p", c_int32), ("x_dtype", c_int32), ("w_dtype", c_int32),
                ("connection", c_int32), ("radial_mlp", c_int32), ("deterministic", c_int32)]


class TpconvGraph(ctypes.Structure):
    _fields_ = [("num_nodes", c_int64), ("num_edges", c_int64), ("rowptr", c_void_p), ("senders", c_void_p),
                ("csc_colptr", c_void_p), ("csc_receivers", c_void_p), ("node_order", c_void_p)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = c_void_p
        L.tpconv_plan_create.argtypes = [POINTER(c_void_p), POINTER(TpconvDesc)]
        L.tpconv_plan_destroy.argtypes = [P]
        L.tpconv_plan_info.argtypes = [P, POINTER(c_int32), POINTER(c_int64), POINTER(c_int32), POINTER(c_int32),
                                       POINTER(c_int32), POINTER(c_int32)]
        L.tpconv_plan_path.argtypes = [P, c_int32, POINTER(c_int32), POINTER(c_int32)]
        L.tpconv_plan_features.argtypes = [P, POINTER(c_int64), POINTER(c_int64)]
        L.tpconv_plan_cg.argtypes = [P, c_int32, POINTER(c_double)]
        L.tpconv_workspace_size.argtypes = [P, c_int32, c_int64, c_int64, POINTER(c_size_t)]
        L.tpconv_state_size.argtypes = [P, c_int64, POINTER(c_size_t)]
        L.tpconv_graph_prepare.argtypes = [P, POINTER(TpconvGraph), P, P, c_int32, P, c_size_t, P]
        L.tpconv_graph_order.argtypes = [P, POINTER(TpconvGraph), P, P, P, c_size_t, P]
        L.tpconv_forward.argtypes = [P, POINTER(TpconvGraph), P, P, P, P, P, P, c_size_t, P]
        L.tpconv_forward_static.argtypes = [P, POINTER(TpconvGraph), P, P, P, P, P]
        L.tpconv_backward.argtypes = [P, POINTER(TpconvGraph), P, P, P, P, P, P, P, P, P, c_size_t, P]
        L.tpconv_double_backward.argtypes = [P, POINTER(TpconvGraph), P, P, P, P, P, P, P, P, P, P, c_size_t, P]
        L.tpconv_forward_mlp.argtypes = [P, POINTER(TpconvGraph), P, P, P, P, P, P, P, c_size_t, P]
        L.tpconv_backward_mlp.argtypes = [P, POINTER(TpconvGraph), P, P, P, P, P, P, P, P, P, P, P, c_size_t, P]
        L.tpconv_double_backward_mlp.argtypes = [P, POINTER(TpconvGraph), P, P, P, P, P, P, P, P, P, P, P, P,
                                                 c_size_t, P]
        L.tpconv_kernel_timing.argtypes = [c_int32]
        L.tpconv_kernel_timing_read.argtypes = [c_int32, POINTER(c_int64), POINTER(c_double)]
        L.tpconv_status_string.argtypes = [c_int32]
        L.tpconv_status_string.restype = c_char_p
        for name in EXPORTS:
            if name != "tpconv_status_string":
                getattr(L, name).restype = c_int32
        _LIB = L
    return _LIB


def _check(st: int, where: str):
    if st != 0:
        raise TpconvError(st, where)


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return c_void_p(s.cuda_stream)


class Plan:
    """Owning handle of a tpconv_plan (host-side tables; no device memory)."""

    def __init__(self, irreps_in: str, irreps_out: str, sh_lmax: int, num_basis: int, cutoff: float = 5.0,
                 envelope_p: int = 6, x_dtype: int = TPCONV_F32, w_dtype: int = TPCONV_F32,
                 connection: int = FULLY_CONNECTED, radial_mlp: bool = False, deterministic: bool = False):
        self._keep = (irreps_in.encode(), irreps_out.encode())
        desc = TpconvDesc(self._keep[0], self._keep[1], sh_lmax, num_basis, cutoff, envelope_p, x_dtype, w_dtype,
                          connection, int(radial_mlp), int(deterministic))
        self.connection = connection
        self.radial_mlp = bool(radial_mlp)
        h = c_void_p()
        _check(_lib().tpconv_plan_create(ctypes.byref(h), ctypes.byref(desc)), "tpconv_plan_create")
        self.handle = h
        self.x_dtype, self.w_dtype = x_dtype, w_dtype
        P, wn, ri, ci, ro, co = c_int32(), c_int64(), c_int32(), c_int32(), c_int32(), c_int32()
        _check(_lib().tpconv_plan_info(h, *(ctypes.byref(v) for v in (P, wn, ri, ci, ro, co))), "tpconv_plan_info")
        self.num_paths, self.w_numel = P.value, wn.value
        self.rows_in, self.ch_in, self.rows_out, self.ch_out = ri.value, ci.value, ro.value, co.value
        self.num_basis = num_basis
        fi, fo = c_int64(), c_int64()
        _check(_lib().tpconv_plan_features(h, ctypes.byref(fi), ctypes.byref(fo)), "tpconv_plan_features")
        self.feat_in, self.feat_out = fi.value, fo.value
        self.ragged = self.ch_in == 0 or self.ch_out == 0

    def in_shape(self, N):
        """Shape of x, grad_x, d_x: [N][rows][C], or [N][F] for ragged multiplicities."""
        return (N, self.feat_in) if self.ragged else (N, self.rows_in, self.ch_in)

    def out_shape(self, N):
        return (N, self.feat_out) if self.ragged else (N, self.rows_out, self.ch_out)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _LIB is not None:
            _LIB.tpconv_plan_destroy(h)
            self.handle = None

    def path(self, i: int):
        l123 = (c_int32 * 3)()
        idx = (c_int32 * 2)()
        _check(_lib().tpconv_plan_path(self.handle, i, l123, idx), "tpconv_plan_path")
        return tuple(l123), tuple(idx)

    def cg(self, i: int) -> np.ndarray:
        (l1, l2, l3), _ = self.path(i)
        out = np.zeros((2 * l1 + 1) * (2 * l2 + 1) * (2 * l3 + 1), dtype=np.float64)
        _check(_lib().tpconv_plan_cg(self.handle, i, out.ctypes.data_as(POINTER(c_double))), "tpconv_plan_cg")
        return out.reshape(2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1)

    def workspace_size(self, op: int, num_nodes: int, num_edges: int) -> int:
        b = c_size_t()
        _check(_lib().tpconv_workspace_size(self.handle, op, num_nodes, num_edges, ctypes.byref(b)),
               "tpconv_workspace_size")
        return b.value

    def state_size(self, num_nodes: int) -> int:
        b = c_size_t()
        _check(_lib().tpconv_state_size(self.handle, num_nodes, ctypes.byref(b)), "tpconv_state_size")
        return b.value

    @property
    def w_shape(self):
        if self.ragged:
            return (self.num_basis, self.w_numel // self.num_basis)
        if self.connection == CHANNELWISE:
            return (self.num_basis, self.num_paths, self.ch_in)
        return (self.num_basis, self.num_paths, self.ch_in, self.ch_out)


class Graph:
    """Receiver-sorted CSR (device int32 tensors), the sender-sorted view and
    an optional visiting order of the nodes."""

    def __init__(self, rowptr, senders, csc_colptr=None, csc_receivers=None, node_order=None):
        self.rowptr, self.senders = rowptr, senders
        self.csc_colptr, self.csc_receivers = csc_colptr, csc_receivers
        self.node_order = node_order
        self.num_nodes = rowptr.numel() - 1
        self.num_edges = senders.numel()

    def c(self) -> TpconvGraph:
        return TpconvGraph(self.num_nodes, self.num_edges, _ptr(self.rowptr), _ptr(self.senders),
                           _ptr(self.csc_colptr), _ptr(self.csc_receivers), _ptr(self.node_order))

    def _with(self, **kw):
        g = Graph(self.rowptr, self.senders, self.csc_colptr, self.csc_receivers, self.node_order)
        g.num_edges = self.num_edges
        for k, v in kw.items():
            setattr(g, k, v)
        return g


def _workspace(nbytes, device):
    import torch

    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _require(t, name, dtype, numel, device, min_bytes=None):
    """Reject a tensor the kernels would misread: wrong dtype, not contiguous,
    too few elements or on another device (None is passed through)."""
    if t is None:
        return
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, at least {min_bytes} needed")


def _feature_dtype(code):
    import torch

    return torch.bfloat16 if code == TPCONV_BF16 else torch.float32


def _check_inputs(plan, graph, pos, x, W, **more):
    """Checks shared by the passes: graph index tensors, pos, x, W, and the
    named fp32 node tensors in `more` (name -> (tensor, values per node))."""
    import torch

    dev = pos.device
    N = graph.num_nodes
    _require(graph.rowptr, "rowptr", torch.int32, N + 1, dev)
    _require(graph.senders, "senders", torch.int32, None, dev)
    if graph.senders.numel() < graph.num_edges:
        raise ValueError("senders: fewer entries than num_edges")
    _require(pos, "pos", torch.float32, 3 * N, dev)
    _require(x, "x", _feature_dtype(plan.x_dtype), N * plan.feat_in, dev)
    _require(W, "W", _feature_dtype(plan.w_dtype), plan.w_numel, dev)
    for name, (t, per_node) in more.items():
        _require(t, name, torch.float32, N * per_node, dev)


def _keep_for_stream(stream, *tensors):
    """Tensors allocated here but used on a stream other than the current one
    must not be reused by the caching allocator before that stream is done."""
    import torch

    if stream is None or stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def tpconv_graph_prepare(plan: Plan, graph: Graph, validate: bool = True, stream=None) -> Graph:
    import torch

    dev = graph.rowptr.device
    _require(graph.rowptr, "rowptr", torch.int32, graph.num_nodes + 1, dev)
    _require(graph.senders, "senders", torch.int32, None, dev)
    if graph.senders.numel() < graph.num_edges:
        raise ValueError("senders: fewer entries than num_edges")
    colptr = torch.empty(graph.num_nodes + 1, dtype=torch.int32, device=dev)
    recv = torch.empty(max(graph.num_edges, 1), dtype=torch.int32, device=dev)
    ws = _workspace(plan.workspace_size(OP_GRAPH_PREPARE, graph.num_nodes, graph.num_edges), dev)
    _keep_for_stream(stream, colptr, recv, ws)
    g = graph.c()
    _check(_lib().tpconv_graph_prepare(plan.handle, ctypes.byref(g), _ptr(colptr), _ptr(recv), int(validate),
                                       _ptr(ws), ws.numel(), _stream(stream)), "tpconv_graph_prepare")
    return graph._with(csc_colptr=colptr, csc_receivers=recv)


def tpconv_graph_order(plan: Plan, graph: Graph, pos, stream=None) -> Graph:
    """The graph with node_order set to the Morton order of `pos`."""
    import torch

    dev = pos.device
    _require(pos, "pos", torch.float32, 3 * graph.num_nodes, dev)
    order = torch.empty(max(graph.num_nodes, 1), dtype=torch.int32, device=dev)
    ws = _workspace(plan.workspace_size(OP_GRAPH_ORDER, graph.num_nodes, graph.num_edges), dev)
    _keep_for_stream(stream, order, ws)
    g = graph.c()
    _check(_lib().tpconv_graph_order(plan.handle, ctypes.byref(g), _ptr(pos), _ptr(order), _ptr(ws), ws.numel(),
                                     _stream(stream)), "tpconv_graph_order")
    return graph._with(node_order=order)


def _check_radial(plan, radial_w, dev):
    import torch

    if plan.radial_mlp != (radial_w is not None):
        raise ValueError("radial_w must be given exactly for plans created with radial_mlp=True")
    _require(radial_w, "radial_w", torch.float32, plan.num_basis ** 2, dev)


def tpconv_forward(plan: Plan, graph: Graph, pos, x, W, out=None, saved_state=None, workspace=None, stream=None,
                   radial_w=None):
    """radial_w: the [K][K] weights of the radial MLP for plans created with radial_mlp=True."""
    import torch

    dev = pos.device
    N = graph.num_nodes
    if out is None:
        out = torch.empty(plan.out_shape(N), dtype=torch.float32, device=dev)
        _keep_for_stream(stream, out)
    _check_inputs(plan, graph, pos, x, W, out=(out, plan.feat_out))
    _check_radial(plan, radial_w, dev)
    _require(saved_state, "saved_state", torch.float32, plan.state_size(N) // 4, dev)
    if workspace is None:
        need = plan.workspace_size(OP_FORWARD if saved_state is None else OP_FORWARD_SAVED, N, graph.num_edges)
        if need > 0:
            workspace = _workspace(need, dev)
            _keep_for_stream(stream, workspace)
    _require(workspace, "workspace", None, None, dev)
    g = graph.c()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if plan.radial_mlp:
        _check(_lib().tpconv_forward_mlp(plan.handle, ctypes.byref(g), _ptr(pos), _ptr(x), _ptr(W), _ptr(radial_w),
                                         _ptr(out), _ptr(saved_state), _ptr(workspace), nbytes, _stream(stream)),
               "tpconv_forward_mlp")
    else:
        _check(_lib().tpconv_forward(plan.handle, ctypes.byref(g), _ptr(pos), _ptr(x), _ptr(W), _ptr(out),
                                     _ptr(saved_state), _ptr(workspace), nbytes, _stream(stream)), "tpconv_forward")
    return out


def tpconv_forward_static(plan: Plan, graph: Graph, pos, x, W, out, stream=None):
    """tpconv_forward with the receiver state in the library's static device
    scratch: no workspace, nothing allocated (`out` must be given)."""
    _check_inputs(plan, graph, pos, x, W, out=(out, plan.feat_out))
    g = graph.c()
    _check(_lib().tpconv_forward_static(plan.handle, ctypes.byref(g), _ptr(pos), _ptr(x), _ptr(W), _ptr(out),
                                        _stream(stream)), "tpconv_forward_static")
    return out


def tpconv_backward(plan: Plan, graph: Graph, pos, x, W, grad_out, saved_state=None, want=("x", "W", "pos"),
                    workspace=None, stream=None, grad_x=None, grad_W=None, grad_pos=None, radial_w=None,
                    grad_radial_w=None):
    """(grad_x, grad_W, grad_pos) for the names in `want`; with the radial MLP
    (radial_w given) also grad_radial_w, requested as "radial_w"."""
    import torch

    dev = pos.device
    N = graph.num_nodes
    if grad_x is None and "x" in want:
        grad_x = torch.empty(plan.in_shape(N), dtype=torch.float32, device=dev)
    if grad_W is None and "W" in want:
        grad_W = torch.empty(plan.w_shape, dtype=torch.float32, device=dev)
    if grad_pos is None and "pos" in want:
        grad_pos = torch.empty((N, 3), dtype=torch.float32, device=dev)
    K = plan.num_basis
    if grad_radial_w is None and "radial_w" in want and plan.radial_mlp:
        grad_radial_w = torch.empty((K, K), dtype=torch.float32, device=dev)
    _keep_for_stream(stream, grad_x, grad_W, grad_pos, grad_radial_w)
    _check_inputs(plan, graph, pos, x, W, grad_out=(grad_out, plan.feat_out), grad_x=(grad_x, plan.feat_in),
                  grad_pos=(grad_pos, 3))
    _check_radial(plan, radial_w, dev)
    _require(grad_W, "grad_W", torch.float32, plan.w_numel, dev)
    _require(grad_radial_w, "grad_radial_w", torch.float32, K * K, dev)
    _require(saved_state, "saved_state", torch.float32, plan.state_size(N) // 4, dev)
    if workspace is None:
        workspace = _workspace(plan.workspace_size(OP_BACKWARD, N, graph.num_edges), dev)
        _keep_for_stream(stream, workspace)
    _require(workspace, "workspace", None, None, dev)
    g = graph.c()
    nbytes = workspace.numel() * workspace.element_size()
    if plan.radial_mlp:
        _check(_lib().tpconv_backward_mlp(plan.handle, ctypes.byref(g), _ptr(pos), _ptr(x), _ptr(W), _ptr(radial_w),
                                          _ptr(grad_out), _ptr(saved_state), _ptr(grad_x), _ptr(grad_W),
                                          _ptr(grad_pos), _ptr(grad_radial_w), _ptr(workspace), nbytes,
                                          _stream(stream)), "tpconv_backward_mlp")
        return grad_x, grad_W, grad_pos, grad_radial_w
    _check(_lib().tpconv_backward(plan.handle, ctypes.byref(g), _ptr(pos), _ptr(x), _ptr(W), _ptr(grad_out),
                                  _ptr(saved_state), _ptr(grad_x), _ptr(grad_W), _ptr(grad_pos), _ptr(workspace),
                                  nbytes, _stream(stream)), "tpconv_backward")
    return grad_x, grad_W, grad_pos


def tpconv_double_backward(plan: Plan, graph: Graph, pos, x, W, grad_out, gg_pos, want=("W", "x", "grad_out", "pos"),
                           workspace=None, stream=None, d_W=None, d_x=None, d_grad_out=None, d_pos=None,
                           radial_w=None, d_radial_w=None):
    """Gradients of sum_n <gg_pos[n], grad_pos[n]>: (d_W, d_x, d_grad_out, d_pos) for the names in
    `want` ("W", "x", "grad_out", "pos"); the others are None.  With the radial
    MLP (radial_w given) also d_radial_w, requested as "radial_w"."""
    import torch

    dev = pos.device
    N = graph.num_nodes
    if d_W is None and "W" in want:
        d_W = torch.empty(plan.w_shape, dtype=torch.float32, device=dev)
    if d_x is None and "x" in want:
        d_x = torch.empty(plan.in_shape(N), dtype=torch.float32, device=dev)
    if d_grad_out is None and "grad_out" in want:
        d_grad_out = torch.empty(plan.out_shape(N), dtype=torch.float32, device=dev)
    if d_pos is None and "pos" in want:
        d_pos = torch.empty((N, 3), dtype=torch.float32, device=dev)
    K = plan.num_basis
    if d_radial_w is None and "radial_w" in want and plan.radial_mlp:
        d_radial_w = torch.empty((K, K), dtype=torch.float32, device=dev)
    _keep_for_stream(stream, d_W, d_x, d_grad_out, d_pos, d_radial_w)
    _check_inputs(plan, graph, pos, x, W, grad_out=(grad_out, plan.feat_out), gg_pos=(gg_pos, 3),
                  d_x=(d_x, plan.feat_in), d_grad_out=(d_grad_out, plan.feat_out), d_pos=(d_pos, 3))
    _check_radial(plan, radial_w, dev)
    _require(d_W, "d_W", torch.float32, plan.w_numel, dev)
    _require(d_radial_w, "d_radial_w", torch.float32, K * K, dev)
    if workspace is None:
        workspace = _workspace(plan.workspace_size(OP_DOUBLE_BACKWARD, N, graph.num_edges), dev)
        _keep_for_stream(stream, workspace)
    _require(workspace, "workspace", None, None, dev)
    g = graph.c()
    nbytes = workspace.numel() * workspace.element_size()
    if plan.radial_mlp:
        _check(_lib().tpconv_double_backward_mlp(plan.handle, ctypes.byref(g), _ptr(pos), _ptr(x), _ptr(W),
                                                 _ptr(radial_w), _ptr(grad_out), _ptr(gg_pos), _ptr(d_W), _ptr(d_x),
                                                 _ptr(d_grad_out), _ptr(d_pos), _ptr(d_radial_w), _ptr(workspace),
                                                 nbytes, _stream(stream)), "tpconv_double_backward_mlp")
        return d_W, d_x, d_grad_out, d_pos, d_radial_w
    _check(_lib().tpconv_double_backward(plan.handle, ctypes.byref(g), _ptr(pos), _ptr(x), _ptr(W),
                                         _ptr(grad_out), _ptr(gg_pos), _ptr(d_W), _ptr(d_x), _ptr(d_grad_out),
                                         _ptr(d_pos), _ptr(workspace), nbytes, _stream(stream)),
           "tpconv_double_backward")
    return d_W, d_x, d_grad_out, d_pos


def tpconv_kernel_timing(enable: bool):
    _check(_lib().tpconv_kernel_timing(int(enable)), "tpconv_kernel_timing")


def tpconv_kernel_timing_read():
    """{kernel name: (launches, total ms)} for every class with at least one launch."""
    out = {}
    for i, name in enumerate(KERNELS):
        n, ms = c_int64(), c_double()
        _check(_lib().tpconv_kernel_timing_read(i, ctypes.byref(n), ctypes.byref(ms)), "tpconv_kernel_timing_read")
        if n.value:
            out[name] = (n.value, ms.value)
    return out


def to_device_bf16(a: np.ndarray, device):
    """Upload fp32 values that are exact in bf16 as a torch.bfloat16 tensor."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device).to(torch.bfloat16)
