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
OP_FORWARD, OP_BACKWARD, OP_DOUBLE_BACKWARD, OP_GRAPH_PREPARE = 0, 1, 2, 3
STATUS = {0: "SUCCESS", 1: "INVALID_VALUE", 2: "IRREPS", 3: "GRAPH", 4: "WORKSPACE", 5: "UNSUPPORTED",
          6: "DEVICE"}

EXPORTS = ("tpconv_plan_create", "tpconv_plan_destroy", "tpconv_plan_info", "tpconv_plan_path",
           "tpconv_plan_cg", "tpconv_workspace_size", "tpconv_state_size", "tpconv_graph_prepare",
           "tpconv_forward", "tpconv_backward", "tpconv_double_backward", "tpconv_status_string",
           "tpconv_kernel_timing", "tpconv_kernel_timing_read")
KERNELS = ("stream_fwd", "stream_jvp", "stream_snd", "stream_sndt", "stream_bwdpos", "gemm_out", "gemm_gs",
           "gemm_gx", "gemm_gw", "gw_reduce", "fill", "graph", "cw_contract", "cw_gw", "cw_reduce")


class TpconvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: TPCONV_ERROR_{STATUS.get(status, status)} ({_lib().tpconv_status_string(status).decode()})")


class TpconvDesc(ctypes.Structure):
    _fields_ = [("irreps_in", c_char_p), ("irreps_out", c_char_p), ("sh_lmax", c_int32), ("num_basis", c_int32),
                ("cutoff", c_float), ("envelope_p", c_int32), ("x_dtype", c_int32), ("w_dtype", c_int32),
                ("connection", c_int32)]


class TpconvGraph(ctypes.Structure):
    _fields_ = [("num_nodes", c_int64), ("num_edges", c_int64), ("rowptr", c_void_p), ("senders", c_void_p),
                ("csc_colptr", c_void_p), ("csc_receivers", c_void_p)]


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
        L.tpconv_plan_cg.argtypes = [P, c_int32, POINTER(c_double)]
        L.tpconv_workspace_size.argtypes = [P, c_int32, c_int64, c_int64, POINTER(c_size_t)]
        L.tpconv_state_size.argtypes = [P, c_int64, POINTER(c_size_t)]
        L.tpconv_graph_prepare.argtypes = [P, POINTER(TpconvGraph), P, P, c_int32, P, c_size_t, P]
        L.tpconv_forward.argtypes = [P, POINTER(TpconvGraph), P, P, P, P, P, P, c_size_t, P]
        L.tpconv_backward.argtypes = [P, POINTER(TpconvGraph), P, P, P, P, P, P, P, P, P, c_size_t, P]
        L.tpconv_double_backward.argtypes = [P, POINTER(TpconvGraph), P, P, P, P, P, P, P, P, P, c_size_t, P]
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
                 connection: int = FULLY_CONNECTED):
        self._keep = (irreps_in.encode(), irreps_out.encode())
        desc = TpconvDesc(self._keep[0], self._keep[1], sh_lmax, num_basis, cutoff, envelope_p, x_dtype, w_dtype,
                          connection)
        self.connection = connection
        h = c_void_p()
        _check(_lib().tpconv_plan_create(ctypes.byref(h), ctypes.byref(desc)), "tpconv_plan_create")
        self.handle = h
        self.x_dtype, self.w_dtype = x_dtype, w_dtype
        P, wn, ri, ci, ro, co = c_int32(), c_int64(), c_int32(), c_int32(), c_int32(), c_int32()
        _check(_lib().tpconv_plan_info(h, *(ctypes.byref(v) for v in (P, wn, ri, ci, ro, co))), "tpconv_plan_info")
        self.num_paths, self.w_numel = P.value, wn.value
        self.rows_in, self.ch_in, self.rows_out, self.ch_out = ri.value, ci.value, ro.value, co.value
        self.num_basis = num_basis

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
        if self.connection == CHANNELWISE:
            return (self.num_basis, self.num_paths, self.ch_in)
        return (self.num_basis, self.num_paths, self.ch_in, self.ch_out)


class Graph:
    """Receiver-sorted CSR (device int32 tensors) plus the sender-sorted view."""

    def __init__(self, rowptr, senders, csc_colptr=None, csc_receivers=None):
        self.rowptr, self.senders = rowptr, senders
        self.csc_colptr, self.csc_receivers = csc_colptr, csc_receivers
        self.num_nodes = rowptr.numel() - 1
        self.num_edges = senders.numel()

    def c(self) -> TpconvGraph:
        return TpconvGraph(self.num_nodes, self.num_edges, _ptr(self.rowptr), _ptr(self.senders),
                           _ptr(self.csc_colptr), _ptr(self.csc_receivers))


def _workspace(nbytes, device):
    import torch

    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def tpconv_graph_prepare(plan: Plan, graph: Graph, validate: bool = True, stream=None) -> Graph:
    import torch

    dev = graph.rowptr.device
    colptr = torch.empty(graph.num_nodes + 1, dtype=torch.int32, device=dev)
    recv = torch.empty(max(graph.num_edges, 1), dtype=torch.int32, device=dev)
    ws = _workspace(plan.workspace_size(OP_GRAPH_PREPARE, graph.num_nodes, graph.num_edges), dev)
    g = graph.c()
    _check(_lib().tpconv_graph_prepare(plan.handle, ctypes.byref(g), _ptr(colptr), _ptr(recv), int(validate),
                                       _ptr(ws), ws.numel(), _stream(stream)), "tpconv_graph_prepare")
    return Graph(graph.rowptr, graph.senders, colptr, recv)


def tpconv_forward(plan: Plan, graph: Graph, pos, x, W, out=None, saved_state=None, workspace=None, stream=None):
    import torch

    dev = pos.device
    if out is None:
        out = torch.empty((graph.num_nodes, plan.rows_out, plan.ch_out), dtype=torch.float32, device=dev)
    if workspace is None and saved_state is None:
        workspace = _workspace(plan.workspace_size(OP_FORWARD, graph.num_nodes, graph.num_edges), dev)
    g = graph.c()
    nbytes = 0 if workspace is None else workspace.numel()
    _check(_lib().tpconv_forward(plan.handle, ctypes.byref(g), _ptr(pos), _ptr(x), _ptr(W), _ptr(out),
                                 _ptr(saved_state), _ptr(workspace), nbytes, _stream(stream)), "tpconv_forward")
    return out


def tpconv_backward(plan: Plan, graph: Graph, pos, x, W, grad_out, saved_state=None, want=("x", "W", "pos"),
                    workspace=None, stream=None, grad_x=None, grad_W=None, grad_pos=None):
    import torch

    dev = pos.device
    N = graph.num_nodes
    if grad_x is None and "x" in want:
        grad_x = torch.empty((N, plan.rows_in, plan.ch_in), dtype=torch.float32, device=dev)
    if grad_W is None and "W" in want:
        grad_W = torch.empty(plan.w_shape, dtype=torch.float32, device=dev)
    if grad_pos is None and "pos" in want:
        grad_pos = torch.empty((N, 3), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = _workspace(plan.workspace_size(OP_BACKWARD, N, graph.num_edges), dev)
    g = graph.c()
    _check(_lib().tpconv_backward(plan.handle, ctypes.byref(g), _ptr(pos), _ptr(x), _ptr(W), _ptr(grad_out),
                                  _ptr(saved_state), _ptr(grad_x), _ptr(grad_W), _ptr(grad_pos), _ptr(workspace),
                                  workspace.numel(), _stream(stream)), "tpconv_backward")
    return grad_x, grad_W, grad_pos


def tpconv_double_backward(plan: Plan, graph: Graph, pos, x, W, grad_out, gg_pos, want=("W", "x", "grad_out"),
                           workspace=None, stream=None, d_W=None, d_x=None, d_grad_out=None):
    import torch

    dev = pos.device
    N = graph.num_nodes
    if d_W is None and "W" in want:
        d_W = torch.empty(plan.w_shape, dtype=torch.float32, device=dev)
    if d_x is None and "x" in want:
        d_x = torch.empty((N, plan.rows_in, plan.ch_in), dtype=torch.float32, device=dev)
    if d_grad_out is None and "grad_out" in want:
        d_grad_out = torch.empty((N, plan.rows_out, plan.ch_out), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = _workspace(plan.workspace_size(OP_DOUBLE_BACKWARD, N, graph.num_edges), dev)
    g = graph.c()
    _check(_lib().tpconv_double_backward(plan.handle, ctypes.byref(g), _ptr(pos), _ptr(x), _ptr(W),
                                         _ptr(grad_out), _ptr(gg_pos), _ptr(d_W), _ptr(d_x), _ptr(d_grad_out),
                                         _ptr(workspace), workspace.numel(), _stream(stream)),
           "tpconv_double_backward")
    return d_W, d_x, d_grad_out


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
