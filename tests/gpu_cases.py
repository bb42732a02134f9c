"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and compare with the fp64 oracle on the same seeded inputs.

Tolerances (per tensor, against the oracle's max magnitude):
  forward:   max|gpu - oracle| <= 1e-4 * max|oracle|
  gradients: max|gpu - oracle| <= 1e-3 * max|oracle|   (backward and double backward)
"""
from __future__ import annotations

import sys

import numpy as np

from equivariant_gnn_tensor_receiver_amd import inputs
from equivariant_gnn_tensor_receiver_amd import tpconv as tp
from oracle import tpconv as otp

FWD_TOL = 1e-4
GRAD_TOL = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max() if ref.size else 0.0
    if scale == 0.0:
        return float(np.abs(gpu).max() if gpu.size else 0.0)
    return float(np.abs(gpu - ref).max() / scale)


class DeviceCase:
    """Seeded problem uploaded to cuda:0 plus the matching oracle Problem."""

    def __init__(self, irreps_in, irreps_out, sh_lmax, K, pos, rowptr, senders, rng, dtype="f32",
                 channelwise=False, w_dtype=None, env_p=6, ordered=True, radial_mlp=False, deterministic=False):
        import torch

        self.dev = torch.device("cuda:0")
        w_dtype = dtype if w_dtype is None else w_dtype
        xd = tp.TPCONV_BF16 if dtype == "bf16" else tp.TPCONV_F32
        wd = tp.TPCONV_BF16 if w_dtype == "bf16" else tp.TPCONV_F32
        conn = tp.CHANNELWISE if channelwise else tp.FULLY_CONNECTED
        self.plan = tp.Plan(irreps_in, irreps_out, sh_lmax, K, inputs.CUTOFF, env_p, xd, wd, conn, radial_mlp,
                            deterministic)
        self.prob = otp.Problem(irreps_in, irreps_out, sh_lmax, K, envelope_p=env_p, channelwise=channelwise)
        assert self.plan.num_paths == self.prob.P
        assert tuple(self.plan.w_shape) == tuple(self.prob.w_shape)
        N = len(rowptr) - 1
        if self.prob.uniform:
            t = inputs.make_tensors(rng, N, self.prob.D_in, self.prob.C_in, self.prob.D_out, self.prob.C_out, K,
                                    self.prob.P, dtype, channelwise=channelwise, w_dtype=w_dtype)
        else:  # ragged multiplicities: the flat per-irrep layout
            cmax = max(m for m, _, _ in self.prob.ir_in)
            t = dict(x=rng.standard_normal((N, self.prob.F_in), dtype=np.float32),
                     W=(rng.standard_normal(self.prob.w_shape, dtype=np.float32)
                        * np.float32((1.0 / (K * (1 if channelwise else cmax))) ** 0.5)),
                     g_out=rng.standard_normal((N, self.prob.F_out), dtype=np.float32),
                     gg_pos=rng.standard_normal((N, 3), dtype=np.float32))
            if dtype == "bf16":
                t["x"] = inputs.bf16_round(t["x"])
            if w_dtype == "bf16":
                t["W"] = inputs.bf16_round(t["W"])
        # weights of the radial MLP, from a generator of their own (the other draws stay as they are)
        self.A = (np.random.default_rng(1234 + N).standard_normal((K, K)).astype(np.float32)
                  * np.float32(1.5 / K ** 0.5)) if radial_mlp else None
        self.np = dict(pos=pos, rowptr=rowptr, senders=senders, **t)
        self.receivers = otp.csr_receivers(rowptr)
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(self.dev)
        self.pos = to(pos.astype(np.float32))
        self.rowptr = to(rowptr.astype(np.int32))
        self.senders = to(senders.astype(np.int32)) if len(senders) else torch.zeros(1, dtype=torch.int32,
                                                                                      device=self.dev)
        self.x = tp.to_device_bf16(t["x"], self.dev) if dtype == "bf16" else to(t["x"])
        self.W = tp.to_device_bf16(t["W"], self.dev) if w_dtype == "bf16" else to(t["W"])
        self.g_out = to(t["g_out"])
        self.gg = to(t["gg_pos"])
        self.A_dev = None if self.A is None else to(self.A)
        self.mlp = {} if self.A is None else dict(radial_w=self.A_dev)
        g = tp.Graph(self.rowptr, self.senders)
        g.num_edges = len(senders)
        self.graph = tp.tpconv_graph_prepare(self.plan, g, validate=True)
        if ordered:  # the streams visit nodes in Morton order, as in bench.py
            self.graph = tp.tpconv_graph_order(self.plan, self.graph, self.pos)

    def forward(self, **kw):
        import torch

        out = tp.tpconv_forward(self.plan, self.graph, self.pos, self.x, self.W, **self.mlp, **kw)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def backward(self, g_out=None, **kw):
        import torch

        go = self.g_out if g_out is None else g_out
        if self.A is not None and "want" not in kw:
            kw["want"] = ("x", "W", "pos", "radial_w")
        r = tp.tpconv_backward(self.plan, self.graph, self.pos, self.x, self.W, go, **self.mlp, **kw)
        torch.cuda.synchronize()
        return [None if a is None else a.cpu().numpy() for a in r]

    def double_backward(self, g_out=None, **kw):
        import torch

        go = self.g_out if g_out is None else g_out
        if self.A is not None and "want" not in kw:
            kw["want"] = ("W", "x", "grad_out", "pos", "radial_w")
        r = tp.tpconv_double_backward(self.plan, self.graph, self.pos, self.x, self.W, go, self.gg, **self.mlp, **kw)
        torch.cuda.synchronize()
        return [None if a is None else a.cpu().numpy() for a in r]

    # oracle side
    def o_forward(self, snd=None, rcv=None):
        n = self.np
        snd = n["senders"] if snd is None else snd
        rcv = self.receivers if rcv is None else rcv
        return otp.forward(self.prob, n["pos"], snd, rcv, n["x"], n["W"], num_nodes=len(n["rowptr"]) - 1,
                           radial_w=self.A)

    def o_backward(self, g_out, snd=None, rcv=None):
        n = self.np
        snd = n["senders"] if snd is None else snd
        rcv = self.receivers if rcv is None else rcv
        return otp.backward(self.prob, n["pos"], snd, rcv, n["x"], n["W"], g_out, radial_w=self.A)

    def o_double_backward(self, g_out, snd=None, rcv=None):
        """Oracle (d_W, d_x, d_grad_out, d_pos), and d_A with the radial MLP."""
        n = self.np
        snd = n["senders"] if snd is None else snd
        rcv = self.receivers if rcv is None else rcv
        r = otp.double_backward(self.prob, n["pos"], snd, rcv, n["x"], n["W"], g_out, n["gg_pos"], radial_w=self.A)
        dp = otp.double_backward_pos(self.prob, n["pos"], snd, rcv, n["x"], n["W"], g_out, n["gg_pos"],
                                     radial_w=self.A)
        return tuple(r[:3]) + (dp,) + tuple(r[3:])


def small_case(irreps_in, irreps_out, sh_lmax, K, N, deg, seed, dtype="f32", channelwise=False, w_dtype=None,
               env_p=6):
    pos, rowptr, senders, rng = inputs.random_graph(N, deg, seed)
    return DeviceCase(irreps_in, irreps_out, sh_lmax, K, pos, rowptr, senders, rng, dtype, channelwise, w_dtype,
                      env_p)


def workload_case(name):
    w = inputs.WORKLOADS[name]
    pos, rowptr, senders, _, rng = inputs.make_graph(w)
    return DeviceCase(w.irreps, w.irreps, w.lmax, w.num_basis, pos, rowptr, senders, rng, w.dtype,
                      w.channelwise)
