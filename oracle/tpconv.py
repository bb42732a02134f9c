"""Edge-conditioned CG tensor-product convolution, conventional schedule (fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed ("Sobek" page, abstract: equivariant GNNs apply
edge-conditioned tensor-product convolutions over graph edges; conventional
implementations materialise edge-specific weights, messages and adjoints).  For
every directed edge e = (s -> v) of the receiver-sorted graph:

  r_e = pos[s] - pos[v],  d = |r_e|,  r_hat = r_e / d
  R_e[k]            radial basis (oracle.radial)
  Y_e[l2, m2]       real spherical harmonics of r_hat (oracle.sh)
  w_e[p, ci, co]  = sum_k R_e[k] W[k, p, ci, co]                (per-edge weights)
  U_e[p, ci, m3]  = sum_{m1,m2} C^p[m1,m2,m3] x[s][l1, ci, m1] Y_e[l2, m2]
  m_e[l3, co, m3] = sum_{p -> l3} sum_ci w_e[p, ci, co] U_e[p, ci, m3]   (message)
  out[v]         += m_e                                          (scatter-add)

This module deliberately keeps that order: it materialises w_e, U_e and m_e
for a bounded chunk of edges at a time and scatter-adds with ``np.add.at``.
The backward and double backward are written out by hand from the chain rule
on the same materialised intermediates (adjoints g_w, g_U, g_Y, g_R per edge).

Two connections of the channels are covered.  Fully connected ("uvw"): one
C_in x C_out matrix per (k, path), W[k, p, ci, co].  Channel-wise ("uvu",
C_in = C_out = C): one weight per (k, path, channel), W[k, p, c], so
w_e[p, c] = sum_k R_e[k] W[k, p, c] and m_e[l3, c, m3] = sum_p w_e[p, c]
U_e[p, c, m3] (the Sobek page's abstract names two operator families; this
reading takes the channel-wise product as the second).

Layouts (shared with the library's public header only as a data contract):
  x   [N][D_in][C_in],  out [N][D_out][C_out]   rows ordered by irreps, l^2+l+m
  W   [K][P][C_in][C_out] (uvw) or [K][P][C] (uvu), P paths in oracle.cg order
  pos [N][3]
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import cg as _cg
from . import radial as _radial
from . import sh as _sh


@dataclass
class Problem:
    irreps_in: str
    irreps_out: str
    sh_lmax: int
    num_basis: int
    cutoff: float = 5.0
    envelope_p: int = 6
    channelwise: bool = False
    ir_in: list = field(init=False)
    ir_out: list = field(init=False)
    paths: list = field(init=False)

    def __post_init__(self):
        self.ir_in = _cg.parse_irreps(self.irreps_in)
        self.ir_out = _cg.parse_irreps(self.irreps_out)
        muls_in = {m for m, _, _ in self.ir_in}
        muls_out = {m for m, _, _ in self.ir_out}
        if len(muls_in) != 1 or len(muls_out) != 1:
            raise ValueError("uniform multiplicity per irreps string is required")
        self.C_in = muls_in.pop()
        self.C_out = muls_out.pop()
        if self.channelwise and self.C_in != self.C_out:
            raise ValueError("the channel-wise product needs equal multiplicities")
        self.D_in = _cg.irreps_dim(self.ir_in)
        self.D_out = _cg.irreps_dim(self.ir_out)
        self.off_in = _cg.irreps_offsets(self.ir_in)
        self.off_out = _cg.irreps_offsets(self.ir_out)
        self.paths = _cg.enumerate_paths(self.ir_in, self.sh_lmax, self.ir_out)
        self.P = len(self.paths)
        for p in self.paths:
            p["C"] = _cg.real_cg(p["l1"], p["l2"], p["l3"])

    @property
    def w_shape(self):
        if self.channelwise:
            return (self.num_basis, self.P, self.C_in)
        return (self.num_basis, self.P, self.C_in, self.C_out)

    # einsum forms of the weight contractions.  Index letters: e edge, k basis,
    # p path, i input channel, o output channel, c (in U) the m3 component.
    @property
    def ops(self):
        if self.channelwise:  # w_e[e, p, i]; messages and adjoints keep the channel i
            return dict(w="ek,kpi->epi", msg="ei,eic->eci", g_w="eic,eci->ei", g_U="ei,eci->eic",
                        g_W="ek,epi->kpi", g_R="kpi,epi->ek", dW_a="ek,ei->ki", dW_b="ek,eic,eci->ki")
        return dict(w="ek,kpio->epio", msg="eio,eic->eco", g_w="eic,eco->eio", g_U="eio,eco->eic",
                    g_W="ek,epio->kpio", g_R="kpio,epio->ek", dW_a="ek,eio->kio", dW_b="ek,eic,eco->kio")


def csr_receivers(rowptr: np.ndarray) -> np.ndarray:
    """Receiver id of every edge of a receiver-sorted CSR graph."""
    rowptr = np.asarray(rowptr, dtype=np.int64)
    return np.repeat(np.arange(len(rowptr) - 1), np.diff(rowptr))


def _geometry(pos, s, v):
    r = pos[s] - pos[v]
    d = np.linalg.norm(r, axis=-1)
    rhat = np.where((d > 0)[:, None], r / np.where(d > 0, d, 1.0)[:, None], 0.0)
    return r, d, rhat


def _chunks(prob: Problem, E: int):
    per_edge = 8 * max(1, prob.P * prob.C_in * prob.C_out)
    step = int(max(1, min(E, 48_000_000 // per_edge)))
    for a in range(0, E, step):
        yield a, min(E, a + step)


def _edge_terms(prob, pos, s, v):
    r, d, rhat = _geometry(pos, s, v)
    R = _radial.bessel_radial(d, prob.num_basis, prob.cutoff, prob.envelope_p)
    Y = _sh.spherical_harmonics(prob.sh_lmax, r)
    return r, d, rhat, R, Y


def _x_block(prob, x, s, p):
    o = prob.off_in[p["i1"]]
    return x[s, o:o + 2 * p["l1"] + 1, :]               # [e, m1, ci]


def _y_block(Y, p):
    l2 = p["l2"]
    return Y[:, l2 * l2:(l2 + 1) * (l2 + 1)]            # [e, m2]


def _out_rows(prob, p):
    o = prob.off_out[p["i3"]]
    return slice(o, o + 2 * p["l3"] + 1)


def _in_rows(prob, p):
    o = prob.off_in[p["i1"]]
    return slice(o, o + 2 * p["l1"] + 1)


def _coupling(C, xs, y):
    """U[e, ci, m3] = sum_{m1,m2} C[m1,m2,m3] xs[e,m1,ci] y[e,m2]."""
    return np.einsum("abc,eai,eb->eic", C, xs, y, optimize=True)


def _as64(a):
    return np.asarray(a, dtype=np.float64)


def forward(prob: Problem, pos, senders, receivers, x, W, num_nodes=None):
    """out[v] = sum over edges into v of the materialised message m_e."""
    pos, x, W = _as64(pos), _as64(x), _as64(W)
    senders = np.asarray(senders, dtype=np.int64)
    receivers = np.asarray(receivers, dtype=np.int64)
    N = x.shape[0] if num_nodes is None else num_nodes
    out = np.zeros((N, prob.D_out, prob.C_out))
    for a, b in _chunks(prob, len(senders)):
        s, v = senders[a:b], receivers[a:b]
        _, _, _, R, Y = _edge_terms(prob, pos, s, v)
        ops = prob.ops
        w_e = np.einsum(ops["w"], R, W, optimize=True)              # per-edge weights
        for pi, p in enumerate(prob.paths):
            U = _coupling(p["C"], _x_block(prob, x, s, p), _y_block(Y, p))
            msg = np.einsum(ops["msg"], w_e[:, pi], U, optimize=True)      # message
            np.add.at(out[:, _out_rows(prob, p), :], v, msg)
    return out


def backward(prob: Problem, pos, senders, receivers, x, W, g_out):
    """Materialised adjoints; returns (g_x, g_W, g_pos) for the loss <g_out, out>."""
    pos, x, W, g_out = _as64(pos), _as64(x), _as64(W), _as64(g_out)
    senders = np.asarray(senders, dtype=np.int64)
    receivers = np.asarray(receivers, dtype=np.int64)
    N = x.shape[0]
    K = prob.num_basis
    g_x = np.zeros_like(x)
    g_W = np.zeros_like(W)
    g_pos = np.zeros_like(pos)
    for a, b in _chunks(prob, len(senders)):
        s, v = senders[a:b], receivers[a:b]
        r, d, rhat, R, Y = _edge_terms(prob, pos, s, v)
        dR = _radial.bessel_radial_deriv(d, K, prob.cutoff, prob.envelope_p)
        JY = _sh.sh_jacobian(prob.sh_lmax, r)                     # [e, Dsh, 3]
        ops = prob.ops
        w_e = np.einsum(ops["w"], R, W, optimize=True)
        g_m = g_out[v]                                           # message adjoint
        g_w = np.zeros_like(w_e)
        g_Y = np.zeros_like(Y)
        for pi, p in enumerate(prob.paths):
            C = p["C"]
            xs = _x_block(prob, x, s, p)
            y = _y_block(Y, p)
            U = _coupling(C, xs, y)
            gm = g_m[:, _out_rows(prob, p), :]                     # [e, m3, co]
            g_w[:, pi] = np.einsum(ops["g_w"], U, gm, optimize=True)
            g_U = np.einsum(ops["g_U"], w_e[:, pi], gm, optimize=True)
            gx_e = np.einsum("abc,eb,eic->eai", C, y, g_U, optimize=True)
            np.add.at(g_x[:, _in_rows(prob, p), :], s, gx_e)
            l2 = p["l2"]
            g_Y[:, l2 * l2:(l2 + 1) * (l2 + 1)] += np.einsum(
                "abc,eai,eic->eb", C, xs, g_U, optimize=True)
        g_W += np.einsum(ops["g_W"], R, g_w, optimize=True)
        g_R = np.einsum(ops["g_R"], W, g_w, optimize=True)
        g_r = (np.einsum("ek,ek->e", g_R, dR)[:, None] * rhat
               + np.einsum("em,emj->ej", g_Y, JY))
        np.add.at(g_pos, s, g_r)
        np.add.at(g_pos, v, -g_r)
    return g_x, g_W, g_pos


def double_backward(prob: Problem, pos, senders, receivers, x, W, g_out, gg_pos):
    """Gradients of L_F = sum_n <gg_pos[n], g_pos[n]> w.r.t. W, x and g_out.

    With phi_e = gg_pos[s] - gg_pos[v], L_F = sum_e <phi_e, g_r_e>, the
    derivative of the edge energy <g_m_e, m_e> along phi_e.  The tangents are
    R_dot = R'(d) (r_hat . phi), Y_dot = J_Y phi, U_dot = CG(x_s, Y_dot) and
    w_dot = sum_k R_dot[k] W[k]; L_F is linear in W, x and g_out, so no second
    derivatives of R or Y appear.  d/dpos (the Hessian term) is not computed.
    """
    pos, x, W = _as64(pos), _as64(x), _as64(W)
    g_out, gg_pos = _as64(g_out), _as64(gg_pos)
    senders = np.asarray(senders, dtype=np.int64)
    receivers = np.asarray(receivers, dtype=np.int64)
    K = prob.num_basis
    d_W = np.zeros_like(W)
    d_x = np.zeros_like(x)
    d_gout = np.zeros_like(g_out)
    for a, b in _chunks(prob, len(senders)):
        s, v = senders[a:b], receivers[a:b]
        r, d, rhat, R, Y = _edge_terms(prob, pos, s, v)
        dR = _radial.bessel_radial_deriv(d, K, prob.cutoff, prob.envelope_p)
        JY = _sh.sh_jacobian(prob.sh_lmax, r)
        phi = gg_pos[s] - gg_pos[v]
        R_dot = dR * np.einsum("ej,ej->e", rhat, phi)[:, None]
        Y_dot = np.einsum("emj,ej->em", JY, phi)
        ops = prob.ops
        w_e = np.einsum(ops["w"], R, W, optimize=True)
        w_dot = np.einsum(ops["w"], R_dot, W, optimize=True)
        g_m = g_out[v]
        for pi, p in enumerate(prob.paths):
            C = p["C"]
            xs = _x_block(prob, x, s, p)
            y = _y_block(Y, p)
            y_dot = _y_block(Y_dot, p)
            U = _coupling(C, xs, y)
            U_dot = _coupling(C, xs, y_dot)
            gm = g_m[:, _out_rows(prob, p), :]
            g_w = np.einsum(ops["g_w"], U, gm, optimize=True)
            g_U = np.einsum(ops["g_U"], w_e[:, pi], gm, optimize=True)
            gUdot_w = np.einsum(ops["g_U"], w_dot[:, pi], gm, optimize=True)
            d_W[:, pi] += (np.einsum(ops["dW_a"], R_dot, g_w, optimize=True)
                           + np.einsum(ops["dW_b"], R, U_dot, gm, optimize=True))
            dx_e = (np.einsum("abc,eb,eic->eai", C, y_dot, g_U, optimize=True)
                    + np.einsum("abc,eb,eic->eai", C, y, gUdot_w, optimize=True))
            np.add.at(d_x[:, _in_rows(prob, p), :], s, dx_e)
            dgo = (np.einsum(ops["msg"], w_dot[:, pi], U, optimize=True)
                   + np.einsum(ops["msg"], w_e[:, pi], U_dot, optimize=True))
            np.add.at(d_gout[:, _out_rows(prob, p), :], v, dgo)
    return d_W, d_x, d_gout


def double_backward_pos(prob: Problem, pos, senders, receivers, x, W, g_out, gg_pos):
    """dL_F/dpos for L_F = sum_n <gg_pos[n], g_pos[n]> (the Hessian term).

    For an edge e, the energy <g_m_e, m_e> is eps(r) = sum_k R_k(|r|) b_k . Y(r)
    with b_k[l2, m2] = sum_{p -> l2} sum W[k,p,ci,co] g_m[l3,co,m3] C^p[m1,m2,m3]
    x_s[l1,ci,m1], and g_r_e is its gradient.  With phi_e fixed,
    dL_F/dr_e = H_e phi_e for the Hessian H_e of eps:
      H_e = sum_k [ R''_k B_k rr^T + R'_k B_k (I - rr^T)/d + R'_k (r (J^T b_k)^T + (J^T b_k) r^T)
                    + R_k sum_m2 b_k[m2] Hess Y_m2 ]      (r = r_hat, B_k = b_k . Y)
    and dL_F/dpos[s] += H_e phi_e, dL_F/dpos[v] -= H_e phi_e.  An edge with
    d = 0 or d >= c contributes nothing.
    """
    pos, x, W = _as64(pos), _as64(x), _as64(W)
    g_out, gg_pos = _as64(g_out), _as64(gg_pos)
    senders = np.asarray(senders, dtype=np.int64)
    receivers = np.asarray(receivers, dtype=np.int64)
    K = prob.num_basis
    nsh = (prob.sh_lmax + 1) ** 2
    d_pos = np.zeros_like(pos)
    eye = np.eye(3)
    for a, b in _chunks(prob, len(senders)):
        s, v = senders[a:b], receivers[a:b]
        r, d, rhat, R, Y = _edge_terms(prob, pos, s, v)
        dR = _radial.bessel_radial_deriv(d, K, prob.cutoff, prob.envelope_p)
        d2R = _radial.bessel_radial_deriv2(d, K, prob.cutoff, prob.envelope_p)
        JY = _sh.sh_jacobian(prob.sh_lmax, r)                       # [e, m, 3]
        HY = _sh.sh_hessian(prob.sh_lmax, r)                        # [e, m, 3, 3]
        phi = gg_pos[s] - gg_pos[v]
        g_m = g_out[v]
        bk = np.zeros((len(s), K, nsh))
        for pi, p in enumerate(prob.paths):
            gm = g_m[:, _out_rows(prob, p), :]                       # [e, m3, co]
            if prob.channelwise:
                G = np.einsum("ki,eci->ekic", W[:, pi], gm, optimize=True)
            else:
                G = np.einsum("kio,eco->ekic", W[:, pi], gm, optimize=True)
            l2 = p["l2"]
            bk[:, :, l2 * l2:(l2 + 1) * (l2 + 1)] += np.einsum(
                "abc,eai,ekic->ekb", p["C"], _x_block(prob, x, s, p), G, optimize=True)
        B = np.einsum("ekm,em->ek", bk, Y)
        Jb = np.einsum("ekm,emj->ekj", bk, JY)
        Hb = np.einsum("ekm,emij->eij", np.einsum("ek,ekm->ekm", R, bk), HY)
        rr = rhat[:, :, None] * rhat[:, None, :]
        safe = np.where(d > 0, d, 1.0)
        H = (np.einsum("ek,ek->e", d2R, B)[:, None, None] * rr
             + (np.einsum("ek,ek->e", dR, B) / safe)[:, None, None] * (eye[None] - rr)
             + np.einsum("ek,eki,ej->eij", dR, Jb, rhat) + np.einsum("ek,ei,ekj->eij", dR, rhat, Jb)
             + Hb)
        Hphi = np.einsum("eij,ej->ei", H, phi)
        Hphi = np.where((d > 0)[:, None], Hphi, 0.0)
        np.add.at(d_pos, s, Hphi)
        np.add.at(d_pos, v, -Hphi)
    return d_pos
