"""Edge-conditioned CG tensor-product convolution, conventional schedule (fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What is computed ("Sobek" page, abstract: equivariant GNNs apply
edge-conditioned tensor-product convolutions over graph edges; conventional
implementations materialise edge-specific weights, messages and adjoints).  For
every directed edge e = (s -> v) of the receiver-sorted graph:

  r_e = pos[s] - pos[v],  d = |r_e|,  r_hat = r_e / d
  R_e[k]            radial basis (oracle.radial): the fixed Bessel x envelope
                    functions, or a radial MLP on them whose last hidden width
                    is K (oracle.radial.mlp_radial, weights radial_w)
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
  x   [N][F_in], out [N][F_out]: per irrep a [2l+1][mul] block, irreps in order
      (with one multiplicity per side: [N][D][C], rows l^2+l+m)
  W   per k, per path a [mul(l1 irrep)][mul(l3 irrep)] block (uvw) or a
      [mul] block (uvu), P paths in oracle.cg order (uniform: [K][P][Ci][Co] / [K][P][C])
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
    """Irreps, paths and layouts of one operator.

    Multiplicities may differ between irreps ("varied feature structures"):
    irrep i of a side has mul_i channels.  Node tensors are stored flat,
    [N][F] with F = sum_i (2l_i+1) mul_i, irrep i's block [2l_i+1][mul_i] at
    offset foff[i]; with one multiplicity C per side this is the [N][D][C]
    array.  Fully connected weights are [K][sum_p mul(i1_p) mul(i3_p)], path
    p's block [mul(i1_p)][mul(i3_p)] at woff[p] within each k; with uniform
    multiplicities this is [K][P][C_in][C_out].  Channel-wise weights need
    mul(i1_p) = mul(i3_p) and are [K][sum_p mul_p] (uniform: [K][P][C]).
    """

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
        self.uniform = len(muls_in) == 1 and len(muls_out) == 1
        self.C_in = next(iter(muls_in)) if len(muls_in) == 1 else None
        self.C_out = next(iter(muls_out)) if len(muls_out) == 1 else None
        self.D_in = _cg.irreps_dim(self.ir_in)
        self.D_out = _cg.irreps_dim(self.ir_out)
        self.off_in = _cg.irreps_offsets(self.ir_in)
        self.off_out = _cg.irreps_offsets(self.ir_out)
        self.F_in = sum((2 * l + 1) * m for m, l, _ in self.ir_in)
        self.F_out = sum((2 * l + 1) * m for m, l, _ in self.ir_out)
        self.foff_in = list(np.cumsum([0] + [(2 * l + 1) * m for m, l, _ in self.ir_in])[:-1])
        self.foff_out = list(np.cumsum([0] + [(2 * l + 1) * m for m, l, _ in self.ir_out])[:-1])
        self.paths = _cg.enumerate_paths(self.ir_in, self.sh_lmax, self.ir_out)
        self.P = len(self.paths)
        woff = 0
        for p in self.paths:
            p["C"] = _cg.real_cg(p["l1"], p["l2"], p["l3"])
            p["C1"] = self.ir_in[p["i1"]][0]
            p["C3"] = self.ir_out[p["i3"]][0]
            if self.channelwise and p["C1"] != p["C3"]:
                raise ValueError("the channel-wise product needs equal multiplicities on each path")
            p["woff"] = woff
            woff += p["C1"] if self.channelwise else p["C1"] * p["C3"]
        self.W_per_k = woff
        if self.channelwise and self.uniform and self.C_in != self.C_out:
            raise ValueError("the channel-wise product needs equal multiplicities")

    @property
    def w_shape(self):
        if self.uniform:
            if self.channelwise:
                return (self.num_basis, self.P, self.C_in)
            return (self.num_basis, self.P, self.C_in, self.C_out)
        return (self.num_basis, self.W_per_k)

    def in_shape(self, N):
        return (N, self.D_in, self.C_in) if self.uniform else (N, self.F_in)

    def out_shape(self, N):
        return (N, self.D_out, self.C_out) if self.uniform else (N, self.F_out)


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
    per_edge = 8 * max(1, prob.W_per_k)
    step = int(max(1, min(E, 48_000_000 // per_edge)))
    for a in range(0, E, step):
        yield a, min(E, a + step)


def _radial_terms(prob, d, radial_w):
    """R, R', R'' per edge (the fixed basis, or the radial MLP when radial_w is given) and the MLP's (z, z', B, B')."""
    K = prob.num_basis
    if radial_w is not None:
        return _radial.mlp_radial(d, radial_w, K, prob.cutoff, prob.envelope_p)
    return (_radial.bessel_radial(d, K, prob.cutoff, prob.envelope_p),
            _radial.bessel_radial_deriv(d, K, prob.cutoff, prob.envelope_p),
            _radial.bessel_radial_deriv2(d, K, prob.cutoff, prob.envelope_p), None)


def _edge_terms(prob, pos, s, v, radial_w=None):
    r, d, rhat = _geometry(pos, s, v)
    R, R1, R2, mlp = _radial_terms(prob, d, radial_w)
    Y = _sh.spherical_harmonics(prob.sh_lmax, r)
    return r, d, rhat, R, Y, R1, R2, mlp


# Views of the flat node tensors and weights for one path.
def _in_slice(prob, p):
    o = prob.foff_in[p["i1"]]
    return slice(o, o + (2 * p["l1"] + 1) * p["C1"])


def _out_slice(prob, p):
    o = prob.foff_out[p["i3"]]
    return slice(o, o + (2 * p["l3"] + 1) * p["C3"])


def _x_block(prob, x, s, p):
    return x[s, _in_slice(prob, p)].reshape(len(s), 2 * p["l1"] + 1, p["C1"])      # [e, m1, ci]


def _go_block(prob, g, v, p):
    return g[v, _out_slice(prob, p)].reshape(len(v), 2 * p["l3"] + 1, p["C3"])     # [e, m3, co]


def _w_block(prob, W, p):
    if prob.channelwise:
        return W[:, p["woff"]:p["woff"] + p["C1"]]                                   # [k, i]
    return W[:, p["woff"]:p["woff"] + p["C1"] * p["C3"]].reshape(-1, p["C1"], p["C3"])  # [k, i, o]


def _y_block(Y, p):
    l2 = p["l2"]
    return Y[:, l2 * l2:(l2 + 1) * (l2 + 1)]            # [e, m2]


def _flat(prob, a, side):
    a = np.asarray(a, dtype=np.float64)
    return a.reshape(a.shape[0], prob.F_in if side == "in" else prob.F_out)


def _flat_w(prob, W):
    W = np.asarray(W, dtype=np.float64)
    return W.reshape(W.shape[0], prob.W_per_k)


def _coupling(C, xs, y):
    """U[e, ci, m3] = sum_{m1,m2} C[m1,m2,m3] xs[e,m1,ci] y[e,m2]."""
    return np.einsum("abc,eai,eb->eic", C, xs, y, optimize=True)


# einsum forms of the per-path weight contractions (e edge, k basis, i input
# channel, o output channel, c the m3 component).
def _ops(prob):
    if prob.channelwise:  # w_e[e, i]; messages and adjoints keep the channel i
        return dict(w="ek,ki->ei", msg="ei,eic->eci", g_w="eic,eci->ei", g_U="ei,eci->eic",
                    g_W="ek,ei->ki", g_R="ki,ei->ek", dW_b="ek,eic,eci->ki", G="ki,eci->ekic")
    return dict(w="ek,kio->eio", msg="eio,eic->eco", g_w="eic,eco->eio", g_U="eio,eco->eic",
                g_W="ek,eio->kio", g_R="kio,eio->ek", dW_b="ek,eic,eco->kio", G="kio,eco->ekic")


def _as64(a):
    return np.asarray(a, dtype=np.float64)


def forward(prob: Problem, pos, senders, receivers, x, W, num_nodes=None, radial_w=None):
    """out[v] = sum over edges into v of the materialised message m_e.

    radial_w: None for the fixed radial basis, or the K x K weights A of the
    radial MLP (oracle.radial.mlp_radial)."""
    pos = _as64(pos)
    xf, Wf = _flat(prob, x, "in"), _flat_w(prob, W)
    senders = np.asarray(senders, dtype=np.int64)
    receivers = np.asarray(receivers, dtype=np.int64)
    N = xf.shape[0] if num_nodes is None else num_nodes
    out = np.zeros((N, prob.F_out))
    ops = _ops(prob)
    for a, b in _chunks(prob, len(senders)):
        s, v = senders[a:b], receivers[a:b]
        _, _, _, R, Y, _, _, _ = _edge_terms(prob, pos, s, v, radial_w)
        for p in prob.paths:
            w_e = np.einsum(ops["w"], R, _w_block(prob, Wf, p), optimize=True)       # per-edge weights
            U = _coupling(p["C"], _x_block(prob, xf, s, p), _y_block(Y, p))
            msg = np.einsum(ops["msg"], w_e, U, optimize=True)                        # message [e, m3, co]
            np.add.at(out[:, _out_slice(prob, p)], v, msg.reshape(len(s), -1))
    return out.reshape(prob.out_shape(N))


def backward(prob: Problem, pos, senders, receivers, x, W, g_out, radial_w=None):
    """Materialised adjoints; returns (g_x, g_W, g_pos) for the loss <g_out, out>.

    With the radial MLP (radial_w = A) also g_A, from the per-edge adjoint of
    the radial functions: dL/dA[k, j] = sum_e g_R[e, k] silu'(z_ek) B_j(d_e)."""
    pos = _as64(pos)
    xf, Wf, gf = _flat(prob, x, "in"), _flat_w(prob, W), _flat(prob, g_out, "out")
    senders = np.asarray(senders, dtype=np.int64)
    receivers = np.asarray(receivers, dtype=np.int64)
    N = xf.shape[0]
    K = prob.num_basis
    g_x = np.zeros_like(xf)
    g_W = np.zeros_like(Wf)
    g_pos = np.zeros_like(pos)
    g_A = np.zeros((K, K))
    ops = _ops(prob)
    for a, b in _chunks(prob, len(senders)):
        s, v = senders[a:b], receivers[a:b]
        r, d, rhat, R, Y, dR, _, mlp = _edge_terms(prob, pos, s, v, radial_w)
        JY = _sh.sh_jacobian(prob.sh_lmax, r)                     # [e, Dsh, 3]
        g_Y = np.zeros_like(Y)
        g_R = np.zeros_like(R)
        for p in prob.paths:
            C = p["C"]
            Wp = _w_block(prob, Wf, p)
            w_e = np.einsum(ops["w"], R, Wp, optimize=True)
            xs = _x_block(prob, xf, s, p)
            y = _y_block(Y, p)
            U = _coupling(C, xs, y)
            gm = _go_block(prob, gf, v, p)                            # message adjoint [e, m3, co]
            g_w = np.einsum(ops["g_w"], U, gm, optimize=True)
            g_U = np.einsum(ops["g_U"], w_e, gm, optimize=True)
            gx_e = np.einsum("abc,eb,eic->eai", C, y, g_U, optimize=True)
            np.add.at(g_x[:, _in_slice(prob, p)], s, gx_e.reshape(len(s), -1))
            l2 = p["l2"]
            g_Y[:, l2 * l2:(l2 + 1) * (l2 + 1)] += np.einsum("abc,eai,eic->eb", C, xs, g_U, optimize=True)
            blk = np.einsum(ops["g_W"], R, g_w, optimize=True)
            g_W[:, p["woff"]:p["woff"] + blk[0].size] += blk.reshape(K, -1)
            g_R += np.einsum(ops["g_R"], Wp, g_w, optimize=True)
        g_r = (np.einsum("ek,ek->e", g_R, dR)[:, None] * rhat
               + np.einsum("em,emj->ej", g_Y, JY))
        np.add.at(g_pos, s, g_r)
        np.add.at(g_pos, v, -g_r)
        if mlp is not None:
            z, _, Bj, _ = mlp
            g_A += np.einsum("ek,ej->kj", g_R * _radial.silu_d1(z), Bj)
    res = (g_x.reshape(prob.in_shape(N)), g_W.reshape(np.shape(W)), g_pos)
    return res + (g_A,) if radial_w is not None else res


def double_backward(prob: Problem, pos, senders, receivers, x, W, g_out, gg_pos, radial_w=None):
    """Gradients of L_F = sum_n <gg_pos[n], g_pos[n]> w.r.t. W, x and g_out.

    With phi_e = gg_pos[s] - gg_pos[v], L_F = sum_e <phi_e, g_r_e>, the
    derivative of the edge energy <g_m_e, m_e> along phi_e.  The tangents are
    R_dot = R'(d) (r_hat . phi), Y_dot = J_Y phi, U_dot = CG(x_s, Y_dot) and
    w_dot = sum_k R_dot[k] W[k]; L_F is linear in W, x and g_out, so no second
    derivatives of R or Y appear (those enter only d/dpos, double_backward_pos).

    With the radial MLP (radial_w = A) also d_A: L_F = sum_e sum_k
    [R_dot[e,k] g_R[e,k] + R[e,k] h[e,k]] with g_R[e,k] = <W[k], U gm> and
    h[e,k] = <W[k], U_dot gm>, and R_dot = R'(d)(r_hat . phi), so
    dL_F/dA[k,j] = sum_e (r_hat . phi) g_R (silu''(z) z' B_j + silu'(z) B'_j)
                 + h silu'(z) B_j.
    """
    pos, gg_pos = _as64(pos), _as64(gg_pos)
    xf, Wf, gf = _flat(prob, x, "in"), _flat_w(prob, W), _flat(prob, g_out, "out")
    senders = np.asarray(senders, dtype=np.int64)
    receivers = np.asarray(receivers, dtype=np.int64)
    N = xf.shape[0]
    K = prob.num_basis
    d_W = np.zeros_like(Wf)
    d_x = np.zeros_like(xf)
    d_gout = np.zeros_like(gf)
    d_A = np.zeros((K, K))
    ops = _ops(prob)
    for a, b in _chunks(prob, len(senders)):
        s, v = senders[a:b], receivers[a:b]
        r, d, rhat, R, Y, dR, _, mlp = _edge_terms(prob, pos, s, v, radial_w)
        JY = _sh.sh_jacobian(prob.sh_lmax, r)
        phi = gg_pos[s] - gg_pos[v]
        rphi = np.einsum("ej,ej->e", rhat, phi)
        R_dot = dR * rphi[:, None]
        Y_dot = np.einsum("emj,ej->em", JY, phi)
        g_R = np.zeros_like(R)
        h_R = np.zeros_like(R)
        for p in prob.paths:
            C = p["C"]
            Wp = _w_block(prob, Wf, p)
            w_e = np.einsum(ops["w"], R, Wp, optimize=True)
            w_dot = np.einsum(ops["w"], R_dot, Wp, optimize=True)
            xs = _x_block(prob, xf, s, p)
            y = _y_block(Y, p)
            y_dot = _y_block(Y_dot, p)
            U = _coupling(C, xs, y)
            U_dot = _coupling(C, xs, y_dot)
            gm = _go_block(prob, gf, v, p)
            g_w = np.einsum(ops["g_w"], U, gm, optimize=True)
            g_U = np.einsum(ops["g_U"], w_e, gm, optimize=True)
            gUdot_w = np.einsum(ops["g_U"], w_dot, gm, optimize=True)
            blk = (np.einsum(ops["g_W"], R_dot, g_w, optimize=True)
                   + np.einsum(ops["dW_b"], R, U_dot, gm, optimize=True))
            d_W[:, p["woff"]:p["woff"] + blk[0].size] += blk.reshape(K, -1)
            dx_e = (np.einsum("abc,eb,eic->eai", C, y_dot, g_U, optimize=True)
                    + np.einsum("abc,eb,eic->eai", C, y, gUdot_w, optimize=True))
            np.add.at(d_x[:, _in_slice(prob, p)], s, dx_e.reshape(len(s), -1))
            dgo = (np.einsum(ops["msg"], w_dot, U, optimize=True)
                   + np.einsum(ops["msg"], w_e, U_dot, optimize=True))
            np.add.at(d_gout[:, _out_slice(prob, p)], v, dgo.reshape(len(s), -1))
            if mlp is not None:
                g_R += np.einsum(ops["g_R"], Wp, g_w, optimize=True)
                h_R += np.einsum(ops["g_R"], Wp, np.einsum(ops["g_w"], U_dot, gm, optimize=True), optimize=True)
        if mlp is not None:
            z, z1, Bj, B1 = mlp
            s1, s2 = _radial.silu_d1(z), _radial.silu_d2(z)
            d_A += (np.einsum("ek,ej->kj", rphi[:, None] * g_R * s2 * z1, Bj)
                    + np.einsum("ek,ej->kj", rphi[:, None] * g_R * s1, B1)
                    + np.einsum("ek,ej->kj", h_R * s1, Bj))
    res = (d_W.reshape(np.shape(W)), d_x.reshape(prob.in_shape(N)), d_gout.reshape(prob.out_shape(N)))
    return res + (d_A,) if radial_w is not None else res


def double_backward_pos(prob: Problem, pos, senders, receivers, x, W, g_out, gg_pos, radial_w=None):
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
    pos, gg_pos = _as64(pos), _as64(gg_pos)
    xf, Wf, gf = _flat(prob, x, "in"), _flat_w(prob, W), _flat(prob, g_out, "out")
    ops = _ops(prob)
    senders = np.asarray(senders, dtype=np.int64)
    receivers = np.asarray(receivers, dtype=np.int64)
    K = prob.num_basis
    nsh = (prob.sh_lmax + 1) ** 2
    d_pos = np.zeros_like(pos)
    eye = np.eye(3)
    for a, b in _chunks(prob, len(senders)):
        s, v = senders[a:b], receivers[a:b]
        r, d, rhat, R, Y, dR, d2R, _ = _edge_terms(prob, pos, s, v, radial_w)
        JY = _sh.sh_jacobian(prob.sh_lmax, r)                       # [e, m, 3]
        HY = _sh.sh_hessian(prob.sh_lmax, r)                        # [e, m, 3, 3]
        phi = gg_pos[s] - gg_pos[v]
        bk = np.zeros((len(s), K, nsh))
        for p in prob.paths:
            gm = _go_block(prob, gf, v, p)                            # [e, m3, co]
            G = np.einsum(ops["G"], _w_block(prob, Wf, p), gm, optimize=True)
            l2 = p["l2"]
            bk[:, :, l2 * l2:(l2 + 1) * (l2 + 1)] += np.einsum(
                "abc,eai,ekic->ekb", p["C"], _x_block(prob, xf, s, p), G, optimize=True)
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
