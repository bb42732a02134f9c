"""Pins of the channel-wise ("uvu") oracle.

The channel-wise product with weights W[k, p, c] is, by definition, the fully
connected product with the weights W_full[k, p, ci, co] = delta(ci, co) W[k, p, ci]
(Sobek page, abstract: the edge-conditioned convolution with per-path
multiplicity mixing; here the mixing matrix is diagonal).  The fully connected
oracle is pinned on its own (test_oracle_layer.py), so every output and
gradient of the channel-wise oracle is checked against it on the same inputs,
plus a finite-difference check of the weight gradient that does not go
through that identity.
"""
import numpy as np
import pytest

from equivariant_gnn_tensor_receiver_amd import inputs
from oracle import tpconv as otp

IRREPS = "4x0e+4x1o+4x2e"


def _case(seed=3, N=24, deg=9):
    pos, rowptr, senders, rng = inputs.random_graph(N, deg, seed)
    cw = otp.Problem(IRREPS, IRREPS, 2, 8, channelwise=True)
    full = otp.Problem(IRREPS, IRREPS, 2, 8)
    C = cw.C_in
    x = rng.standard_normal((N, cw.D_in, C))
    W = rng.standard_normal(cw.w_shape) / np.sqrt(8.0)
    W_full = np.einsum("kpi,io->kpio", W, np.eye(C))
    g_out = rng.standard_normal((N, cw.D_out, C))
    gg = rng.standard_normal((N, 3))
    rcv = otp.csr_receivers(rowptr)
    return cw, full, pos.astype(np.float64), senders.astype(np.int64), rcv, x, W, W_full, g_out, gg


def _diag(G):
    return np.einsum("kpii->kpi", G)


def test_shapes_and_validation():
    cw = otp.Problem(IRREPS, IRREPS, 2, 8, channelwise=True)
    assert cw.w_shape == (8, cw.P, 4)
    with pytest.raises(ValueError):
        otp.Problem("4x0e", "8x0e", 0, 8, channelwise=True)


def test_forward_equals_diagonal_fully_connected():
    cw, full, pos, s, v, x, W, Wf, _, _ = _case()
    a = otp.forward(cw, pos, s, v, x, W)
    b = otp.forward(full, pos, s, v, x, Wf)
    assert np.abs(b).max() > 1e-3
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * np.abs(b).max())


def test_backward_equals_diagonal_fully_connected():
    cw, full, pos, s, v, x, W, Wf, g, _ = _case()
    gx, gW, gp = otp.backward(cw, pos, s, v, x, W, g)
    fx, fW, fp = otp.backward(full, pos, s, v, x, Wf, g)
    for a, b in ((gx, fx), (gW, _diag(fW)), (gp, fp)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * np.abs(b).max())


def test_double_backward_equals_diagonal_fully_connected():
    cw, full, pos, s, v, x, W, Wf, g, gg = _case()
    dW, dx, dg = otp.double_backward(cw, pos, s, v, x, W, g, gg)
    fW, fx, fg = otp.double_backward(full, pos, s, v, x, Wf, g, gg)
    for a, b in ((dW, _diag(fW)), (dx, fx), (dg, fg)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * np.abs(b).max())


def test_double_backward_pos_equals_diagonal_fully_connected():
    cw, full, pos, s, v, x, W, Wf, g, gg = _case()
    a = otp.double_backward_pos(cw, pos, s, v, x, W, g, gg)
    b = otp.double_backward_pos(full, pos, s, v, x, Wf, g, gg)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * np.abs(b).max())


def test_weight_gradient_finite_difference():
    cw, _, pos, s, v, x, W, _, g, _ = _case(seed=5)
    _, gW, _ = otp.backward(cw, pos, s, v, x, W, g)
    rng = np.random.default_rng(0)
    dW = rng.standard_normal(W.shape)
    h = 1e-6
    f = lambda w: float(np.sum(g * otp.forward(cw, pos, s, v, x, w)))
    fd = (f(W + h * dW) - f(W - h * dW)) / (2 * h)
    assert abs(fd - float(np.sum(gW * dW))) <= 1e-7 * max(1.0, abs(fd))
