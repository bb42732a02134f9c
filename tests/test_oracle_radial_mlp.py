"""Pins for the radial MLP front end of the oracle (fp64, CPU).

R_k(d) = silu(sum_j A[k, j] B_j(d)) with B the Bessel x envelope basis; the
network's last hidden layer is the K radial functions the reassociated state
uses, its output layer folds into W.  Checks independent of the oracle's own
formulas:
  * silu and its derivatives against z * expit(z) (scipy) and differences;
  * R' and R'' against central differences of R and R' in d; R vanishes at
    the cutoff; the d -> 0 limit is finite with R' = 0;
  * the orientation of A (row k = output function) and the slope silu'(0) = 1/2:
    with A = eps * (a cyclic permutation), the layer equals eps/2 times the
    fixed-basis layer with W's k index permuted the same way, to O(eps);
  * rotation equivariance of the whole layer;
  * every gradient the MLP adds or changes against central differences: the
    backward (g_x, g_W, g_pos, g_A of <g_out, out>) and the double backward
    (d_W, d_x, d_g_out, d_A and d_pos of L_F = <gg_pos, g_pos>).
"""
import numpy as np
import pytest
from scipy.special import expit

from oracle import radial
from oracle.tpconv import backward, double_backward, double_backward_pos, forward

from test_oracle_cg import random_rotation, wigner_from_sh
from test_oracle_layer import block_rotation, case

NAT2 = ("3x0e+3x1o+3x2e", "2x0e+2x1o+2x2e", 2, 4)
MIXED = ("2x0e+2x1o+2x1e+2x2e", "2x0e+2x0o+2x1o+2x1e+2x2e+2x3o", 2, 3)


def mlp_weights(K, seed=5, scale=1.0):
    return np.random.default_rng(seed).standard_normal((K, K)) * scale / np.sqrt(K)


def test_silu_and_derivatives():
    z = np.linspace(-8, 8, 161)
    assert np.allclose(radial.silu(z), z * expit(z), rtol=1e-14, atol=1e-15)
    h = 1e-5
    assert np.allclose(radial.silu_d1(z), (radial.silu(z + h) - radial.silu(z - h)) / (2 * h), rtol=1e-8, atol=1e-10)
    assert np.allclose(radial.silu_d2(z), (radial.silu_d1(z + h) - radial.silu_d1(z - h)) / (2 * h), rtol=1e-7,
                       atol=1e-9)
    assert radial.silu_d1(np.array(0.0)) == pytest.approx(0.5)


@pytest.mark.parametrize("K", [4, 8])
def test_mlp_radial_derivatives_and_limits(K):
    A = mlp_weights(K, scale=2.0)
    c = 5.0
    d = np.linspace(0.05, 4.95, 97)
    R, R1, R2, _ = radial.mlp_radial(d, A, K, c)
    h = 1e-5
    Rp, R1p, _, _ = radial.mlp_radial(d + h, A, K, c)
    Rm, R1m, _, _ = radial.mlp_radial(d - h, A, K, c)
    assert np.allclose(R1, (Rp - Rm) / (2 * h), rtol=1e-6, atol=1e-8)
    assert np.allclose(R2, (R1p - R1m) / (2 * h), rtol=1e-6, atol=1e-7)
    Rc, R1c, R2c, _ = radial.mlp_radial(np.array([c, c + 0.5]), A, K, c)
    assert np.abs(Rc).max() == 0 and np.abs(R1c).max() == 0 and np.abs(R2c).max() == 0
    R0, R10, _, _ = radial.mlp_radial(np.array([0.0, 1e-7]), A, K, c)
    assert np.isfinite(R0).all() and np.abs(R10[0]).max() == 0
    assert np.allclose(R0[0], R0[1], rtol=1e-6)


@pytest.mark.parametrize("spec", [NAT2, MIXED])
def test_small_weights_reduce_to_the_basis_with_permuted_k(spec):
    prob, pos, snd, rcv, x, W, _, _ = case(*spec, N=12, deg=5)
    K = prob.num_basis
    perm = np.roll(np.arange(K), 1)  # a cycle: its inverse differs from it for K > 2
    eps = 1e-6
    A = np.zeros((K, K))
    A[np.arange(K), perm] = eps     # R_k = silu(eps B_perm(k)) = eps/2 B_perm(k) + O(eps^2)
    out = forward(prob, pos, snd, rcv, x, W, radial_w=A)
    W2 = np.empty_like(W)
    W2[perm] = W                    # sum_k B_perm(k) W[k] = sum_j B_j W2[j]
    ref = 0.5 * eps * forward(prob, pos, snd, rcv, x, W2)
    assert np.abs(out - ref).max() <= 1e-5 * np.abs(ref).max()
    # the transposed reading of A gives a different layer
    bad = 0.5 * eps * forward(prob, pos, snd, rcv, x, W[np.roll(np.arange(K), 1)])
    assert np.abs(out - bad).max() > 1e-2 * np.abs(ref).max()


@pytest.mark.parametrize("spec", [NAT2, MIXED])
def test_rotation_equivariance_with_mlp(spec):
    prob, pos, snd, rcv, x, W, *_ = case(*spec, N=14, deg=6)
    A = mlp_weights(prob.num_basis)
    rng = np.random.default_rng(3)
    rot = random_rotation(rng)
    D = [wigner_from_sh(l, rot, rng) for l in range(4)]
    Din = block_rotation(prob.ir_in, D)
    Dout = block_rotation(prob.ir_out, D)
    out = forward(prob, pos, snd, rcv, x, W, radial_w=A)
    out_rot = forward(prob, pos @ rot.T, snd, rcv, np.einsum("ab,nbc->nac", Din, x), W, radial_w=A)
    assert np.abs(out_rot - np.einsum("ab,nbc->nac", Dout, out)).max() < 1e-11 * np.abs(out).max()


@pytest.mark.parametrize("spec", [NAT2, MIXED])
def test_backward_with_mlp_finite_differences(spec):
    prob, pos, snd, rcv, x, W, g_out, _ = case(*spec, N=10, deg=5)
    K = prob.num_basis
    A = mlp_weights(K)
    g_x, g_W, g_pos, g_A = backward(prob, pos, snd, rcv, x, W, g_out, radial_w=A)

    def L(px, pW, ppos, pA):
        return float((forward(prob, ppos, snd, rcv, px, pW, radial_w=pA) * g_out).sum())

    rng = np.random.default_rng(41)
    h = 1e-5
    for _ in range(2):
        dx, dW, dp, dA = (rng.standard_normal(a.shape) for a in (x, W, pos, A))
        assert (L(x + h * dx, W, pos, A) - L(x - h * dx, W, pos, A)) / (2 * h) == pytest.approx((g_x * dx).sum(),
                                                                                                rel=1e-7)
        assert (L(x, W + h * dW, pos, A) - L(x, W - h * dW, pos, A)) / (2 * h) == pytest.approx((g_W * dW).sum(),
                                                                                                rel=1e-7)
        assert (L(x, W, pos + h * dp, A) - L(x, W, pos - h * dp, A)) / (2 * h) == pytest.approx(
            (g_pos * dp).sum(), rel=1e-6)
        assert (L(x, W, pos, A + h * dA) - L(x, W, pos, A - h * dA)) / (2 * h) == pytest.approx(
            (g_A * dA).sum(), rel=1e-7)
    for k, j in [(0, 0), (1, K - 1), (K - 1, 1)]:
        e = np.zeros_like(A)
        e[k, j] = h
        assert (L(x, W, pos, A + e) - L(x, W, pos, A - e)) / (2 * h) == pytest.approx(g_A[k, j], rel=1e-6, abs=1e-9)


@pytest.mark.parametrize("spec", [NAT2, MIXED])
def test_double_backward_with_mlp_finite_differences(spec):
    prob, pos, snd, rcv, x, W, g_out, gg = case(*spec, N=10, deg=5)
    A = mlp_weights(prob.num_basis)
    d_W, d_x, d_g, d_A = double_backward(prob, pos, snd, rcv, x, W, g_out, gg, radial_w=A)
    d_pos = double_backward_pos(prob, pos, snd, rcv, x, W, g_out, gg, radial_w=A)

    def LF(px, pW, pg, ppos, pA):
        return float((backward(prob, ppos, snd, rcv, px, pW, pg, radial_w=pA)[2] * gg).sum())

    rng = np.random.default_rng(43)
    h = 1e-5
    args = (x, W, g_out, pos, A)
    for _ in range(2):
        for i, grad in enumerate((d_x, d_W, d_g, d_pos, d_A)):
            t = rng.standard_normal(args[i].shape)
            plus = list(args)
            minus = list(args)
            plus[i] = args[i] + h * t
            minus[i] = args[i] - h * t
            fd = (LF(*plus) - LF(*minus)) / (2 * h)
            assert fd == pytest.approx((grad * t).sum(), rel=2e-6), i
