"""Pins for oracle.sh and oracle.radial.

Harmonics: scipy's complex harmonics (Condon-Shortley phase) mapped through U
and scaled by sqrt(4 pi); the addition-theorem norm sum_m Y^2 = 2l+1;
harmonicity of r^l Y; the Jacobian against central differences.
Radial: orthonormality of the bare Bessel functions under the d^2 dd measure
(quadrature), the envelope's boundary values and derivative, R' against
central differences, the d -> 0 limit and the cutoff.
"""
import math

import numpy as np
import pytest
from scipy import integrate, special

from oracle import cg, radial, sh


def test_sh_matches_scipy_through_U():
    rng = np.random.default_rng(0)
    pts = rng.normal(size=(40, 3))
    u = pts / np.linalg.norm(pts, axis=1, keepdims=True)
    theta = np.arccos(np.clip(u[:, 2], -1, 1))
    phi = np.arctan2(u[:, 1], u[:, 0])
    for l in range(sh.LMAX + 1):
        Yc = np.stack([special.sph_harm_y(l, m, theta, phi) for m in range(-l, l + 1)], -1)
        Yr = math.sqrt(4 * math.pi) * np.einsum("mk,ek->em", cg.complex_to_real(l), Yc)
        assert np.abs(Yr.imag).max() < 1e-13
        assert np.abs(Yr.real - sh.sh_single_l(l, pts)).max() < 1e-13


def test_sh_norm_and_l1_form():
    rng = np.random.default_rng(1)
    pts = rng.normal(size=(30, 3)) * 3.0
    for l in range(sh.LMAX + 1):
        Y = sh.sh_single_l(l, pts)
        assert np.abs((Y ** 2).sum(-1) - (2 * l + 1)).max() < 1e-12
    u = pts / np.linalg.norm(pts, axis=1, keepdims=True)
    assert np.abs(sh.sh_single_l(1, pts) - math.sqrt(3) * u[:, [1, 2, 0]]).max() < 1e-14


def test_sh_harmonic_polynomials():
    # |r|^l Y_lm(r) is a harmonic polynomial: its Laplacian vanishes (the central
    # second difference is exact for polynomials of degree <= 3)
    rng = np.random.default_rng(2)
    pts = rng.normal(size=(10, 3))
    h = 1e-2
    for l in range(1, sh.LMAX + 1):
        def P(r):
            return sh.sh_single_l(l, r) * np.linalg.norm(r, axis=-1, keepdims=True) ** l
        lap = sum((P(pts + h * e) - 2 * P(pts) + P(pts - h * e)) / h ** 2 for e in np.eye(3))
        assert np.abs(lap).max() < 1e-8


def test_sh_jacobian_fd():
    rng = np.random.default_rng(3)
    pts = rng.normal(size=(15, 3)) * 2.0
    h = 1e-6
    J = sh.sh_jacobian(sh.LMAX, pts)
    for j in range(3):
        e = np.zeros(3)
        e[j] = h
        fd = (sh.spherical_harmonics(sh.LMAX, pts + e) - sh.spherical_harmonics(sh.LMAX, pts - e)) / (2 * h)
        assert np.abs(fd - J[..., j]).max() < 1e-7


def test_sh_zero_vector():
    Y = sh.spherical_harmonics(3, np.zeros((2, 3)))
    assert np.all(Y[:, 0] == 1) and np.all(Y[:, 1:] == 0)
    assert np.all(sh.sh_jacobian(3, np.zeros((2, 3))) == 0)


def _envelope_from_conditions(x, p):
    """u(x) = 1 + a x^p + b x^(p+1) + c x^(p+2) with u(1) = u'(1) = u''(1) = 0,
    the coefficients solved here from those three conditions (not read from
    the oracle), so this is an independent statement of the cutoff polynomial."""
    A = np.array([[1.0, 1.0, 1.0],
                  [p, p + 1.0, p + 2.0],
                  [p * (p - 1.0), (p + 1.0) * p, (p + 2.0) * (p + 1.0)]])
    a, b, c = np.linalg.solve(A, np.array([-1.0, 0.0, 0.0]))
    x = np.asarray(x, dtype=np.float64)
    return np.where(x < 1.0, 1.0 + a * x ** p + b * x ** (p + 1) + c * x ** (p + 2), 0.0)


@pytest.mark.parametrize("p", [2, 3, 6, 9])
def test_envelope_matches_boundary_conditions(p):
    xs = np.linspace(0.0, 1.2, 61)
    assert np.abs(radial.envelope(xs, p) - _envelope_from_conditions(xs, p)).max() < 1e-12


@pytest.mark.parametrize("p", [3, 6, 8])
def test_bessel_radial_interior_values(p):
    # R_k(d) = sqrt(2/c) sin(k pi d / c) / d * u(d / c), with sin(t)/t = j0(t):
    # sin(k pi d / c) / d = (k pi / c) j0(k pi d / c).  A radial basis whose
    # envelope were taken at d instead of d / c, or with the wrong prefactor or
    # frequency, fails this.
    c, K = 5.0, 16
    rng = np.random.default_rng(4)
    d = np.concatenate([rng.uniform(0.01, c, 50), [0.3, 2.5, 4.99]])
    k = np.arange(1, K + 1)
    w = k * math.pi / c
    want = (math.sqrt(2.0 / c) * w[None, :] * special.spherical_jn(0, w[None, :] * d[:, None])
            * _envelope_from_conditions(d / c, p)[:, None])
    got = radial.bessel_radial(d, K, c, p)
    assert np.abs(got - want).max() < 1e-12


def test_bessel_orthonormal():
    # the oracle's own basis with its envelope divided out is orthonormal under
    # the d^2 dd measure on [0, c]
    c, K = 5.0, 6
    for n in range(1, K + 1):
        for m in range(n, K + 1):
            def f(d):
                R = radial.bessel_radial(np.array([d]), K, c)[0] / radial.envelope(np.array(d / c))
                return R[n - 1] * R[m - 1] * d * d
            val, _ = integrate.quad(f, 1e-9, c * (1 - 1e-12), limit=200)
            assert val == pytest.approx(float(n == m), abs=1e-9)


def test_envelope_boundary_and_derivative():
    p = 6
    assert radial.envelope(np.array(0.0), p) == 1.0
    x1 = np.array(1.0 - 1e-12)
    assert abs(radial.envelope(x1, p)) < 1e-20
    assert abs(radial.envelope_deriv(x1, p)) < 1e-20
    xs = np.linspace(0.05, 0.95, 19)
    assert np.abs(radial.envelope_deriv(xs, p) + 168 * xs ** 5 * (1 - xs) ** 2).max() < 1e-12
    h = 1e-6
    fd = (radial.envelope(xs + h, p) - radial.envelope(xs - h, p)) / (2 * h)
    assert np.abs(fd - radial.envelope_deriv(xs, p)).max() < 1e-8
    # u''(1) = 0: the second difference of u at 1-h shrinks linearly with h
    for h in (1e-3, 1e-4):
        x = 1.0 - h
        second = (radial.envelope(np.array(x + h / 2)) - 2 * radial.envelope(np.array(x))
                  + radial.envelope(np.array(x - h / 2))) / (h / 2) ** 2
        assert abs(second) < 400 * h
    assert radial.envelope(np.array([1.0, 1.5])).tolist() == [0.0, 0.0]


def test_radial_derivative_limit_and_cutoff():
    c, K = 5.0, 16
    d = np.linspace(0.2, 4.9, 40)
    h = 1e-6
    fd = (radial.bessel_radial(d + h, K, c) - radial.bessel_radial(d - h, K, c)) / (2 * h)
    assert np.abs(fd - radial.bessel_radial_deriv(d, K, c)).max() < 1e-6
    r0 = radial.bessel_radial(np.array([0.0]), K, c)
    rs = radial.bessel_radial(np.array([1e-7]), K, c)
    assert np.abs(r0 - rs).max() < 1e-9
    assert np.allclose(r0[0], math.sqrt(2 / c) * np.arange(1, K + 1) * math.pi / c)
    assert np.all(radial.bessel_radial(np.array([5.0, 6.0]), K, c) == 0)
    assert np.all(radial.bessel_radial_deriv(np.array([0.0, 5.0, 6.0]), K, c) == 0)


def test_sh_hessian_against_jacobian_differences():
    rng = np.random.default_rng(5)
    pts = rng.normal(size=(15, 3)) * 2.0
    H = sh.sh_hessian(sh.LMAX, pts)
    assert np.abs(H - np.swapaxes(H, -1, -2)).max() < 1e-12
    h = 1e-6
    for j in range(3):
        e = np.zeros(3)
        e[j] = h
        fd = (sh.sh_jacobian(sh.LMAX, pts + e) - sh.sh_jacobian(sh.LMAX, pts - e)) / (2 * h)
        assert np.abs(fd - H[..., j]).max() < 1e-7
    assert np.all(sh.sh_hessian(3, np.zeros((2, 3))) == 0)


@pytest.mark.parametrize("p", [3, 6])
def test_radial_second_derivative(p):
    c, K = 5.0, 16
    d = np.linspace(0.2, 4.9, 40)
    h = 1e-6
    fd = (radial.bessel_radial_deriv(d + h, K, c, p) - radial.bessel_radial_deriv(d - h, K, c, p)) / (2 * h)
    assert np.abs(fd - radial.bessel_radial_deriv2(d, K, c, p)).max() < 1e-5
    xs = np.linspace(0.05, 0.95, 19)
    fd = (radial.envelope_deriv(xs + h, p) - radial.envelope_deriv(xs - h, p)) / (2 * h)
    assert np.abs(fd - radial.envelope_deriv2(xs, p)).max() < 1e-6
    assert abs(radial.envelope_deriv2(np.array(1.0 - 1e-12), p)) < 1e-9
    assert np.all(radial.bessel_radial_deriv2(np.array([0.0, 5.0, 6.0]), K, c, p) == 0)
