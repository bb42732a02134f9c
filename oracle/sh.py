"""Real spherical harmonics of the edge direction and their Jacobian (fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The abstract of the Sobek page names spherical-harmonic coupling as one of the
three reassociated factors; it does not fix a basis.  The reading taken here:
real harmonics, component normalised (sum_m Y_lm^2 = 2l+1, Y_00 = 1), order
m = -l..l, obtained from the Condon-Shortley complex harmonics through the
matrix U of ``oracle.cg.complex_to_real`` and scaled by sqrt(4 pi).  In
Cartesian form each Y_lm(r_hat) = P_lm(r) / |r|^l with P_lm a homogeneous
harmonic polynomial of degree l, written out below for l <= 3.  The tests pin
these polynomials against scipy's complex harmonics mapped through U.

At r = 0 the direction is undefined; the reading taken is r_hat := 0, so
Y_00 = 1, Y_{l>=1} = 0 and the Jacobian (and Hessian) is 0.
"""
from __future__ import annotations

import math

import numpy as np

LMAX = 3

_S3 = math.sqrt(3.0)
_S5 = math.sqrt(5.0)
_S7 = math.sqrt(7.0)
_S15 = math.sqrt(15.0)
_S42 = math.sqrt(42.0)
_S70 = math.sqrt(70.0)
_S105 = math.sqrt(105.0)


def _poly(l, x, y, z):
    """Homogeneous polynomials P_lm, m = -l..l, stacked on the last axis."""
    if l == 0:
        return np.stack([np.ones_like(x)], -1)
    if l == 1:
        return np.stack([_S3 * y, _S3 * z, _S3 * x], -1)
    if l == 2:
        return np.stack([
            _S15 * x * y,
            _S15 * y * z,
            0.5 * _S5 * (2 * z * z - x * x - y * y),
            _S15 * x * z,
            0.5 * _S15 * (x * x - y * y),
        ], -1)
    if l == 3:
        return np.stack([
            0.25 * _S70 * y * (3 * x * x - y * y),
            _S105 * x * y * z,
            0.25 * _S42 * y * (4 * z * z - x * x - y * y),
            0.5 * _S7 * z * (2 * z * z - 3 * x * x - 3 * y * y),
            0.25 * _S42 * x * (4 * z * z - x * x - y * y),
            0.5 * _S105 * z * (x * x - y * y),
            0.25 * _S70 * x * (x * x - 3 * y * y),
        ], -1)
    raise ValueError(f"l={l} > {LMAX} not supported")


def _poly_grad(l, x, y, z):
    """Gradients of P_lm: shape (..., 2l+1, 3)."""
    zero = np.zeros_like(x)
    if l == 0:
        return np.stack([np.stack([zero, zero, zero], -1)], -2)
    if l == 1:
        one = np.ones_like(x) * _S3
        return np.stack([
            np.stack([zero, one, zero], -1),
            np.stack([zero, zero, one], -1),
            np.stack([one, zero, zero], -1),
        ], -2)
    if l == 2:
        return np.stack([
            _S15 * np.stack([y, x, zero], -1),
            _S15 * np.stack([zero, z, y], -1),
            _S5 * np.stack([-x, -y, 2 * z], -1),
            _S15 * np.stack([z, zero, x], -1),
            _S15 * np.stack([x, -y, zero], -1),
        ], -2)
    if l == 3:
        a = 0.25 * _S70
        b = 0.25 * _S42
        return np.stack([
            a * np.stack([6 * x * y, 3 * x * x - 3 * y * y, zero], -1),
            _S105 * np.stack([y * z, x * z, x * y], -1),
            b * np.stack([-2 * x * y, 4 * z * z - x * x - 3 * y * y, 8 * y * z], -1),
            0.5 * _S7 * np.stack([-6 * x * z, -6 * y * z, 6 * z * z - 3 * x * x - 3 * y * y], -1),
            b * np.stack([4 * z * z - 3 * x * x - y * y, -2 * x * y, 8 * x * z], -1),
            0.5 * _S105 * np.stack([2 * x * z, -2 * y * z, x * x - y * y], -1),
            a * np.stack([3 * x * x - 3 * y * y, -6 * x * y, zero], -1),
        ], -2)
    raise ValueError(f"l={l} > {LMAX} not supported")


def sh_single_l(l: int, r: np.ndarray) -> np.ndarray:
    """Y_l(r_hat) for vectors r (..., 3) -> (..., 2l+1); r = 0 gives r_hat := 0."""
    r = np.asarray(r, dtype=np.float64)
    d = np.linalg.norm(r, axis=-1)
    safe = np.where(d > 0, d, 1.0)
    u = r / safe[..., None]
    u = np.where((d > 0)[..., None], u, 0.0)
    return _poly(l, u[..., 0], u[..., 1], u[..., 2])


def spherical_harmonics(lmax: int, r: np.ndarray) -> np.ndarray:
    """All degrees 0..lmax concatenated: (..., (lmax+1)^2), row l^2+l+m."""
    return np.concatenate([sh_single_l(l, r) for l in range(lmax + 1)], -1)


def sh_jacobian_single_l(l: int, r: np.ndarray) -> np.ndarray:
    """dY_lm/dr (..., 2l+1, 3) for Y_lm(r) = P_lm(r)/|r|^l; zero at r = 0.

    d/dr [P / |r|^l] = grad P / |r|^l - l P r / |r|^(l+2).
    """
    r = np.asarray(r, dtype=np.float64)
    d = np.linalg.norm(r, axis=-1)
    ok = d > 0
    safe = np.where(ok, d, 1.0)
    x, y, z = r[..., 0], r[..., 1], r[..., 2]
    P = _poly(l, x, y, z)
    G = _poly_grad(l, x, y, z)
    J = G / safe[..., None, None] ** l - l * P[..., :, None] * r[..., None, :] / safe[..., None, None] ** (l + 2)
    return np.where(ok[..., None, None], J, 0.0)


def sh_jacobian(lmax: int, r: np.ndarray) -> np.ndarray:
    """(..., (lmax+1)^2, 3)."""
    return np.concatenate([sh_jacobian_single_l(l, r) for l in range(lmax + 1)], -2)


def _poly_hess(l, x, y, z):
    """Hessians of P_lm: shape (..., 2l+1, 3, 3) (constant for l = 2, linear for l = 3)."""
    zero = np.zeros_like(x)

    def sym(xx, xy, xz, yy, yz, zz):
        return np.stack([np.stack([xx, xy, xz], -1), np.stack([xy, yy, yz], -1), np.stack([xz, yz, zz], -1)], -2)

    if l <= 1:
        return np.zeros(x.shape + (2 * l + 1, 3, 3))
    one = np.ones_like(x)
    if l == 2:
        return np.stack([
            sym(zero, _S15 * one, zero, zero, zero, zero),
            sym(zero, zero, zero, zero, _S15 * one, zero),
            sym(-_S5 * one, zero, zero, -_S5 * one, zero, 2 * _S5 * one),
            sym(zero, zero, _S15 * one, zero, zero, zero),
            sym(_S15 * one, zero, zero, -_S15 * one, zero, zero),
        ], -3)
    if l == 3:
        a = 0.25 * _S70
        b = 0.25 * _S42
        c = 0.5 * _S7
        e = 0.5 * _S105
        return np.stack([
            sym(6 * a * y, 6 * a * x, zero, -6 * a * y, zero, zero),
            sym(zero, _S105 * z, _S105 * y, zero, _S105 * x, zero),
            sym(-2 * b * y, -2 * b * x, zero, -6 * b * y, 8 * b * z, 8 * b * y),
            sym(-6 * c * z, zero, -6 * c * x, -6 * c * z, -6 * c * y, 12 * c * z),
            sym(-6 * b * x, -2 * b * y, 8 * b * z, -2 * b * x, zero, 8 * b * x),
            sym(2 * e * z, zero, 2 * e * x, -2 * e * z, -2 * e * y, zero),
            sym(6 * a * x, -6 * a * y, zero, -6 * a * x, zero, zero),
        ], -3)
    raise ValueError(f"l={l} > {LMAX} not supported")


def sh_hessian_single_l(l: int, r: np.ndarray) -> np.ndarray:
    """d^2 Y_lm / dr dr (..., 2l+1, 3, 3) for Y = P q, q = |r|^-l; zero at r = 0.

    Product rule: H = H_P q + grad P (x) grad q + grad q (x) grad P + P H_q, with
    grad q = -l r |r|^-(l+2) and H_q = -l |r|^-(l+2) I + l (l+2) |r|^-(l+4) r r^T.
    """
    r = np.asarray(r, dtype=np.float64)
    d = np.linalg.norm(r, axis=-1)
    ok = d > 0
    safe = np.where(ok, d, 1.0)[..., None, None]
    x, y, z = r[..., 0], r[..., 1], r[..., 2]
    P = _poly(l, x, y, z)[..., None, None]                     # (..., m, 1, 1)
    G = _poly_grad(l, x, y, z)                                 # (..., m, 3)
    HP = _poly_hess(l, x, y, z)                                # (..., m, 3, 3)
    rr = r[..., None, :, None] * r[..., None, None, :]         # (..., 1, 3, 3)
    eye = np.eye(3)
    q = safe[..., None] ** (-l)                                # (..., 1, 1, 1)
    gq = -l * r[..., None, :] / safe ** (l + 2)                # (..., 1, 3)
    Hq = (-l * eye / safe[..., None] ** (l + 2) + l * (l + 2) * rr / safe[..., None] ** (l + 4))
    H = (HP * q + G[..., :, :, None] * gq[..., :, None, :] + gq[..., :, :, None] * G[..., :, None, :]
         + P * Hq)
    return np.where(ok[..., None, None, None], H, 0.0)


def sh_hessian(lmax: int, r: np.ndarray) -> np.ndarray:
    """(..., (lmax+1)^2, 3, 3)."""
    return np.concatenate([sh_hessian_single_l(l, r) for l in range(lmax + 1)], -3)
