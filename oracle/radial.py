"""Radial basis R_e[k] and its derivative (fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The Sobek abstract reassociates a "radial projection" with the harmonic
coupling and the aggregation; the workload description fixes K Bessel
functions with a p = 6 polynomial cutoff.  Reading taken:

    R_k(d) = sqrt(2/c) * sin(k pi d / c) / d * u(d / c),   k = 1..K,
    u(x)   = 1 - (p+1)(p+2)/2 x^p + p(p+2) x^(p+1) - p(p+1)/2 x^(p+2)   (x < 1)
           = 0                                                        (x >= 1)

so u(0) = 1 and u, u', u'' vanish at x = 1.  The frequencies are fixed (no
trainable radial network), so R feeds the weights W directly, which is what the
reassociation needs.  At d = 0, R_k takes its limit sqrt(2/c) k pi / c and the
derivative is 0 (the function is even in d); the second derivative, which only
the position Hessian of the force loss uses, is taken as 0 there as well (the
reading for a coincident edge: it contributes no position derivatives).
"""
from __future__ import annotations

import math

import numpy as np


def envelope(x: np.ndarray, p: int = 6) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    a = (p + 1) * (p + 2) / 2.0
    b = p * (p + 2.0)
    c = p * (p + 1) / 2.0
    u = 1.0 - a * x ** p + b * x ** (p + 1) - c * x ** (p + 2)
    return np.where(x < 1.0, u, 0.0)


def envelope_deriv(x: np.ndarray, p: int = 6) -> np.ndarray:
    """u'(x) = -p(p+1)(p+2)/2 * x^(p-1) (1-x)^2 for x < 1, else 0."""
    x = np.asarray(x, dtype=np.float64)
    k = p * (p + 1) * (p + 2) / 2.0
    du = -k * x ** (p - 1) * (1.0 - x) ** 2
    return np.where(x < 1.0, du, 0.0)


def bessel_radial(d: np.ndarray, K: int, cutoff: float, p: int = 6) -> np.ndarray:
    """R[..., k-1] = R_k(d) for k = 1..K."""
    d = np.asarray(d, dtype=np.float64)
    k = np.arange(1, K + 1, dtype=np.float64)
    pref = math.sqrt(2.0 / cutoff)
    w = k * math.pi / cutoff
    safe = np.where(d > 0, d, 1.0)[..., None]
    R = pref * np.sin(w * d[..., None]) / safe * envelope(d / cutoff, p)[..., None]
    limit = pref * w * np.ones_like(R)
    return np.where((d > 0)[..., None], R, limit)


def bessel_radial_deriv(d: np.ndarray, K: int, cutoff: float, p: int = 6) -> np.ndarray:
    """dR_k/dd; 0 at d = 0 and for d >= cutoff."""
    d = np.asarray(d, dtype=np.float64)
    k = np.arange(1, K + 1, dtype=np.float64)
    pref = math.sqrt(2.0 / cutoff)
    w = k * math.pi / cutoff
    safe = np.where(d > 0, d, 1.0)[..., None]
    dd = d[..., None]
    s = np.sin(w * dd)
    c = np.cos(w * dd)
    u = envelope(d / cutoff, p)[..., None]
    du = envelope_deriv(d / cutoff, p)[..., None] / cutoff
    dR = pref * ((w * c / safe - s / safe ** 2) * u + s / safe * du)
    return np.where((d > 0)[..., None], dR, 0.0)


def envelope_deriv2(x: np.ndarray, p: int = 6) -> np.ndarray:
    """u''(x) = -p(p+1)(p+2)/2 * [(p-1) x^(p-2) (1-x)^2 - 2 x^(p-1) (1-x)] for x < 1, else 0."""
    x = np.asarray(x, dtype=np.float64)
    k = p * (p + 1) * (p + 2) / 2.0
    d2 = -k * ((p - 1) * x ** (p - 2) * (1.0 - x) ** 2 - 2.0 * x ** (p - 1) * (1.0 - x))
    return np.where(x < 1.0, d2, 0.0)


def bessel_radial_deriv2(d: np.ndarray, K: int, cutoff: float, p: int = 6) -> np.ndarray:
    """d^2 R_k / dd^2 (product rule on pref * f(d) * u(d/c), f = sin(w d) / d); 0 at d = 0 and d >= cutoff."""
    d = np.asarray(d, dtype=np.float64)
    k = np.arange(1, K + 1, dtype=np.float64)
    pref = math.sqrt(2.0 / cutoff)
    w = k * math.pi / cutoff
    safe = np.where(d > 0, d, 1.0)[..., None]
    dd = d[..., None]
    s = np.sin(w * dd)
    c = np.cos(w * dd)
    f = s / safe
    f1 = w * c / safe - s / safe ** 2
    f2 = -w * w * s / safe - 2.0 * w * c / safe ** 2 + 2.0 * s / safe ** 3
    u = envelope(d / cutoff, p)[..., None]
    u1 = envelope_deriv(d / cutoff, p)[..., None] / cutoff
    u2 = envelope_deriv2(d / cutoff, p)[..., None] / cutoff ** 2
    d2R = pref * (f2 * u + 2.0 * f1 * u1 + f * u2)
    return np.where((d > 0)[..., None], d2R, 0.0)


# Radial MLP front end.  The pages name learned radial networks only as the
# usual setting of the layer; the reading taken keeps the reassociation intact
# by letting the network's last hidden layer be the K radial functions the
# streams consume, and folding its output layer into W:
#   R_k(d) = silu(z_k),  z_k = sum_j A[k, j] B_j(d),   silu(z) = z / (1 + exp(-z)),
# with B_j the Bessel x envelope basis above (K functions) and A the K x K
# weights of the hidden layer (no bias, so R vanishes with B at the cutoff).

def silu(z):
    return z / (1.0 + np.exp(-z))


def silu_d1(z):
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def silu_d2(z):
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 - s) * (2.0 + z * (1.0 - 2.0 * s))


def mlp_radial(d: np.ndarray, A: np.ndarray, K: int, cutoff: float, p: int = 6):
    """R, dR/dd and d2R/dd2 of the radial MLP, plus (z, z', B, B') for its weight gradients."""
    A = np.asarray(A, dtype=np.float64).reshape(K, K)
    B = bessel_radial(d, K, cutoff, p)
    B1 = bessel_radial_deriv(d, K, cutoff, p)
    B2 = bessel_radial_deriv2(d, K, cutoff, p)
    z = B @ A.T
    z1 = B1 @ A.T
    z2 = B2 @ A.T
    R = silu(z)
    R1 = silu_d1(z) * z1
    R2 = silu_d2(z) * z1 * z1 + silu_d1(z) * z2
    return R, R1, R2, (z, z1, B, B1)
