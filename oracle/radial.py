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
derivative is 0 (the function is even in d).
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
