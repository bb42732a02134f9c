"""Clebsch-Gordan coefficients, real-basis coupling tables, irreps and paths (fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The operator couples sender features of degree l1 with the spherical harmonics
of the edge direction (degree l2) into output degree l3 through the full
Clebsch-Gordan tensor product ("The Price of Freedom", Approach and Key results:
the CG product is the fully expressive equivariant bilinear map, governed by
nonzero selection rules, and it can form the antisymmetric 1e cross-product
term).

Conventions (the pages fix none of them; these are the readings taken here):

* complex CG <l1 m1 l2 m2 | l3 m3> from the Racah closed form, evaluated in
  exact rational arithmetic and rounded once to fp64;
* real basis: the real spherical harmonic Y_{l,m} is the combination
  sum_mu U^l[m, mu] Y_l^mu of complex harmonics (Condon-Shortley phase) with
      m > 0 : (Y^{-m} + (-1)^m Y^{m}) / sqrt2
      m < 0 : i (Y^{m} - (-1)^m Y^{-m}) / sqrt2
      m = 0 : Y^0 ;
* the real table is C[m1,m2,m3] = sum U1[m1,mu1] U2[m2,mu2] conj(U3[m3,mu3]) CG.
  It is real when l1+l2+l3 is even and purely imaginary when odd; in the odd
  case the imaginary part is taken.  Tables are orthonormal in (m1,m2) for each
  m3 and carry no extra path normalisation.
"""
from __future__ import annotations

import math
import re
from fractions import Fraction
from functools import lru_cache

import numpy as np

_IRREP_RE = re.compile(r"^\s*(?:(\d+)\s*x\s*)?(\d+)\s*([eo])\s*$")


def parse_irreps(text: str):
    """Parse '32x0e+32x1o+32x2e' into a list of (mul, l, parity) with parity +1/-1."""
    out = []
    for term in text.split("+"):
        m = _IRREP_RE.match(term)
        if m is None:
            raise ValueError(f"bad irreps term {term!r} in {text!r}")
        mul = int(m.group(1)) if m.group(1) else 1
        out.append((mul, int(m.group(2)), 1 if m.group(3) == "e" else -1))
    return out


def irreps_dim(irreps) -> int:
    """Number of (l, m) rows: sum of 2l+1 over the irreps (channels are separate)."""
    return sum(2 * l + 1 for _, l, _ in irreps)


def irreps_offsets(irreps):
    """Row offset of each irrep block in the [rows][channels] feature layout."""
    offs, o = [], 0
    for _, l, _ in irreps:
        offs.append(o)
        o += 2 * l + 1
    return offs


def enumerate_paths(irreps_in, sh_lmax: int, irreps_out):
    """Selection rules ("The Price of Freedom", Approach: interactability).

    A path (i1, l2, i3) couples input irrep i1 = (l1, p1) with the degree-l2
    spherical harmonic (parity (-1)^l2) into output irrep i3 = (l3, p3).  It is
    kept iff the triangle |l1-l2| <= l3 <= l1+l2 holds and p1 * (-1)^l2 == p3.
    Order: input irrep, then l2, then output irrep.
    """
    paths = []
    for i1, (_, l1, p1) in enumerate(irreps_in):
        for l2 in range(sh_lmax + 1):
            p2 = 1 if l2 % 2 == 0 else -1
            for i3, (_, l3, p3) in enumerate(irreps_out):
                if abs(l1 - l2) <= l3 <= l1 + l2 and p1 * p2 == p3:
                    paths.append(dict(i1=i1, l1=l1, l2=l2, i3=i3, l3=l3))
    return paths


def _fact(n: int) -> int:
    return math.factorial(n)


def cg_complex_exact(j1, m1, j2, m2, J, M):
    """Return (sign, square) with <j1 m1 j2 m2 | J M> = sign * sqrt(square), exact.

    Racah's closed form: the coefficient is delta(M, m1+m2) times
    sqrt[(2J+1)(J+j1-j2)!(J-j1+j2)!(j1+j2-J)!/(j1+j2+J+1)!]
    * sqrt[(J+M)!(J-M)!(j1-m1)!(j1+m1)!(j2-m2)!(j2+m2)!]
    * sum_k (-1)^k / [k!(j1+j2-J-k)!(j1-m1-k)!(j2+m2-k)!(J-j2+m1+k)!(J-j1-m2+k)!].
    """
    if m1 + m2 != M or abs(m1) > j1 or abs(m2) > j2 or abs(M) > J:
        return 0, Fraction(0)
    if not (abs(j1 - j2) <= J <= j1 + j2):
        return 0, Fraction(0)
    pre = Fraction(
        (2 * J + 1) * _fact(J + j1 - j2) * _fact(J - j1 + j2) * _fact(j1 + j2 - J),
        _fact(j1 + j2 + J + 1),
    )
    pre *= (_fact(J + M) * _fact(J - M) * _fact(j1 - m1) * _fact(j1 + m1)
            * _fact(j2 - m2) * _fact(j2 + m2))
    s = Fraction(0)
    for k in range(0, j1 + j2 - J + 1):
        args = (j1 + j2 - J - k, j1 - m1 - k, j2 + m2 - k, J - j2 + m1 + k, J - j1 - m2 + k)
        if min(args) < 0:
            continue
        den = _fact(k)
        for a in args:
            den *= _fact(a)
        s += Fraction((-1) ** k, den)
    if s == 0:
        return 0, Fraction(0)
    return (1 if s > 0 else -1), s * s * pre


def cg_complex(j1, m1, j2, m2, J, M) -> float:
    """<j1 m1 j2 m2 | J M> in fp64 (one rounding of an exact value)."""
    sign, sq = cg_complex_exact(j1, m1, j2, m2, J, M)
    if sign == 0:
        return 0.0
    return sign * math.sqrt(sq)  # Fraction -> float is correctly rounded; sqrt adds <= 1 ulp


@lru_cache(maxsize=None)
def complex_to_real(l: int) -> np.ndarray:
    """U^l with rows = real index m (-l..l) and columns = complex index mu (-l..l)."""
    n = 2 * l + 1
    U = np.zeros((n, n), dtype=np.complex128)
    r2 = 1.0 / math.sqrt(2.0)
    for m in range(-l, l + 1):
        row = m + l
        if m > 0:
            U[row, -m + l] = r2
            U[row, m + l] = (-1) ** m * r2
        elif m < 0:
            U[row, m + l] = 1j * r2
            U[row, -m + l] = -1j * (-1) ** m * r2
        else:
            U[row, l] = 1.0
    return U


@lru_cache(maxsize=None)
def _cg_block_complex(l1, l2, l3) -> np.ndarray:
    out = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    for m1 in range(-l1, l1 + 1):
        for m2 in range(-l2, l2 + 1):
            m3 = m1 + m2
            if abs(m3) <= l3:
                out[m1 + l1, m2 + l2, m3 + l3] = cg_complex(l1, m1, l2, m2, l3, m3)
    return out


@lru_cache(maxsize=None)
def real_cg(l1: int, l2: int, l3: int) -> np.ndarray:
    """Real-basis coupling table C[m1, m2, m3] (shape (2l1+1, 2l2+1, 2l3+1)).

    C = sum_{mu} U1[m1,mu1] U2[m2,mu2] conj(U3[m3,mu3]) <l1 mu1 l2 mu2 | l3 mu3>;
    real part for even l1+l2+l3, imaginary part for odd (the other part is zero
    up to rounding; ``tests/test_oracle_cg.py`` checks that).
    """
    if not (abs(l1 - l2) <= l3 <= l1 + l2):
        raise ValueError(f"triangle rule fails for ({l1},{l2},{l3})")
    cg = _cg_block_complex(l1, l2, l3)
    U1, U2, U3 = complex_to_real(l1), complex_to_real(l2), complex_to_real(l3)
    C = np.einsum("ai,bj,ck,ijk->abc", U1, U2, U3.conj(), cg)
    out = C.real if (l1 + l2 + l3) % 2 == 0 else C.imag
    out = np.where(np.abs(out) < 1e-15, 0.0, out)
    out.setflags(write=False)
    return out


def real_cg_other_part(l1: int, l2: int, l3: int) -> np.ndarray:
    """The discarded part (imaginary for even sums, real for odd): must vanish."""
    cg = _cg_block_complex(l1, l2, l3)
    U1, U2, U3 = complex_to_real(l1), complex_to_real(l2), complex_to_real(l3)
    C = np.einsum("ai,bj,ck,ijk->abc", U1, U2, U3.conj(), cg)
    return C.imag if (l1 + l2 + l3) % 2 == 0 else C.real
