"""Pins for oracle.cg: Racah CG, real tables, selection rules.

Pinned against things other than the oracle itself: the two orthogonality
relations, textbook special values, an independent closed form for
<l1 0 l2 0 | L 0>, sympy's CG routine, rotation equivariance with Wigner
matrices fitted from the spherical harmonics, the Gaunt identity that ties the
table basis to the harmonic basis, and the closed forms of the 1 x 1 couplings
(the antisymmetric cross product of "The Price of Freedom", Key results).
"""
import math
import itertools

import numpy as np
import pytest

from oracle import cg, sh

LMAX = 3


def all_triples(lmax=LMAX):
    for l1, l2 in itertools.product(range(lmax + 1), repeat=2):
        for l3 in range(abs(l1 - l2), min(l1 + l2, lmax) + 1):
            yield l1, l2, l3


def test_cg_orthogonality_first_relation():
    # sum_{m1,m2} <j1 m1 j2 m2|J M><j1 m1 j2 m2|J' M'> = delta_JJ' delta_MM'
    for j1, j2 in itertools.product(range(LMAX + 1), repeat=2):
        Js = range(abs(j1 - j2), j1 + j2 + 1)
        for J, Jp in itertools.product(Js, Js):
            for M in range(-J, J + 1):
                for Mp in range(-Jp, Jp + 1):
                    s = sum(cg.cg_complex(j1, m1, j2, m2, J, M) * cg.cg_complex(j1, m1, j2, m2, Jp, Mp)
                            for m1 in range(-j1, j1 + 1) for m2 in range(-j2, j2 + 1))
                    assert abs(s - (J == Jp and M == Mp)) < 1e-14


def test_cg_orthogonality_second_relation():
    # sum_{J,M} <j1 m1 j2 m2|J M><j1 m1' j2 m2'|J M> = delta_m1m1' delta_m2m2'
    for j1, j2 in itertools.product(range(LMAX + 1), repeat=2):
        ms = [(a, b) for a in range(-j1, j1 + 1) for b in range(-j2, j2 + 1)]
        for (m1, m2), (n1, n2) in itertools.product(ms, ms):
            s = sum(cg.cg_complex(j1, m1, j2, m2, J, M) * cg.cg_complex(j1, n1, j2, n2, J, M)
                    for J in range(abs(j1 - j2), j1 + j2 + 1) for M in range(-J, J + 1))
            assert abs(s - ((m1, m2) == (n1, n2))) < 1e-14


def test_cg_special_values():
    for l in range(5):
        for m in range(-l, l + 1):
            assert cg.cg_complex(l, m, 0, 0, l, m) == pytest.approx(1.0, abs=1e-15)
    for m in (-1, 0, 1):
        assert cg.cg_complex(1, m, 1, -m, 0, 0) == pytest.approx((-1) ** (1 - m) / math.sqrt(3), abs=1e-15)


def cg_m0_closed_form(l1, l2, L):
    """<l1 0 l2 0 | L 0>: zero for odd l1+l2+L, else with J = l1+l2+L, g = J/2:
    (-1)^(g-L) sqrt(2L+1) g!/((g-l1)!(g-l2)!(g-L)!) sqrt((J-2l1)!(J-2l2)!(J-2L)!/(J+1)!)."""
    J = l1 + l2 + L
    if J % 2:
        return 0.0
    g = J // 2
    f = math.factorial
    return ((-1) ** (g - L) * math.sqrt(2 * L + 1) * f(g) / (f(g - l1) * f(g - l2) * f(g - L))
            * math.sqrt(f(J - 2 * l1) * f(J - 2 * l2) * f(J - 2 * L) / f(J + 1)))


def test_cg_m0_closed_form():
    for l1, l2, l3 in all_triples(4):
        assert cg.cg_complex(l1, 0, l2, 0, l3, 0) == pytest.approx(cg_m0_closed_form(l1, l2, l3), abs=1e-14)


def test_cg_matches_sympy():
    from sympy.physics.quantum.cg import CG

    for l1, l2, l3 in all_triples():
        for m1 in range(-l1, l1 + 1):
            for m2 in range(-l2, l2 + 1):
                m3 = m1 + m2
                if abs(m3) > l3:
                    continue
                ref = float(CG(l1, m1, l2, m2, l3, m3).doit())
                assert cg.cg_complex(l1, m1, l2, m2, l3, m3) == pytest.approx(ref, abs=1e-14)


def test_real_tables_real_and_orthonormal():
    for l1, l2, l3 in all_triples():
        assert np.abs(cg.real_cg_other_part(l1, l2, l3)).max() < 1e-14
        C = cg.real_cg(l1, l2, l3)
        G = np.einsum("abc,abd->cd", C, C)
        assert np.abs(G - np.eye(2 * l3 + 1)).max() < 1e-14


def wigner_from_sh(l, rot, rng):
    """Fit D^l(rot) from Y_l(rot r) = D^l Y_l(r) over random directions."""
    pts = rng.normal(size=(4 * l + 8, 3))
    Y = sh.sh_single_l(l, pts)
    Yr = sh.sh_single_l(l, pts @ rot.T)
    Dt, *_ = np.linalg.lstsq(Y, Yr, rcond=None)
    return Dt.T


def random_rotation(rng):
    q, r = np.linalg.qr(rng.normal(size=(3, 3)))
    q = q * np.sign(np.diag(r))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


def test_real_tables_equivariant():
    rng = np.random.default_rng(7)
    for _ in range(3):
        rot = random_rotation(rng)
        D = [wigner_from_sh(l, rot, rng) for l in range(LMAX + 1)]
        for l in range(LMAX + 1):
            assert np.abs(D[l] @ D[l].T - np.eye(2 * l + 1)).max() < 1e-12
        for l1, l2, l3 in all_triples():
            C = cg.real_cg(l1, l2, l3)
            rotated = np.einsum("ai,bj,ck,ijk->abc", D[l1], D[l2], D[l3], C)
            assert np.abs(rotated - C).max() < 1e-12, (l1, l2, l3)


def test_gaunt_identity_ties_tables_to_harmonics():
    # sum C[m1,m2,m3] Y_l1[m1] Y_l2[m2] = alpha Y_l3[m3] for even paths,
    # alpha = sqrt((2l1+1)(2l2+1)/(2l3+1)) <l1 0 l2 0|l3 0>
    rng = np.random.default_rng(3)
    pts = rng.normal(size=(20, 3))
    for l1, l2, l3 in all_triples():
        if (l1 + l2 + l3) % 2:
            continue
        C = cg.real_cg(l1, l2, l3)
        lhs = np.einsum("abc,ea,eb->ec", C, sh.sh_single_l(l1, pts), sh.sh_single_l(l2, pts))
        alpha = math.sqrt((2 * l1 + 1) * (2 * l2 + 1) / (2 * l3 + 1)) * cg_m0_closed_form(l1, l2, l3)
        assert np.abs(lhs - alpha * sh.sh_single_l(l3, pts)).max() < 1e-12, (l1, l2, l3)
    # the printed constants for the first few paths
    expected = {(1, 1, 0): -math.sqrt(3), (1, 1, 2): math.sqrt(6 / 5), (2, 2, 0): math.sqrt(5),
                (1, 2, 1): -math.sqrt(2), (2, 2, 2): -math.sqrt(10 / 7)}
    for (l1, l2, l3), a in expected.items():
        alpha = math.sqrt((2 * l1 + 1) * (2 * l2 + 1) / (2 * l3 + 1)) * cg_m0_closed_form(l1, l2, l3)
        assert alpha == pytest.approx(a, rel=1e-14)


def test_closed_forms_small_couplings():
    for l in range(LMAX + 1):
        C = cg.real_cg(0, l, l)
        assert np.abs(C[0] - np.eye(2 * l + 1)).max() < 1e-15
        C = cg.real_cg(l, 0, l)
        assert np.abs(C[:, 0, :] - np.eye(2 * l + 1)).max() < 1e-15
    # 1 x 1 -> 0 : -dot / sqrt3
    assert np.abs(cg.real_cg(1, 1, 0)[:, :, 0] + np.eye(3) / math.sqrt(3)).max() < 1e-15
    # 1 x 1 -> 1 (odd sum): C[a,b,c] = -eps_abc / sqrt2 in (y, z, x) labels
    eps = np.zeros((3, 3, 3))
    for (a, b, c), s in {(0, 1, 2): 1, (1, 2, 0): 1, (2, 0, 1): 1,
                         (0, 2, 1): -1, (2, 1, 0): -1, (1, 0, 2): -1}.items():
        eps[a, b, c] = s
    C = cg.real_cg(1, 1, 1)
    assert np.abs(C + eps / math.sqrt(2)).max() < 1e-15
    a, b = np.array([0.3, -1.2, 0.7]), np.array([1.1, 0.4, -0.5])
    coupled = np.einsum("abc,a,b->c", C, a, b)
    assert np.abs(coupled + np.cross(a, b) / math.sqrt(2)).max() < 1e-15
    assert np.abs(np.einsum("abc,a,b->c", C, b, a) + coupled).max() < 1e-15   # antisymmetric


def natural(lmax, mul=1):
    return [(mul, l, 1 if l % 2 == 0 else -1) for l in range(lmax + 1)]


def test_path_enumeration_counts_and_brute_force():
    nnz_expected = {1: 10, 2: 83, 3: 353}
    m3_expected = {1: 8, 2: 35, 3: 99}
    p_expected = {1: 4, 2: 11, 3: 23}
    for L in (1, 2, 3):
        paths = cg.enumerate_paths(natural(L), L, natural(L))
        assert len(paths) == p_expected[L]
        assert sum(2 * p["l3"] + 1 for p in paths) == m3_expected[L]
        assert sum(2 * p["l1"] + 1 for p in paths) == m3_expected[L]
        nnz = sum(int((np.abs(cg.real_cg(p["l1"], p["l2"], p["l3"])) > 1e-14).sum()) for p in paths)
        assert nnz == nnz_expected[L]
    # brute force over mixed parities: a path exists iff some complex CG in its block
    # is nonzero and the parities multiply correctly
    ir_in = [(1, 0, 1), (1, 1, -1), (1, 1, 1), (1, 2, 1)]
    ir_out = [(1, 0, 1), (1, 0, -1), (1, 1, -1), (1, 1, 1), (1, 2, 1), (1, 2, -1), (1, 3, -1)]
    got = {(p["i1"], p["l2"], p["i3"]) for p in cg.enumerate_paths(ir_in, 2, ir_out)}
    want = set()
    for i1, (_, l1, p1) in enumerate(ir_in):
        for l2 in range(3):
            for i3, (_, l3, p3) in enumerate(ir_out):
                nz = any(abs(cg.cg_complex(l1, m1, l2, m2, l3, m1 + m2)) > 0
                         for m1 in range(-l1, l1 + 1) for m2 in range(-l2, l2 + 1) if abs(m1 + m2) <= l3)
                if nz and p1 * (-1) ** l2 == p3:
                    want.add((i1, l2, i3))
    assert got == want
    paths = cg.enumerate_paths(ir_in, 2, ir_out)
    assert [(p["i1"], p["l2"], p["i3"]) for p in paths] == sorted(got)


def test_parse_irreps():
    assert cg.parse_irreps("32x0e+32x1o+32x2e") == [(32, 0, 1), (32, 1, -1), (32, 2, 1)]
    assert cg.parse_irreps("0e + 2x1e") == [(1, 0, 1), (2, 1, 1)]
    with pytest.raises(ValueError):
        cg.parse_irreps("8x1q")
