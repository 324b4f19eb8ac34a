"""Pins of the oracle's real CG blocks (oracle/cg.py) against mathematics.

Each test ties the oracle to something other than itself: a textbook table, a
library routine (sympy), closed forms, orthogonality, and the coupling of real
spherical harmonics (Gaunt).  The pages print no coefficient; see the
readings in oracle/cg.py.
"""
import itertools
import os
from math import factorial, sqrt

import numpy as np
import pytest

from oracle import cg, sh

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def triples(lmax):
    for l1, l2 in itertools.product(range(lmax + 1), repeat=2):
        for l3 in range(abs(l1 - l2), min(l1 + l2, lmax) + 1):
            yield l1, l2, l3


def test_complex_cg_textbook_table():
    path = os.path.join(GOLDEN, "cg_textbook_1x1.txt")
    n = 0
    for line in open(path):
        if not line.strip() or line.startswith("#"):
            continue
        j1, m1, j2, m2, J, M, expr = line.split(None, 6)
        want = eval(expr, {"sqrt": sqrt})
        got = cg.cg_complex(int(j1), int(m1), int(j2), int(m2), int(J), int(M))
        assert abs(got - want) < 1e-15, line
        n += 1
    assert n == 18


def test_complex_cg_matches_sympy():
    from sympy.physics.quantum.cg import CG
    rng = np.random.default_rng(1)
    cases = list(itertools.product(range(4), range(4)))
    for j1, j2 in cases:
        for J in range(abs(j1 - j2), j1 + j2 + 1):
            for m1 in range(-j1, j1 + 1):
                for m2 in range(-j2, j2 + 1):
                    if abs(m1 + m2) > J:
                        continue
                    want = float(CG(j1, m1, j2, m2, J, m1 + m2).doit())
                    assert abs(cg.cg_complex(j1, m1, j2, m2, J, m1 + m2) - want) < 1e-14
    # a few high-l entries up to l = 7
    for _ in range(25):
        j1, j2 = rng.integers(4, 8, 2)
        J = int(rng.integers(abs(j1 - j2), min(j1 + j2, 7) + 1))
        m1 = int(rng.integers(-j1, j1 + 1))
        m2 = int(rng.integers(max(-j2, -J - m1), min(j2, J - m1) + 1))
        want = float(CG(int(j1), m1, int(j2), m2, J, m1 + m2).doit())
        assert abs(cg.cg_complex(int(j1), m1, int(j2), m2, J, m1 + m2) - want) < 1e-14


@pytest.mark.parametrize("lmax", [7])
def test_orthogonality_and_completeness(lmax):
    """G1: M^T M = I/(2l3+1); distinct l3 orthogonal; the stacked sqrt(2l3+1) C is orthogonal."""
    for l1, l2 in itertools.product(range(lmax + 1), repeat=2):
        n12 = (2 * l1 + 1) * (2 * l2 + 1)
        blocks = []
        for l3 in range(abs(l1 - l2), l1 + l2 + 1):
            m = cg.real_cg_block(l1, l2, l3).reshape(n12, 2 * l3 + 1)
            assert np.allclose(m.T @ m, np.eye(2 * l3 + 1) / (2 * l3 + 1), atol=1e-14)
            blocks.append(np.sqrt(2 * l3 + 1) * m)
        full = np.concatenate(blocks, axis=1)
        assert full.shape == (n12, n12)
        assert np.allclose(full.T @ full, np.eye(n12), atol=1e-13)
        assert np.allclose(full @ full.T, np.eye(n12), atol=1e-13)


def test_special_cases():
    """G2: (l,0,l), (0,l,l), (l,l,0) are +I/sqrt(2l+1); (1,1,1) = eps/sqrt6 in (y,z,x) order."""
    for l in range(8):
        n = 2 * l + 1
        eye = np.eye(n) / np.sqrt(n)
        assert np.allclose(cg.real_cg_block(l, 0, l)[:, 0, :], eye, atol=1e-15)
        assert np.allclose(cg.real_cg_block(0, l, l)[0, :, :], eye, atol=1e-15)
        assert np.allclose(cg.real_cg_block(l, l, 0)[:, :, 0], eye, atol=1e-15)
    eps = np.zeros((3, 3, 3))
    for (i, j, k), s in {(0, 1, 2): 1, (1, 2, 0): 1, (2, 0, 1): 1,
                         (0, 2, 1): -1, (2, 1, 0): -1, (1, 0, 2): -1}.items():
        eps[i, j, k] = s
    assert np.allclose(cg.real_cg_block(1, 1, 1), eps / np.sqrt(6), atol=1e-15)


def _cg_m0_closed_form(l1, l2, L):
    """<l1 0 l2 0 | L 0> from its closed form (zero for odd l1+l2+L)."""
    J = l1 + l2 + L
    if J % 2:
        return 0.0
    g = J // 2
    v = sqrt(2 * L + 1) * sqrt(factorial(J - 2 * l1) * factorial(J - 2 * l2) * factorial(J - 2 * L)
                              / factorial(J + 1))
    v *= factorial(g) / (factorial(g - l1) * factorial(g - l2) * factorial(g - L))
    return (-1) ** (g - L) * v


def test_sh_coupling_gaunt():
    """G3: sum_ij C_ijk Y_i Y_j = c Y_k with |c| = sqrt((2l1+1)(2l2+1)) |<l1 0 l2 0|l3 0>| / (2l3+1)."""
    rng = np.random.default_rng(7)
    pts = rng.standard_normal((40, 3))
    for l1, l2, l3 in triples(7):
        c = cg.real_cg_block(l1, l2, l3)
        lhs = np.einsum("ijk,ni,nj->nk", c, sh.real_sh(l1, pts), sh.real_sh(l2, pts))
        y3 = sh.real_sh(l3, pts)
        want = sqrt((2 * l1 + 1) * (2 * l2 + 1)) * abs(_cg_m0_closed_form(l1, l2, l3)) / (2 * l3 + 1)
        if (l1 + l2 + l3) % 2:
            assert np.abs(lhs).max() < 1e-12
            continue
        coef = float(np.sum(lhs * y3) / np.sum(y3 * y3))
        assert np.abs(lhs - coef * y3).max() < 1e-11
        assert abs(abs(coef) - want) < 1e-12
    # sign of the simplest coupling follows from the special case (1,1,0) = +I/sqrt3: Y1.Y1 = 3
    c = cg.real_cg_block(1, 1, 0)
    v = sh.real_sh(1, pts)
    assert np.allclose(np.einsum("ijk,ni,nj->nk", c, v, v), np.sqrt(3.0), atol=1e-13)


# Signed coupling constants c of sum_ij C_ijk Y_l1,i(r) Y_l2,j(r) = c Y_l3,k(r) under the real basis
# and first-nonzero-positive sign rule (values to 12 decimals; e.g. (1,1,2) = -sqrt(6)/5,
# (2,2,2) = -sqrt(2/7), (1,2,3) = -3/7, (7,7,0) = sqrt(15)).  A sign error in the basis change or
# the sign rule of either the CG block or the harmonics flips one of these.
GAUNT_SIGNED = {
    (1, 1, 0): 1.732050807569, (1, 1, 2): -0.489897948557, (2, 2, 0): 2.236067977500,
    (2, 2, 2): -0.534522483825, (1, 2, 1): 0.816496580928, (1, 2, 3): -0.428571428571,
    (2, 2, 4): 0.398409536445, (3, 3, 2): -0.611010092661, (7, 7, 0): 3.872983346207,
}


@pytest.mark.parametrize("triple", sorted(GAUNT_SIGNED))
def test_sh_coupling_signed_constants(triple):
    """G3 with signs: the coupling constant itself, not only its magnitude."""
    l1, l2, l3 = triple
    pts = np.random.default_rng(11).standard_normal((40, 3))
    lhs = np.einsum("ijk,ni,nj->nk", cg.real_cg_block(l1, l2, l3), sh.real_sh(l1, pts), sh.real_sh(l2, pts))
    y3 = sh.real_sh(l3, pts)
    coef = float(np.sum(lhs * y3) / np.sum(y3 * y3))
    assert np.abs(lhs - coef * y3).max() < 1e-11
    assert abs(coef - GAUNT_SIGNED[triple]) < 1e-11


def test_swap_symmetry():
    """G4: C^{l2 l1 l3}[j,i,k] = +-C^{l1 l2 l3}[i,j,k]."""
    for l1, l2, l3 in triples(6):
        a = cg.real_cg_block(l1, l2, l3)
        b = cg.real_cg_block(l2, l1, l3).transpose(1, 0, 2)
        assert np.allclose(a, b, atol=1e-14) or np.allclose(a, -b, atol=1e-14)


def test_real_or_imaginary_rule():
    """G5: the transformed block is purely real iff l1+l2+l3 is even, else purely imaginary."""
    for l1, l2, l3 in triples(7):
        cc = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
        for m1 in range(-l1, l1 + 1):
            for m2 in range(-l2, l2 + 1):
                if abs(m1 + m2) <= l3:
                    cc[m1 + l1, m2 + l2, m1 + m2 + l3] = cg.cg_complex(l1, m1, l2, m2, l3, m1 + m2)
        t = np.einsum("ia,jb,kc,abc->ijk", cg.real_basis_q(l1).conj(), cg.real_basis_q(l2).conj(),
                      cg.real_basis_q(l3), cc)
        zero = t.imag if (l1 + l2 + l3) % 2 == 0 else t.real
        assert np.abs(zero).max() < 1e-15


def test_sparsity_threshold_and_counts():
    """Structural zeros are far below every nonzero; block sparsity grows with order (Figure 2)."""
    smallest = min(np.abs(c).min() for c in
                   (np.array([v for *_, v in cg.nonzeros(*t)]) for t in triples(7)))
    assert smallest > 1e-3
    counts = {(1, 0, 1): 3, (1, 1, 0): 3, (1, 1, 1): 6, (1, 1, 2): 11, (2, 2, 2): 25, (3, 3, 3): 42,
              (7, 7, 0): 15, (7, 7, 7): 258}
    for t, n in counts.items():
        assert len(cg.nonzeros(*t)) == n
    # the zero fraction grows with order: compare l with l+2 (odd and even l alternate)
    fill = {l: len(cg.nonzeros(l, l, l)) / (2 * l + 1) ** 3 for l in range(1, 8)}
    assert all(fill[l + 2] < fill[l] for l in range(1, 6))
    top = {l: len(cg.nonzeros(l, l, 2 * l)) / ((2 * l + 1) ** 2 * (4 * l + 1)) for l in range(1, 4)}
    assert top[1] > top[2] > top[3]


def test_sign_rule_and_norm():
    for l1, l2, l3 in triples(7):
        c = cg.real_cg_block(l1, l2, l3)
        assert abs(np.linalg.norm(c) - 1.0) < 1e-14
        flat = c.reshape(-1)
        assert flat[np.nonzero(np.abs(flat) > 1e-9)[0][0]] > 0
