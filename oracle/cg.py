"""Real Clebsch-Gordan blocks, exact to the last double (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages call the coupling tensor a block-sparse tensor whose blocks are
themselves sparse, more so at higher order, with repeated identical blocks
(sciencestack.ai page, Figures 1-2).  They do not print the coefficients, the
real basis or the normalisation.  The readings used here:

1. complex CG <j1 m1 j2 m2 | J M> from Racah's closed form (Condon-Shortley
   phase), evaluated exactly with ``fractions.Fraction``; one square root at
   the end, taken in 60-digit decimal arithmetic;
2. real basis: real = Q_l . complex with, for rows m = -l..l,
   m > 0:  Q[m,-m] = 1/sqrt2,  Q[m,m] = (-1)^m/sqrt2;
   m < 0:  Q[m,m] = i/sqrt2,   Q[m,-m] = -i(-1)^m/sqrt2;
   m = 0:  Q[0,0] = 1            (so l=1 is ordered (y, z, x));
   C[i,j,k] = sum conj(Q1[i,m1]) conj(Q2[j,m2]) Q3[k,m3] <l1 m1 l2 m2|l3 m3>;
   this is purely real (l1+l2+l3 even) or purely imaginary (odd): keep the
   non-zero part;
3. normalise every block to Frobenius norm 1;
4. sign: the first entry in row-major (i, j, k) order with |C| > 1e-9 is
   made positive;
5. entries with |C| <= 1e-9 are structural zeros.
"""
from decimal import Decimal, getcontext
from fractions import Fraction
from functools import lru_cache
from math import factorial

import numpy as np

ZERO_TOL = 1e-9


def _fact(n: int) -> int:
    return factorial(n)


def cg_complex_squared_sign(j1, m1, j2, m2, J, M):
    """Return (sign, value**2) of <j1 m1 j2 m2|J M> as exact rationals (Racah 1942)."""
    if M != m1 + m2 or J < abs(j1 - j2) or J > j1 + j2 or abs(m1) > j1 or abs(m2) > j2 or abs(M) > J:
        return 0, Fraction(0)
    pref = Fraction((2 * J + 1) * _fact(J + j1 - j2) * _fact(J - j1 + j2) * _fact(j1 + j2 - J),
                    _fact(j1 + j2 + J + 1))
    pref *= (_fact(J + M) * _fact(J - M) * _fact(j1 - m1) * _fact(j1 + m1)
             * _fact(j2 - m2) * _fact(j2 + m2))
    s = Fraction(0)
    for k in range(0, j1 + j2 + J + 1):
        args = (k, j1 + j2 - J - k, j1 - m1 - k, j2 + m2 - k, J - j2 + m1 + k, J - j1 - m2 + k)
        if min(args) < 0:
            continue
        den = 1
        for a in args:
            den *= _fact(a)
        s += Fraction((-1) ** k, den)
    if s == 0:
        return 0, Fraction(0)
    return (1 if s > 0 else -1), pref * s * s


def _sqrt_fraction(q: Fraction) -> float:
    getcontext().prec = 60
    return float((Decimal(q.numerator) / Decimal(q.denominator)).sqrt())


def cg_complex(j1, m1, j2, m2, J, M) -> float:
    sgn, sq = cg_complex_squared_sign(j1, m1, j2, m2, J, M)
    return 0.0 if sgn == 0 else sgn * _sqrt_fraction(sq)


def real_basis_q(l: int) -> np.ndarray:
    """Q_l with real_SH = Q_l @ complex_SH; rows and columns indexed m = -l..l."""
    q = np.zeros((2 * l + 1, 2 * l + 1), dtype=complex)
    r = 1.0 / np.sqrt(2.0)
    for m in range(-l, l + 1):
        row = m + l
        if m > 0:
            q[row, -m + l] = r
            q[row, m + l] = (-1) ** m * r
        elif m < 0:
            q[row, m + l] = 1j * r
            q[row, -m + l] = -1j * (-1) ** m * r
        else:
            q[row, l] = 1.0
    return q


@lru_cache(maxsize=None)
def real_cg_block(l1: int, l2: int, l3: int) -> np.ndarray:
    """The (2l1+1, 2l2+1, 2l3+1) real CG block, Frobenius norm 1, sign-fixed."""
    if l3 < abs(l1 - l2) or l3 > l1 + l2:
        raise ValueError("triangle rule violated")
    cc = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    for m1 in range(-l1, l1 + 1):
        for m2 in range(-l2, l2 + 1):
            m3 = m1 + m2
            if abs(m3) <= l3:
                cc[m1 + l1, m2 + l2, m3 + l3] = cg_complex(l1, m1, l2, m2, l3, m3)
    q1, q2, q3 = real_basis_q(l1), real_basis_q(l2), real_basis_q(l3)
    c = np.einsum("ia,jb,kc,abc->ijk", q1.conj(), q2.conj(), q3, cc)
    part = c.real if (l1 + l2 + l3) % 2 == 0 else c.imag
    part = part / np.linalg.norm(part)
    part[np.abs(part) <= ZERO_TOL] = 0.0
    flat = part.reshape(-1)
    first = flat[np.nonzero(np.abs(flat) > ZERO_TOL)[0][0]]
    if first < 0:
        part = -part
    part.setflags(write=False)
    return part


def nonzeros(l1: int, l2: int, l3: int):
    """List of (i, j, k, value) of the real block, row-major order."""
    c = real_cg_block(l1, l2, l3)
    idx = np.argwhere(np.abs(c) > ZERO_TOL)
    return [(int(i), int(j), int(k), float(c[i, j, k])) for i, j, k in idx]
