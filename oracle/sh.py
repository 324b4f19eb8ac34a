"""Real spherical harmonics with component normalisation (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The edge features of the graph convolution are the spherical harmonics of the
edge direction (sciencestack.ai page, Figure 4B: node features combined with
edge features; the fused-convolution north star names Y(r_ij)).  The pages fix
no convention; the reading here is

    Y_l^real(r) = sqrt(4 pi) * Q_l @ Y_l^complex(r / |r|)

with Q_l the real-basis matrix of ``oracle.cg`` and Y_l^complex the standard
orthonormal harmonics with the Condon-Shortley phase.  Then
sum_m (Y_lm^real)^2 = 2l+1 and Y_1 = sqrt3 (y, z, x).

The complex harmonics are written from their textbook definition: Legendre
polynomials from the explicit binomial sum, the associated functions by
differentiating that polynomial m times, times e^{i m phi}.
"""
from fractions import Fraction
from math import comb, factorial, pi, sqrt

import numpy as np

from .cg import real_basis_q


def _legendre_coeffs(l: int):
    """Exact coefficients c[n] of P_l(x) = sum_n c[n] x^n."""
    c = [Fraction(0)] * (l + 1)
    for k in range(l // 2 + 1):
        c[l - 2 * k] += Fraction((-1) ** k * comb(l, k) * comb(2 * l - 2 * k, l), 2 ** l)
    return c


def _derivative(c, m: int):
    for _ in range(m):
        c = [c[n] * n for n in range(1, len(c))] or [Fraction(0)]
    return c


def _poly_eval(c, x):
    acc = np.zeros_like(x)
    for coef in reversed(c):
        acc = acc * x + float(coef)
    return acc


def complex_sh(l: int, vec: np.ndarray) -> np.ndarray:
    """Orthonormal complex Y_l^m for m = -l..l, Condon-Shortley phase; shape (n, 2l+1)."""
    v = np.asarray(vec, dtype=np.float64)
    v = v / np.linalg.norm(v, axis=-1, keepdims=True)
    x, y, z = v[..., 0], v[..., 1], v[..., 2]
    rho = np.hypot(x, y)
    phi = np.arctan2(y, x)
    out = np.zeros(v.shape[:-1] + (2 * l + 1,), dtype=complex)
    pl = _legendre_coeffs(l)
    for m in range(0, l + 1):
        norm = sqrt((2 * l + 1) / (4 * pi) * factorial(l - m) / factorial(l + m))
        assoc = rho ** m * _poly_eval(_derivative(pl, m), z)  # no Condon-Shortley factor yet
        ylm = (-1) ** m * norm * assoc * np.exp(1j * m * phi)
        out[..., l + m] = ylm
        if m > 0:
            out[..., l - m] = (-1) ** m * np.conj(ylm)
    return out


def real_sh(l: int, vec: np.ndarray) -> np.ndarray:
    """Component-normalised real harmonics of degree l; shape (n, 2l+1)."""
    yc = complex_sh(l, vec)
    yr = np.sqrt(4 * pi) * np.einsum("km,...m->...k", real_basis_q(l), yc)
    return yr.real.copy()


def real_sh_all(lmax: int, vec: np.ndarray) -> np.ndarray:
    """Concatenation l = 0..lmax, i.e. the layout of the irreps 1x0e+1x1o+...; shape (n, (lmax+1)^2)."""
    return np.concatenate([real_sh(l, vec) for l in range(lmax + 1)], axis=-1)
