"""Pins of the oracle's real spherical harmonics (oracle/sh.py) and Wigner D (oracle/wigner.py)."""
import numpy as np
import pytest

from oracle import sh, wigner


@pytest.fixture(scope="module")
def pts():
    return np.random.default_rng(3).standard_normal((64, 3))


def test_closed_forms_l1_l2(pts):
    """G6: Y_1 = sqrt3 (y, z, x); Y_2 = (sqrt15 xy, sqrt15 yz, sqrt5/2 (3z^2-1), sqrt15 xz, sqrt15/2 (x^2-y^2))."""
    v = pts / np.linalg.norm(pts, axis=1, keepdims=True)
    x, y, z = v.T
    assert np.allclose(sh.real_sh(0, pts), 1.0, atol=1e-15)
    assert np.allclose(sh.real_sh(1, pts), np.sqrt(3) * np.stack([y, z, x], 1), atol=1e-14)
    y2 = np.stack([np.sqrt(15) * x * y, np.sqrt(15) * y * z, np.sqrt(5) / 2 * (3 * z * z - 1),
                   np.sqrt(15) * x * z, np.sqrt(15) / 2 * (x * x - y * y)], 1)
    assert np.allclose(sh.real_sh(2, pts), y2, atol=1e-14)


def test_component_norm_and_parity(pts):
    for l in range(8):
        yl = sh.real_sh(l, pts)
        assert np.allclose(np.sum(yl * yl, axis=1), 2 * l + 1, atol=1e-12)
        assert np.allclose(sh.real_sh(l, -pts), (-1) ** l * yl, atol=1e-12)
        # scale invariance: harmonics of the direction
        assert np.allclose(sh.real_sh(l, 3.7 * pts), yl, atol=1e-12)


def test_complex_sh_matches_scipy(pts):
    """The complex harmonics equal scipy's (a library routine with the same phase convention)."""
    from scipy.special import sph_harm_y
    v = pts / np.linalg.norm(pts, axis=1, keepdims=True)
    theta = np.arccos(np.clip(v[:, 2], -1, 1))
    phi = np.arctan2(v[:, 1], v[:, 0])
    for l in range(8):
        ours = sh.complex_sh(l, pts)
        for m in range(-l, l + 1):
            ref = sph_harm_y(l, m, theta, phi)
            assert np.allclose(ours[:, m + l], ref, atol=1e-12), (l, m)


def test_real_sh_orthogonality_on_sphere():
    """Integral of Y_lm Y_l'm' over the sphere is 4pi delta (component normalisation).

    Gauss-Legendre in cos(theta) times a uniform grid in phi integrates the
    products exactly for degrees below the grid order."""
    n = 20
    ct, wt = np.polynomial.legendre.leggauss(n)
    phi = np.arange(2 * n) * np.pi / n
    st = np.sqrt(1 - ct ** 2)
    pts = np.stack([np.outer(st, np.cos(phi)), np.outer(st, np.sin(phi)),
                    np.outer(ct, np.ones_like(phi))], -1).reshape(-1, 3)
    wts = np.outer(wt, np.full(2 * n, np.pi / n)).reshape(-1)
    ys = sh.real_sh_all(7, pts)
    gram = ys.T @ (ys * wts[:, None])
    assert np.allclose(gram, 4 * np.pi * np.eye(64), atol=1e-11)


def test_wigner_d_orthogonal_and_l1():
    """G7: D_l(R) is orthogonal, D_l(R1 R2) = D_l(R1) D_l(R2), and D_1 = Pi R Pi^T with Pi = (y,z,x)."""
    rng = np.random.default_rng(11)
    r1, r2 = wigner.random_rotation(rng), wigner.random_rotation(rng)
    perm = np.array([[0, 1, 0], [0, 0, 1], [1, 0, 0]], dtype=float)
    assert np.allclose(wigner.wigner_d(1, r1), perm @ r1 @ perm.T, atol=1e-12)
    for l in range(8):
        d1, d2 = wigner.wigner_d(l, r1), wigner.wigner_d(l, r2)
        assert np.allclose(d1 @ d1.T, np.eye(2 * l + 1), atol=1e-11)
        assert np.allclose(wigner.wigner_d(l, r1 @ r2), d1 @ d2, atol=1e-10)
        pts = rng.standard_normal((10, 3))
        assert np.allclose(sh.real_sh(l, pts @ r1.T), sh.real_sh(l, pts) @ d1.T, atol=1e-11)
