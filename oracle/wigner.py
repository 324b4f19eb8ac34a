"""Real Wigner D matrices in the harmonics' own basis (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The networks the pages accelerate are built to keep geometric relations
between inputs and outputs (sciencestack.ai page, Abstract): rotating the
inputs rotates the outputs.  To test that, D_l(R) is obtained here as the
least-squares solution of  Y_l(R r_q) = D_l(R) Y_l(r_q)  over 4l+8 random
unit vectors r_q, which is exact up to rounding because the real harmonics of
degree l span an irreducible representation.  For an irrep of parity p and
an improper rotation -R the matrix is p * D_l(R).
"""
import numpy as np

from .sh import real_sh


def random_rotation(rng: np.random.Generator) -> np.ndarray:
    q, r = np.linalg.qr(rng.standard_normal((3, 3)))
    q = q @ np.diag(np.sign(np.diag(r)))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q


def wigner_d(l: int, rot: np.ndarray, rng: np.random.Generator = None) -> np.ndarray:
    """(2l+1, 2l+1) real matrix with Y_l(rot @ r) = D @ Y_l(r)."""
    rng = np.random.default_rng(12345) if rng is None else rng
    pts = rng.standard_normal((4 * l + 8, 3))
    a = real_sh(l, pts)                 # (q, 2l+1)
    b = real_sh(l, pts @ rot.T)         # (q, 2l+1)
    # b = a @ D^T  ->  D^T = lstsq(a, b)
    dt, *_ = np.linalg.lstsq(a, b, rcond=None)
    return dt.T


def irreps_d(irreps, rot: np.ndarray, improper: bool = False) -> np.ndarray:
    """Block-diagonal D for a list of oracle.irreps.Irrep (channel-major blocks)."""
    dim = sum(ir.dim for ir in irreps)
    d = np.zeros((dim, dim))
    off = 0
    for ir in irreps:
        dl = wigner_d(ir.l, rot)
        if improper:
            dl = ir.p * dl
        n = 2 * ir.l + 1
        for u in range(ir.mul):
            d[off + u * n: off + (u + 1) * n, off + u * n: off + (u + 1) * n] = dl
        off += ir.dim
    return d
