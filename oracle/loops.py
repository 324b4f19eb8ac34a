"""ctypes front-end to the explicit-loop oracle in ``cpu_loops.c``.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The nonzero tables come from ``oracle.cg`` and the path table from
``oracle.irreps``: nothing here is shared with the product library.  Inputs
are the caller's arrays (float32 or float64, widened exactly inside the C
code); outputs are float64.
"""
import ctypes
import os
import subprocess

import numpy as np

from .cg import nonzeros
from .irreps import Problem, offsets

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cpu_loops.c")
_LIB = os.path.join(_HERE, "libcpu_loops.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile cpu_loops.c with gcc -O2 -fopenmp into oracle/libcpu_loops.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
    return _lib


def default_threads() -> int:
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


class Tables:
    """Path table and CG nonzeros of a Problem, in the layout cpu_loops.c reads."""

    FIELDS = 11

    def __init__(self, prob: Problem):
        oa, ob, oo = offsets(prob.ins), offsets(prob.sh), offsets(prob.out)
        rows, nzi, nzj, nzk, nzc = [], [], [], [], []
        for p in prob.paths:
            nz = nonzeros(p.l1, p.l2, p.l3)
            rows.append([oa[p.i1], ob[p.i2], oo[p.slot], 2 * p.l1 + 1, 2 * p.l2 + 1, 2 * p.l3 + 1,
                         prob.ins[p.i1].mul, prob.out[p.slot].mul, p.w_off, len(nzi), len(nz)])
            for i, j, k, c in nz:
                nzi.append(i)
                nzj.append(j)
                nzk.append(k)
                nzc.append(c)
        self.prob = prob
        self.n_paths = len(prob.paths)
        self.pt = np.ascontiguousarray(np.array(rows, dtype=np.int32).reshape(-1))
        self.nzi = np.array(nzi, dtype=np.int32)
        self.nzj = np.array(nzj, dtype=np.int32)
        self.nzk = np.array(nzk, dtype=np.int32)
        self.nzc = np.array(nzc, dtype=np.float64)

    def head(self):
        return (ctypes.c_int(self.n_paths), _p(self.pt), _p(self.nzi), _p(self.nzj), _p(self.nzk),
                _p(self.nzc))


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _input(a):
    a = np.ascontiguousarray(a)
    if a.dtype not in (np.float32, np.float64):
        raise TypeError("oracle inputs must be float32 or float64")
    return a


def _same_kind(*arrs):
    f32 = arrs[0].dtype == np.float32
    if any((a.dtype == np.float32) != f32 for a in arrs):
        raise TypeError("oracle inputs must share one dtype")
    return int(f32)


def uvu_forward(tab: Tables, ptr, col, x, y, w, n_threads=None) -> np.ndarray:
    """Per row r of the CSR ``ptr``: sum over its edges of the uvu product (float64 result)."""
    prob = tab.prob
    ptr = np.ascontiguousarray(ptr, dtype=np.int64)
    col = np.ascontiguousarray(col, dtype=np.int64)
    x, y, w = _input(x), _input(y), _input(w)
    f32 = _same_kind(x, y, w)
    n_rows = len(ptr) - 1
    out = np.empty((n_rows, prob.d_out))
    _load().oracle_uvu_forward(*tab.head(), prob.d_in, prob.d_sh, prob.d_out, prob.weight_numel,
                               ctypes.c_int64(n_rows), _p(ptr), _p(col), _p(x), _p(y), _p(w),
                               f32, _p(out), n_threads or default_threads())
    return out


def uvu_backward_edges(tab: Tables, ptr, col, x, y, w, g, n_threads=None):
    """dY and dW of every edge of the rows of ``ptr``; g holds one row per CSR row."""
    prob = tab.prob
    ptr = np.ascontiguousarray(ptr, dtype=np.int64)
    col = np.ascontiguousarray(col, dtype=np.int64)
    x, y, w, g = _input(x), _input(y), _input(w), _input(g)
    f32 = _same_kind(x, y, w, g)
    n_rows = len(ptr) - 1
    n_e = int(ptr[-1])
    dy = np.empty((n_e, prob.d_sh))
    dw = np.empty((n_e, prob.weight_numel))
    _load().oracle_uvu_backward_edges(*tab.head(), prob.d_in, prob.d_sh, prob.d_out,
                                      prob.weight_numel, ctypes.c_int64(n_rows), _p(ptr), _p(col),
                                      _p(x), _p(y), _p(w), _p(g), f32, _p(dy), _p(dw),
                                      n_threads or default_threads())
    return dy, dw


def uvu_backward_x(tab: Tables, sptr, gidx, y, w, g, n_threads=None) -> np.ndarray:
    """dx of each sender row of ``sptr``; y, w rows are in sender order, gidx picks g rows."""
    prob = tab.prob
    sptr = np.ascontiguousarray(sptr, dtype=np.int64)
    gidx = np.ascontiguousarray(gidx, dtype=np.int64)
    y, w, g = _input(y), _input(w), _input(g)
    f32 = _same_kind(y, w, g)
    n_rows = len(sptr) - 1
    dx = np.empty((n_rows, prob.d_in))
    _load().oracle_uvu_backward_x(*tab.head(), prob.d_in, prob.d_sh, prob.d_out, prob.weight_numel,
                                  ctypes.c_int64(n_rows), _p(sptr), _p(gidx), _p(y), _p(w), _p(g),
                                  f32, _p(dx), n_threads or default_threads())
    return dx


def uvw_forward(tab: Tables, x, y, w, n_threads=None) -> np.ndarray:
    prob = tab.prob
    x, y, w = _input(x), _input(y), _input(w)
    f32 = _same_kind(x, y, w)
    n_rows = x.shape[0]
    out = np.empty((n_rows, prob.d_out))
    _load().oracle_uvw_forward(*tab.head(), prob.d_in, prob.d_sh, prob.d_out,
                               ctypes.c_int64(n_rows), _p(x), _p(y), _p(w), f32, _p(out),
                               n_threads or default_threads())
    return out


def uvw_backward(tab: Tables, x, y, w, g, rows, wrows, n_threads=None):
    """uvw batched backward: (dx, dy) of the rows ``rows`` and dW summed over the rows ``wrows``."""
    prob = tab.prob
    x, y, w, g = _input(x), _input(y), _input(w), _input(g)
    f32 = _same_kind(x, y, w, g)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    wrows = np.ascontiguousarray(wrows, dtype=np.int64)
    dx = np.empty((len(rows), prob.d_in))
    dy = np.empty((len(rows), prob.d_sh))
    dw = np.empty(prob.weight_numel)
    rc = _load().oracle_uvw_backward(*tab.head(), prob.d_in, prob.d_sh, prob.d_out,
                                     ctypes.c_int64(prob.weight_numel), ctypes.c_int64(len(rows)), _p(rows),
                                     ctypes.c_int64(len(wrows)), _p(wrows), _p(x), _p(y), _p(w), _p(g), f32,
                                     _p(dx), _p(dy), _p(dw), n_threads or default_threads())
    if rc != 0:
        raise MemoryError("oracle_uvw_backward: allocation failed")
    return dx, dy, dw


# ----------------------------------------------------------------------------------------------
# Convenience wrappers on whole or sampled graphs (index bookkeeping only, no arithmetic).

def conv_forward_rows(tab: Tables, row_ptr, col, x, y, w, rows, n_threads=None) -> np.ndarray:
    """Forward output of the receivers ``rows`` (any subset, any order) of a receiver CSR."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    deg = row_ptr[rows + 1] - row_ptr[rows]
    sub_ptr = np.concatenate([[0], np.cumsum(deg)])
    eidx = np.concatenate([np.arange(row_ptr[r], row_ptr[r + 1]) for r in rows]) if len(rows) else \
        np.zeros(0, np.int64)
    return uvu_forward(tab, sub_ptr, np.asarray(col)[eidx], x, np.asarray(y)[eidx],
                       np.asarray(w)[eidx], n_threads)


def conv_backward_edge_rows(tab: Tables, row_ptr, col, x, y, w, g, rows, n_threads=None):
    """(edge ids, dY, dW) for every edge of the receivers ``rows``."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    deg = row_ptr[rows + 1] - row_ptr[rows]
    sub_ptr = np.concatenate([[0], np.cumsum(deg)])
    eidx = np.concatenate([np.arange(row_ptr[r], row_ptr[r + 1]) for r in rows]) if len(rows) else \
        np.zeros(0, np.int64)
    dy, dw = uvu_backward_edges(tab, sub_ptr, np.asarray(col)[eidx], x, np.asarray(y)[eidx],
                                np.asarray(w)[eidx], np.asarray(g)[rows], n_threads)
    return eidx, dy, dw


def conv_backward_x_rows(tab: Tables, row_ptr, col, y, w, g, senders, n_threads=None) -> np.ndarray:
    """dx of the nodes ``senders``: the oracle's own stable sort of the edges by sender."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col = np.asarray(col, dtype=np.int64)
    senders = np.asarray(senders, dtype=np.int64)
    dst = np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr))
    order = np.argsort(col, kind="stable")
    starts = np.searchsorted(col[order], senders, side="left")
    ends = np.searchsorted(col[order], senders, side="right")
    eidx = np.concatenate([order[a:b] for a, b in zip(starts, ends)]) if len(senders) else \
        np.zeros(0, np.int64)
    sptr = np.concatenate([[0], np.cumsum(ends - starts)])
    gd = dst[eidx]
    uniq, inv = np.unique(gd, return_inverse=True)
    return uvu_backward_x(tab, sptr, inv, np.asarray(y)[eidx], np.asarray(w)[eidx],
                          np.asarray(g)[uniq], n_threads)


def conv_double_backward_rows(tab: Tables, row_ptr, col, x, y, w, g, ggx, ggy, ggw, rows, senders,
                              n_threads=None):
    """Second-order gradients on a sample, from the explicit loops above.

    The convolution is linear in each of x, y, W, so the derivatives of
    L2 = <ggx, dx> + <ggy, dy> + <ggw, dW> are first-order passes with one operand
    replaced by its upstream gradient:
      d/dg = conv(ggx, y, W) + conv(x, ggy, W) + conv(x, y, ggw)        (receivers ``rows``)
      d/dy = dY(ggx, y, W; g) + dY(x, y, ggw; g),  d/dW = dW(ggx, y, W; g) + dW(x, ggy, W; g)
                                                                         (edges of ``rows``)
      d/dx = dx(y -> ggy, W; g) + dx(y, W -> ggw; g)                    (nodes ``senders``)
    Returns (edge ids, dx, dy, dw, dg) with dx for ``senders`` and dg for ``rows``.
    """
    dg = (conv_forward_rows(tab, row_ptr, col, ggx, y, w, rows, n_threads)
          + conv_forward_rows(tab, row_ptr, col, x, ggy, w, rows, n_threads)
          + conv_forward_rows(tab, row_ptr, col, x, y, ggw, rows, n_threads))
    eidx, dy_a, dw_a = conv_backward_edge_rows(tab, row_ptr, col, ggx, y, w, g, rows, n_threads)
    _, _, dw_b = conv_backward_edge_rows(tab, row_ptr, col, x, ggy, w, g, rows, n_threads)
    _, dy_c, _ = conv_backward_edge_rows(tab, row_ptr, col, x, y, ggw, g, rows, n_threads)
    dx = (conv_backward_x_rows(tab, row_ptr, col, ggy, w, g, senders, n_threads)
          + conv_backward_x_rows(tab, row_ptr, col, y, ggw, g, senders, n_threads))
    return eidx, dx, dy_a + dy_c, dw_a + dw_b, dg


def conv_forward_uvw_rows(tab: Tables, row_ptr, col, x, y, w, rows, n_threads=None) -> np.ndarray:
    """uvw convolution output of the receivers ``rows``: the explicit uvw loops on every edge
    of those receivers (x gathered by sender), summed per receiver in CSR edge order."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    deg = row_ptr[rows + 1] - row_ptr[rows]
    eidx = np.concatenate([np.arange(row_ptr[r], row_ptr[r + 1]) for r in rows]) if len(rows) else \
        np.zeros(0, np.int64)
    out = np.zeros((len(rows), tab.prob.d_out))
    if len(eidx) == 0:
        return out
    msg = uvw_forward(tab, np.asarray(x)[np.asarray(col)[eidx]], np.asarray(y)[eidx], w, n_threads)
    seg = np.repeat(np.arange(len(rows)), deg)
    np.add.at(out, seg, msg)
    return out


def conv_forward_radial_rows(tab: Tables, row_ptr, col, x, y, rho, theta, rows, n_threads=None) -> np.ndarray:
    """Radial-projection convolution output of the receivers ``rows``: W_e = rho[e] @ Theta formed
    for their edges only (a library matmul), then the explicit uvu loops."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    deg = row_ptr[rows + 1] - row_ptr[rows]
    sub_ptr = np.concatenate([[0], np.cumsum(deg)])
    eidx = np.concatenate([np.arange(row_ptr[r], row_ptr[r + 1]) for r in rows]) if len(rows) else \
        np.zeros(0, np.int64)
    w = np.asarray(rho, np.float64)[eidx] @ np.asarray(theta, np.float64)
    return uvu_forward(tab, sub_ptr, np.asarray(col)[eidx], np.asarray(x, np.float64),
                       np.asarray(y, np.float64)[eidx], w, n_threads)


def conv_backward_radial_rows(tab: Tables, row_ptr, col, x, y, rho, theta, g, rows, senders, n_threads=None):
    """Radial-projection convolution backward on a sample, from the explicit uvu backward loops
    with W_e = rho[e] @ Theta formed per edge (a library matmul): dY and drho = dW_e Theta^T for
    every edge of the receivers ``rows``, dx of the nodes ``senders`` and dTheta = sum over every
    edge of rho[e]^T dW_e.  Returns (edge ids, dx, dy, drho, dtheta)."""
    rho = np.asarray(rho, np.float64)
    theta = np.asarray(theta, np.float64)
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    g = np.asarray(g, np.float64)
    w = rho @ theta
    eidx, dy, dw = conv_backward_edge_rows(tab, row_ptr, col, x, y, w, g, rows, n_threads)
    _, _, dw_all = conv_backward_edge_rows(tab, row_ptr, col, x, y, w, g, np.arange(len(row_ptr) - 1), n_threads)
    dx = conv_backward_x_rows(tab, row_ptr, col, y, w, g, senders, n_threads)
    return eidx, dx, dy, dw @ theta.T, rho.T @ dw_all


def conv_backward_uvw_rows(tab: Tables, row_ptr, col, x, y, w, g, edges, senders, n_threads=None):
    """uvw convolution backward on a sample: dY of the edges ``edges``, dx of the nodes
    ``senders`` (all their edges) and dW over every edge, from the explicit uvw backward loops
    applied to the edges as rows (x gathered by sender, g by receiver)."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col = np.asarray(col, dtype=np.int64)
    senders = np.asarray(senders, dtype=np.int64)
    dst = np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr))
    E = len(col)
    xe, ge = np.asarray(x)[col], np.asarray(g)[dst]
    order = np.argsort(col, kind="stable")
    starts = np.searchsorted(col[order], senders, side="left")
    ends = np.searchsorted(col[order], senders, side="right")
    sedges = np.concatenate([order[a:b] for a, b in zip(starts, ends)]) if len(senders) else np.zeros(0, np.int64)
    rows = np.concatenate([np.asarray(edges, np.int64), sedges])
    dxr, dyr, dw = uvw_backward(tab, xe, np.asarray(y), np.asarray(w), ge, rows, np.arange(E), n_threads)
    dy = dyr[:len(edges)]
    dxs = dxr[len(edges):]
    dx = np.zeros((len(senders), tab.prob.d_in))
    seg = np.repeat(np.arange(len(senders)), ends - starts)
    np.add.at(dx, seg, dxs)
    return dx, dy, dw
