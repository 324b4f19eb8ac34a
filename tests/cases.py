"""Shared helpers of the parity tests: seeded cases, oracle runs, comparisons.

Inputs come from ``clebsch_gordan_tensor_cgtp_amd.synth`` (the seeded
generators).  The GPU side computes Y from the edge vectors with the
library's harmonics kernel; the oracle computes its own Y from the same
vectors with ``oracle.sh``.  Nothing the oracle reads comes from the HIP path.
"""
import numpy as np

from clebsch_gordan_tensor_cgtp_amd import synth
from oracle import irreps as oirreps
from oracle import loops, sh as osh

TOL = {"f32": 1e-4, "f64": 1e-10}


def rel_l2(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    return float(num / den) if den > 0 else float(num)


def oracle_problem(spec):
    out = oirreps.per_path_out_irreps(spec.in_irreps, spec.lmax_sh, spec.lmax_out)
    return oirreps.build_problem(spec.in_irreps, oirreps.sh_irreps(spec.lmax_sh), out, "uvu")


class ConvCase:
    """A seeded convolution case: host arrays (numpy) in the run's dtype."""

    def __init__(self, spec, dtype="f32", seed=0, graph=None):
        self.spec, self.dtype = spec, dtype
        npdt = np.float32 if dtype == "f32" else np.float64
        st = synth.streams(seed)
        if graph is None:
            graph = synth.conv_graph(spec, seed)
        self.row_ptr, self.col = graph
        n, e = len(self.row_ptr) - 1, len(self.col)
        self.N, self.E = n, e
        self.prob = oracle_problem(spec)
        fan_in = max(1.0, e / max(n, 1))
        self.x = synth.normal(st["x"], (n, self.prob.d_in), dtype=npdt)
        self.vec = synth.normal(st["vec"], (e, 3), dtype=npdt)
        self.w = synth.normal(st["w"], (e, self.prob.weight_numel), 1.0 / np.sqrt(fan_in), dtype=npdt)
        self.g = synth.normal(st["sample"], (n, self.prob.d_out), dtype=npdt)
        self._tab = None

    @property
    def tab(self):
        if self._tab is None:
            self._tab = loops.Tables(self.prob)
        return self._tab

    def y_oracle(self, edges=None):
        v = self.vec if edges is None else self.vec[edges]
        return osh.real_sh_all(self.spec.lmax_sh, v.astype(np.float64))

    def oracle_forward(self, rows=None):
        rows = np.arange(self.N) if rows is None else np.asarray(rows)
        return loops.conv_forward_rows(self.tab, self.row_ptr, self.col, self.x.astype(np.float64),
                                       self.y_oracle(), self.w.astype(np.float64), rows)

    def oracle_backward(self, rows=None, senders=None):
        rows = np.arange(self.N) if rows is None else np.asarray(rows)
        senders = np.arange(self.N) if senders is None else np.asarray(senders)
        y = self.y_oracle()
        x, w, g = (a.astype(np.float64) for a in (self.x, self.w, self.g))
        eidx, dy, dw = loops.conv_backward_edge_rows(self.tab, self.row_ptr, self.col, x, y, w, g, rows)
        dx = loops.conv_backward_x_rows(self.tab, self.row_ptr, self.col, y, w, g, senders)
        return dx, eidx, dy, dw


def to_device(case, device):
    import torch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return {"row_ptr": t(case.row_ptr), "col": t(case.col), "x": t(case.x), "vec": t(case.vec), "w": t(case.w),
            "g": t(case.g)}


def edge_case_graph(kind, n_nodes, rng):
    """Irregular receiver CSRs: isolated nodes, self-loops, duplicates, one heavy receiver, empty."""
    if kind == "empty":
        return np.zeros(n_nodes + 1, np.int32), np.zeros(0, np.int32)
    if kind == "heavy":
        deg = rng.integers(0, 4, n_nodes)
        deg[n_nodes // 3] = 5000
    elif kind == "isolated":
        deg = rng.integers(0, 6, n_nodes)
        deg[::3] = 0
    else:  # self-loops and duplicate edges
        deg = rng.integers(1, 8, n_nodes)
    row_ptr = np.concatenate([[0], np.cumsum(deg)]).astype(np.int32)
    e = int(row_ptr[-1])
    col = rng.integers(0, n_nodes, e).astype(np.int32)
    if kind == "selfdup":
        recv = np.repeat(np.arange(n_nodes), deg)
        col[::4] = recv[::4]                       # self-loops
        col[1::5] = col[0:-1:5][: len(col[1::5])]  # duplicates of the previous edge
    return row_ptr, col
