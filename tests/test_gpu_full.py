"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The forward runs with the heavy-first receiver schedule and must equal the natural-order
forward bitwise.  The NequIP-like graph is compared in full.  The MACE-like graph (1M edges, 17-35 GB of
per-edge weights) and the 10M-edge power-law graph are compared on a seeded sample: receivers
(always including the heaviest one) for the output, dY and dW of all their edges, and senders
(always including the one with most edges) for dx.  The oracle reads back only the rows it needs.
"""
import numpy as np
import pytest

from clebsch_gordan_tensor_cgtp_amd import binding as cg
from clebsch_gordan_tensor_cgtp_amd import synth
from oracle import loops
from oracle import sh as osh

from cases import TOL, oracle_problem, rel_l2

pytestmark = pytest.mark.gpu


class DeviceCase:
    """Full-size inputs made by the seeded generators (large tensors drawn on the device)."""

    def __init__(self, spec, dtype, device, seed=0):
        import torch
        self.spec, self.dtype = spec, dtype
        npdt = np.float32 if dtype == "f32" else np.float64
        st = synth.streams(seed)
        self.row_ptr, self.col = synth.conv_graph(spec, seed)
        self.N, self.E = len(self.row_ptr) - 1, len(self.col)
        self.plan = cg.plan_for(spec, dtype)
        self.prob = oracle_problem(spec)
        fan_in = self.E / self.N

        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(device) if isinstance(a, np.ndarray) else a

        self.d = {
            "row_ptr": dev(self.row_ptr), "col": dev(self.col),
            "x": dev(synth.normal(st["x"], (self.N, self.plan.d_x), dtype=npdt, device=device)),
            "vec": dev(synth.normal(st["vec"], (self.E, 3), dtype=npdt, device=device)),
            "w": dev(synth.normal(st["w"], (self.E, self.plan.weight_numel), 1.0 / np.sqrt(fan_in), dtype=npdt,
                                  device=device)),
            "g": dev(synth.normal(st["sample"], (self.N, self.plan.d_out), dtype=npdt, device=device)),
        }
        self.tab = loops.Tables(self.prob)

    def run(self, receiver_ws=None):
        """Forward, then the backward: sender order, or (receiver_ws = workspace bytes) receiver
        order with a bounded workspace, as bench.py times it."""
        import torch
        d = self.d
        y = cg.spherical_harmonics(self.spec.lmax_sh, d["vec"])
        order = cg.graph_order(d["row_ptr"])  # the heavy-first schedule bench.py times
        out = cg.conv_forward(self.plan, d["row_ptr"], d["col"], d["x"], y, d["w"], order=order)
        if self.E <= 20_000_000:
            natural = cg.conv_forward(self.plan, d["row_ptr"], d["col"], d["x"], y, d["w"])
            assert torch.equal(out, natural)
            del natural
        tr = cg.graph_transpose(d["row_ptr"], d["col"])
        if receiver_ws is None:
            gx, gy, gw = cg.conv_backward(self.plan, d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"])
        else:
            full, least = cg.conv_backward_receiver_workspace_size(self.plan, self.N, self.E)
            ws = torch.empty(max(least, min(full, receiver_ws)), dtype=torch.uint8, device=d["x"].device)
            gx, gy, gw = cg.conv_backward_receiver(self.plan, d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"],
                                                   workspace=ws)
            del ws
        torch.cuda.synchronize()
        return out, gx, gy, gw

    def rows(self, t, idx):
        import torch
        return t.index_select(0, torch.from_numpy(np.asarray(idx, dtype=np.int64)).to(t.device)).cpu().numpy()

    def y_of(self, edges):
        return osh.real_sh_all(self.spec.lmax_sh, self.rows(self.d["vec"], edges).astype(np.float64))

    def oracle_receivers(self, recv):
        rp = self.row_ptr.astype(np.int64)
        deg = rp[recv + 1] - rp[recv]
        sub_ptr = np.concatenate([[0], np.cumsum(deg)])
        edges = np.concatenate([np.arange(rp[r], rp[r + 1]) for r in recv])
        x = self.d["x"].double().cpu().numpy()
        y = self.y_of(edges)
        w = self.rows(self.d["w"], edges).astype(np.float64)
        g = self.rows(self.d["g"], recv).astype(np.float64)
        cols = self.col[edges].astype(np.int64)
        out = loops.uvu_forward(self.tab, sub_ptr, cols, x, y, w)
        dy, dw = loops.uvu_backward_edges(self.tab, sub_ptr, cols, x, y, w, g)
        return edges, out, dy, dw

    def oracle_senders(self, senders):
        col = self.col.astype(np.int64)
        order = np.argsort(col, kind="stable")
        starts = np.searchsorted(col[order], senders, side="left")
        ends = np.searchsorted(col[order], senders, side="right")
        edges = np.concatenate([order[a:b] for a, b in zip(starts, ends)])
        sptr = np.concatenate([[0], np.cumsum(ends - starts)])
        dst = np.searchsorted(self.row_ptr.astype(np.int64), edges, side="right") - 1
        uniq, inv = np.unique(dst, return_inverse=True)
        y = self.y_of(edges)
        w = self.rows(self.d["w"], edges).astype(np.float64)
        g = self.rows(self.d["g"], uniq).astype(np.float64)
        return loops.uvu_backward_x(self.tab, sptr, inv, y, w, g)


def check_sampled(case, n_recv, n_send, seed=5, receiver_ws=None):
    out, gx, gy, gw = case.run(receiver_ws)
    rng = np.random.default_rng(seed)
    deg = np.diff(case.row_ptr)
    outdeg = np.bincount(case.col, minlength=case.N)
    recv = np.unique(np.concatenate([rng.choice(case.N, n_recv, replace=False), [int(np.argmax(deg))]]))
    send = np.unique(np.concatenate([rng.choice(case.N, n_send, replace=False), [int(np.argmax(outdeg))]]))
    tol = TOL[case.dtype]
    edges, want_out, want_dy, want_dw = case.oracle_receivers(recv)
    assert rel_l2(case.rows(out, recv), want_out) <= tol
    assert rel_l2(case.rows(gy, edges), want_dy) <= tol
    assert rel_l2(case.rows(gw, edges), want_dw) <= tol
    assert rel_l2(case.rows(gx, send), case.oracle_senders(send)) <= tol
    # receivers without edges are exactly zero
    empty = np.nonzero(deg == 0)[0]
    if len(empty):
        assert np.all(case.rows(out, empty[:64]) == 0)


def test_full_nequip_all_rows(device):
    case = DeviceCase(synth.CONV_NEQUIP, "f32", device)
    out, gx, gy, gw = case.run()
    allr = np.arange(case.N)
    edges, want_out, want_dy, want_dw = case.oracle_receivers(allr)
    assert np.array_equal(edges, np.arange(case.E))
    assert rel_l2(out.cpu().numpy(), want_out) <= TOL["f32"]
    assert rel_l2(gy.cpu().numpy(), want_dy) <= TOL["f32"]
    assert rel_l2(gw.cpu().numpy(), want_dw) <= TOL["f32"]
    assert rel_l2(gx.cpu().numpy(), case.oracle_senders(allr)) <= TOL["f32"]


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_full_mace_sampled(device, dtype):
    import torch
    case = DeviceCase(synth.CONV_MACE, dtype, device)
    check_sampled(case, 192, 128)
    del case
    torch.cuda.empty_cache()


def test_full_stream_powerlaw_sampled(device):
    import torch
    case = DeviceCase(synth.CONV_STREAM, "f32", device)
    assert int(np.diff(case.row_ptr).max()) == 2000
    check_sampled(case, 256, 256)
    del case
    torch.cuda.empty_cache()


# ------------------------------------------------------------------------------ receiver-order backward

def test_full_nequip_receiver_backward_all_rows(device):
    """The NequIP-like graph in full, with a 64 MB workspace: four edge ranges, dx summed over them."""
    case = DeviceCase(synth.CONV_NEQUIP, "f32", device)
    out, gx, gy, gw = case.run(receiver_ws=64 << 20)
    allr = np.arange(case.N)
    edges, want_out, want_dy, want_dw = case.oracle_receivers(allr)
    assert rel_l2(gy.cpu().numpy(), want_dy) <= TOL["f32"]
    assert rel_l2(gw.cpu().numpy(), want_dw) <= TOL["f32"]
    assert rel_l2(gx.cpu().numpy(), case.oracle_senders(allr)) <= TOL["f32"]


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_full_mace_receiver_backward_sampled(device, dtype):
    import torch
    import bench
    case = DeviceCase(synth.CONV_MACE, dtype, device)
    check_sampled(case, 192, 128, receiver_ws=bench.RECEIVER_WORKSPACE_BYTES)
    del case
    torch.cuda.empty_cache()


def test_full_stream_receiver_backward_sampled(device):
    import torch
    import bench
    case = DeviceCase(synth.CONV_STREAM, "f32", device)
    check_sampled(case, 256, 256, receiver_ws=bench.RECEIVER_WORKSPACE_BYTES)
    del case
    torch.cuda.empty_cache()


# ------------------------------------------------------------------------------ double backward

class DoubleBackwardCase(DeviceCase):
    """Full-size inputs plus the upstream gradients gg_x, gg_y, gg_w (seeded, drawn like x, y, w)."""

    def __init__(self, spec, dtype, device, seed=0):
        super().__init__(spec, dtype, device, seed)
        npdt = np.float32 if dtype == "f32" else np.float64
        up = synth.upstream_streams(seed)
        import torch

        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(device) if isinstance(a, np.ndarray) else a

        self.gg = [dev(synth.normal(up["gg_x"], (self.N, self.plan.d_x), dtype=npdt, device=device)),
                   dev(synth.normal(up["gg_y"], (self.E, self.plan.d_sh), dtype=npdt, device=device)),
                   dev(synth.normal(up["gg_w"], (self.E, self.plan.weight_numel), dtype=npdt, device=device))]

    def run_dbl(self):
        import torch
        d = self.d
        y = cg.spherical_harmonics(self.spec.lmax_sh, d["vec"])
        tr = cg.graph_transpose(d["row_ptr"], d["col"])
        order = cg.graph_order(d["row_ptr"])
        res = cg.conv_double_backward(self.plan, d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"], *self.gg,
                                      order=order)
        torch.cuda.synchronize()
        return res

    def oracle_on(self, rp, col_local, senders_global, edges, recv_global, rows, senders):
        """The oracle on a sub-graph: rp/col_local index local senders, whose global ids are
        senders_global; edges are global edge ids in sub-CSR order, recv_global the receivers."""
        f64 = lambda a: np.asarray(a, np.float64)
        x = f64(self.rows(self.d["x"], senders_global))
        ggx = f64(self.rows(self.gg[0], senders_global))
        y = self.y_of(edges)
        ggy = f64(self.rows(self.gg[1], edges))
        w = f64(self.rows(self.d["w"], edges))
        ggw = f64(self.rows(self.gg[2], edges))
        g = f64(self.rows(self.d["g"], recv_global))
        return loops.conv_double_backward_rows(self.tab, rp, col_local, x, y, w, g, ggx, ggy, ggw, rows, senders)

    def oracle_receivers_dbl(self, recv):
        rp = self.row_ptr.astype(np.int64)
        deg = rp[recv + 1] - rp[recv]
        sub_ptr = np.concatenate([[0], np.cumsum(deg)])
        edges = np.concatenate([np.arange(rp[r], rp[r + 1]) for r in recv])
        uniq, inv = np.unique(self.col[edges], return_inverse=True)
        _, _, dy, dw, dg = self.oracle_on(sub_ptr, inv, uniq, edges, recv, np.arange(len(recv)), np.zeros(0, np.int64))
        return edges, dy, dw, dg

    def oracle_senders_dbl(self, send):
        col = self.col.astype(np.int64)
        edges = np.nonzero(np.isin(col, send))[0]              # ascending edge id = receiver order
        dst = np.searchsorted(self.row_ptr.astype(np.int64), edges, side="right") - 1
        runiq, rinv = np.unique(dst, return_inverse=True)
        sub_ptr = np.concatenate([[0], np.cumsum(np.bincount(rinv, minlength=len(runiq)))])
        s_local = np.searchsorted(send, col[edges])
        _, dx, _, _, _ = self.oracle_on(sub_ptr, s_local, send, edges, runiq, np.zeros(0, np.int64),
                                        np.arange(len(send)))
        return dx


def test_full_nequip_double_backward_all_rows(device):
    case = DoubleBackwardCase(synth.CONV_NEQUIP, "f32", device)
    gx, gy, gw, gg = case.run_dbl()
    allr = np.arange(case.N)
    edges, dy, dw, dg = case.oracle_receivers_dbl(allr)
    assert np.array_equal(edges, np.arange(case.E))
    assert rel_l2(gg.cpu().numpy(), dg) <= TOL["f32"]
    assert rel_l2(gy.cpu().numpy(), dy) <= TOL["f32"]
    assert rel_l2(gw.cpu().numpy(), dw) <= TOL["f32"]
    assert rel_l2(gx.cpu().numpy(), case.oracle_senders_dbl(allr)) <= TOL["f32"]


def test_full_mace_double_backward_sampled(device):
    import torch
    case = DoubleBackwardCase(synth.CONV_MACE, "f32", device)
    gx, gy, gw, gg = case.run_dbl()
    rng = np.random.default_rng(31)
    deg = np.diff(case.row_ptr)
    outdeg = np.bincount(case.col, minlength=case.N)
    recv = np.unique(np.concatenate([rng.choice(case.N, 96, replace=False), [int(np.argmax(deg))]]))
    send = np.unique(np.concatenate([rng.choice(case.N, 64, replace=False), [int(np.argmax(outdeg))]]))
    edges, dy, dw, dg = case.oracle_receivers_dbl(recv)
    assert rel_l2(case.rows(gg, recv), dg) <= TOL["f32"]
    assert rel_l2(case.rows(gy, edges), dy) <= TOL["f32"]
    assert rel_l2(case.rows(gw, edges), dw) <= TOL["f32"]
    assert rel_l2(case.rows(gx, send), case.oracle_senders_dbl(send)) <= TOL["f32"]
    del case, gx, gy, gw, gg
    torch.cuda.empty_cache()
