"""GPU parity of the convolution backward in uvw mode (shared weights, caller workspace).

Bars: rel-L2 <= 1e-4 (fp32), <= 1e-10 (fp64) for dx, dY and dW against the oracle
(oracle.loops.conv_backward_uvw_rows: the explicit uvw backward loops with the edges as rows,
pinned against autograd on a dense einsum); dx and dY do not depend on the receiver schedule
(bitwise), repeated calls are bitwise identical, and a skipped output changes no other.
At the NequIP-like size (5000 receivers, 200k edges, the launch configuration of the
benchmark) dY and dx are checked on sampled edges and senders, dW in full.
"""
import numpy as np
import pytest

from clebsch_gordan_tensor_cgtp_amd import binding as cg
from clebsch_gordan_tensor_cgtp_amd import synth
from oracle import irreps as oirreps
from oracle import loops
from oracle import sh as osh

from cases import TOL, edge_case_graph, rel_l2

pytestmark = pytest.mark.gpu

LADDER5 = "+".join(f"16x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(6))
CASES = {
    # name: (in irreps, SH lmax, out irreps, N, E, dtypes)
    "nequip-32": ("32x0e+32x1o+32x2e", 2, "32x0e+32x1o+32x2e+32x1e+32x2o", 300, 12_001, ("f32", "f64")),
    "mixed": ("5x0e+3x1o+7x2e+2x3o", 3, "6x0e+4x1o+3x2e+2x1e+1x3o+17x2o", 61, 1_777, ("f32", "f64")),
    "mul64": ("64x0e+64x1o", 1, "16x0e+48x1o+64x1e", 97, 3_001, ("f32",)),
    "mul128": ("128x0e+128x1o", 1, "32x0e+32x1o+16x1e", 45, 1_500, ("f32",)),
    "high-l": (LADDER5, 5, LADDER5, 37, 401, ("f32", "f64")),
}
PARAMS = [(k, d) for k, v in CASES.items() for d in v[5]]


def make_case(name, dtype, seed, graph=None):
    ins, lmax, outs, n, e, _ = CASES[name]
    npdt = np.float32 if dtype == "f32" else np.float64
    prob = oirreps.build_problem(ins, oirreps.sh_irreps(lmax), outs, "uvw")
    st = synth.streams(seed)
    row_ptr, col = graph if graph is not None else synth.uniform_graph(n, e, synth.rng(st["graph"]))
    n, e = len(row_ptr) - 1, len(col)
    return {"prob": prob, "ins": ins, "lmax": lmax, "outs": outs, "dtype": dtype, "row_ptr": row_ptr, "col": col,
            "x": synth.normal(st["x"], (n, prob.d_in), dtype=npdt),
            "vec": synth.normal(st["vec"], (e, 3), dtype=npdt),
            "w": synth.normal(st["w"], (prob.weight_numel,), dtype=npdt),
            "g": synth.normal(st["sample"], (n, prob.d_out), dtype=npdt)}


def run_gpu(c, device, ordered=False, need=(True, True, True), plan=None):
    import torch
    plan = plan or cg.Plan(c["ins"], cg.sh_irreps(c["lmax"]), c["outs"], "uvw", c["dtype"])
    t = {k: torch.from_numpy(np.ascontiguousarray(c[k])).to(device) for k in ("row_ptr", "col", "x", "vec", "w", "g")}
    y = cg.spherical_harmonics(c["lmax"], t["vec"])
    tr = cg.graph_transpose(t["row_ptr"], t["col"])
    order = cg.graph_order(t["row_ptr"]) if ordered else None
    res = cg.conv_backward(plan, t["row_ptr"], t["col"], tr, t["x"], y, t["w"], t["g"], need=need, order=order)
    torch.cuda.synchronize()
    return res


def oracle(c, edges=None, senders=None):
    n, e = len(c["row_ptr"]) - 1, len(c["col"])
    edges = np.arange(e) if edges is None else edges
    senders = np.arange(n) if senders is None else senders
    y = osh.real_sh_all(c["lmax"], c["vec"].astype(np.float64))
    return loops.conv_backward_uvw_rows(loops.Tables(c["prob"]), c["row_ptr"], c["col"], c["x"].astype(np.float64), y,
                                        c["w"].astype(np.float64), c["g"].astype(np.float64), edges, senders)


def check(got, want, dtype):
    for name, a, b in zip(("dx", "dy", "dw"), got, want):
        err = rel_l2(a.cpu().numpy(), b)
        assert err <= TOL[dtype], f"{name}: rel-L2 {err:.3e}"


@pytest.mark.parametrize("name,dtype", PARAMS)
def test_uvw_conv_backward_parity(device, name, dtype):
    c = make_case(name, dtype, seed=51)
    check(run_gpu(c, device, ordered=True), oracle(c), dtype)


@pytest.mark.parametrize("kind", ["empty", "heavy", "isolated", "selfdup"])
def test_uvw_conv_backward_edge_cases(device, kind):
    c = make_case("nequip-32", "f32", seed=52, graph=edge_case_graph(kind, 333, np.random.default_rng(11)))
    dx, dy, dw = run_gpu(c, device)
    outdeg = np.bincount(c["col"], minlength=len(c["row_ptr"]) - 1)
    assert np.all(dx.cpu().numpy()[outdeg == 0] == 0)
    if len(c["col"]) == 0:
        assert np.all(dx.cpu().numpy() == 0) and np.all(dw.cpu().numpy() == 0) and dy.shape[0] == 0
    else:
        check((dx, dy, dw), oracle(c), "f32")


def test_uvw_conv_backward_no_receivers(device):
    """N = 0: nothing to differentiate; the shared-weight gradient is zero."""
    import torch
    c = make_case("nequip-32", "f32", seed=53, graph=(np.zeros(1, np.int32), np.zeros(0, np.int32)))
    plan = cg.Plan(c["ins"], cg.sh_irreps(c["lmax"]), c["outs"], "uvw", "f32")
    gw = torch.full((plan.weight_numel,), 7.0, device=device)
    t = {k: torch.from_numpy(np.ascontiguousarray(c[k])).to(device) for k in ("row_ptr", "col", "x", "w", "g")}
    y = torch.zeros((0, plan.d_sh), device=device)
    tr = (torch.zeros(1, dtype=torch.int32, device=device), torch.zeros(0, dtype=torch.int32, device=device),
          torch.zeros(0, dtype=torch.int32, device=device))
    cg.conv_backward(plan, t["row_ptr"], t["col"], tr, t["x"], y, t["w"], t["g"], grad_w=gw, need=(False, False, True))
    torch.cuda.synchronize()
    assert torch.all(gw == 0)


def test_uvw_conv_backward_subsets_schedule_repeat(device):
    import torch
    c = make_case("nequip-32", "f32", seed=54,
                  graph=synth.powerlaw_graph(1000, 30_000, 2.0, 400, np.random.default_rng(5)))
    full = run_gpu(c, device, ordered=True)
    again = run_gpu(c, device, ordered=True)
    natural = run_gpu(c, device, ordered=False)
    for a, b in zip(full, again):
        assert torch.equal(a, b)
    assert torch.equal(full[0], natural[0]) and torch.equal(full[1], natural[1])
    assert rel_l2(natural[2].cpu().numpy(), full[2].cpu().numpy()) <= TOL["f32"]
    only_x = run_gpu(c, device, ordered=True, need=(True, False, False))
    only_y = run_gpu(c, device, ordered=True, need=(False, True, False))
    only_w = run_gpu(c, device, ordered=True, need=(False, False, True))
    assert torch.equal(only_x[0], full[0]) and only_x[1] is None and only_x[2] is None
    assert torch.equal(only_y[1], full[1])
    assert torch.equal(only_w[2], full[2])
    check(full, oracle(c), "f32")


def test_uvw_conv_backward_workspace_errors(device):
    import torch
    c = make_case("mixed", "f32", seed=55)
    plan = cg.Plan(c["ins"], cg.sh_irreps(c["lmax"]), c["outs"], "uvw", "f32")
    n, e = len(c["row_ptr"]) - 1, len(c["col"])
    need = cg.conv_backward_workspace_size(plan, n, e)
    assert need > 0
    small = torch.empty(need - 256, dtype=torch.uint8, device=device)
    with pytest.raises(cg.CgtpError, match="workspace too small"):
        run_gpu_ws(c, device, plan, small)
    exact = torch.empty(need, dtype=torch.uint8, device=device)
    check(run_gpu_ws(c, device, plan, exact), oracle(c), "f32")


def run_gpu_ws(c, device, plan, workspace):
    import torch
    t = {k: torch.from_numpy(np.ascontiguousarray(c[k])).to(device) for k in ("row_ptr", "col", "x", "vec", "w", "g")}
    y = cg.spherical_harmonics(c["lmax"], t["vec"])
    tr = cg.graph_transpose(t["row_ptr"], t["col"])
    res = cg.conv_backward(plan, t["row_ptr"], t["col"], tr, t["x"], y, t["w"], t["g"], workspace=workspace)
    torch.cuda.synchronize()
    return res


def test_uvw_conv_backward_full_size_sampled(device):
    """The NequIP-like workload with uvw mixing (5000 receivers, 200k edges) as the benchmark
    launches it (heavy-first schedule): dY on 2000 sampled edges, dx on 300 sampled senders,
    dW in full (every edge)."""
    spec = synth.CONV_NEQUIP_UVW
    st = synth.streams(0)
    row_ptr, col = synth.conv_graph(spec, 0)
    n, e = len(row_ptr) - 1, len(col)
    prob = oirreps.build_problem(spec.in_irreps, oirreps.sh_irreps(spec.lmax_sh), spec.out_irreps, "uvw")
    c = {"prob": prob, "ins": spec.in_irreps, "lmax": spec.lmax_sh, "outs": spec.out_irreps, "dtype": "f32",
         "row_ptr": row_ptr, "col": col,
         "x": synth.normal(st["x"], (n, prob.d_in), dtype=np.float32),
         "vec": synth.normal(st["vec"], (e, 3), dtype=np.float32),
         "w": synth.normal(st["w"], (prob.weight_numel,), 1.0 / np.sqrt(e / n), dtype=np.float32),
         "g": synth.normal(st["sample"], (n, prob.d_out), dtype=np.float32)}
    dx, dy, dw = run_gpu(c, device, ordered=True)
    rs = np.random.default_rng(17)
    edges = np.sort(rs.choice(e, 2000, replace=False))
    senders = np.sort(rs.choice(n, 300, replace=False))
    wx, wy, ww = oracle(c, edges, senders)
    assert rel_l2(dy.cpu().numpy()[edges], wy) <= TOL["f32"]
    assert rel_l2(dx.cpu().numpy()[senders], wx) <= TOL["f32"]
    assert rel_l2(dw.cpu().numpy(), ww) <= TOL["f32"]
