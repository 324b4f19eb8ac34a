"""GPU parity of the convolution double backward (cgtp_conv_double_backward).

Bars as elsewhere: rel-L2 <= 1e-4 (fp32), <= 1e-10 (fp64) per output tensor against the oracle
(oracle.loops.conv_double_backward_rows, pinned against torch autograd applied twice to a dense
einsum, finite differences and the Euler identities); outputs bitwise repeatable and independent
of the receiver schedule and of which outputs are requested.
"""
import numpy as np
import pytest

from clebsch_gordan_tensor_cgtp_amd import binding as cg
from clebsch_gordan_tensor_cgtp_amd import synth
from oracle import loops

from cases import TOL, ConvCase, edge_case_graph, rel_l2, to_device

pytestmark = pytest.mark.gpu

SMALL = {
    "nequip-small": (synth.scaled(synth.CONV_NEQUIP, 300, 12_001), ("f32", "f64")),
    "stream-small": (synth.scaled(synth.CONV_STREAM, 257, 9_001), ("f32", "f64")),
    "mace-small": (synth.scaled(synth.CONV_MACE, 97, 2_999), ("f32", "f64")),
    "mixed-mul": (synth.ConvSpec("mixed", 61, 1_777, "5x0e+3x1o+7x2e+2x3o", 3, 3), ("f32", "f64")),
    "mul4": (synth.ConvSpec("mul4", 53, 1_201, "4x0e+4x1o", 2, 2), ("f32",)),
    "mul80": (synth.ConvSpec("mul80", 41, 997, "80x0e+80x1o", 1, 1), ("f32",)),
}
CASES = [(k, d) for k, (_, ds) in SMALL.items() for d in ds]


def upstream(case, seed):
    npdt = np.float32 if case.dtype == "f32" else np.float64
    st = synth.upstream_streams(seed)
    return (synth.normal(st["gg_x"], case.x.shape, dtype=npdt), synth.normal(st["gg_y"], (case.E, case.prob.d_sh),
                                                                            dtype=npdt),
            synth.normal(st["gg_w"], case.w.shape, dtype=npdt))


def run_dbl(case, device, gg, order=False, need=(True, True, True, True)):
    import torch
    plan = cg.plan_for(case.spec, case.dtype)
    d = to_device(case, device)
    y = cg.spherical_harmonics(case.spec.lmax_sh, d["vec"])
    tr = cg.graph_transpose(d["row_ptr"], d["col"])
    ggd = [None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device) for a in gg]
    o = cg.graph_order(d["row_ptr"]) if order else None
    res = cg.conv_double_backward(plan, d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"], *ggd, order=o,
                                  need=need)
    torch.cuda.synchronize()
    return res


def oracle_dbl(case, gg):
    z = [np.zeros(s) if a is None else a for a, s in zip(gg, (case.x.shape, (case.E, case.prob.d_sh), case.w.shape))]
    allr = np.arange(case.N)
    f64 = [np.asarray(a, np.float64) for a in (case.x, case.w, case.g, *z)]
    eidx, dx, dy, dw, dg = loops.conv_double_backward_rows(case.tab, case.row_ptr, case.col, f64[0], case.y_oracle(),
                                                           f64[1], f64[2], *f64[3:], allr, allr)
    assert np.array_equal(eidx, np.arange(case.E))
    return dx, dy, dw, dg


@pytest.mark.parametrize("name,dtype", CASES)
def test_double_backward_small(device, name, dtype):
    case = ConvCase(SMALL[name][0], dtype, seed=21)
    gg = upstream(case, 21)
    got = run_dbl(case, device, gg, order=True)
    for a, b in zip(got, oracle_dbl(case, gg)):
        assert rel_l2(a.cpu().numpy(), b) <= TOL[dtype]


@pytest.mark.parametrize("kind", ["empty", "heavy", "isolated", "selfdup"])
def test_double_backward_edge_cases(device, kind):
    spec = synth.ConvSpec("dbl-edge-" + kind, 600, 0, "32x0e+32x1o+32x2e", 2, 2)
    case = ConvCase(spec, "f32", seed=22, graph=edge_case_graph(kind, 600, np.random.default_rng(7)))
    gg = upstream(case, 22)
    got = [t.cpu().numpy() for t in run_dbl(case, device, gg)]
    if case.E == 0:
        assert all(np.all(t == 0) for t in (got[0], got[3]))
        return
    deg = np.diff(case.row_ptr)
    assert np.all(got[3][deg == 0] == 0)
    for a, b in zip(got, oracle_dbl(case, gg)):
        assert rel_l2(a, b) <= TOL["f32"]


def test_double_backward_absent_upstream_is_zero(device):
    """An upstream gradient passed as None acts as zeros (the binding passes a zero buffer)."""
    case = ConvCase(synth.scaled(synth.CONV_NEQUIP, 120, 4_000), "f32", seed=23)
    gg = list(upstream(case, 23))
    for drop in range(3):
        part = list(gg)
        part[drop] = None
        got = run_dbl(case, device, part)
        for a, b in zip(got, oracle_dbl(case, part)):
            assert rel_l2(a.cpu().numpy(), b) <= TOL["f32"]


def test_double_backward_bitwise_schedule_outputs_repeat(device):
    import torch
    case = ConvCase(synth.scaled(synth.CONV_STREAM, 900, 40_000), "f32", seed=24)
    gg = upstream(case, 24)
    full = run_dbl(case, device, gg, order=False)
    again = run_dbl(case, device, gg, order=True)
    for a, b in zip(full, again):
        assert torch.equal(a, b)
    for k in range(4):
        need = tuple(i == k for i in range(4))
        part = run_dbl(case, device, gg, need=need)
        for i in range(4):
            if i == k:
                assert torch.equal(part[i], full[i])
            else:
                assert part[i] is None
