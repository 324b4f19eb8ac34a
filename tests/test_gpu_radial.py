"""GPU parity of the convolution with radially projected weights (cgtp_conv_forward_radial).

Bars: rel-L2 <= 1e-4 (fp32), <= 1e-10 (fp64) against the oracle (oracle.ref.conv_forward_radial /
oracle.loops.conv_forward_radial_rows, pinned by a dense einsum, linearity in Theta and one-hot
radial features); the receiver schedule does not change a bit; the result equals the ordinary
forward given W = rho @ Theta, within the rounding of forming W.
"""
import numpy as np
import pytest

from clebsch_gordan_tensor_cgtp_amd import binding as cg
from clebsch_gordan_tensor_cgtp_amd import synth
from oracle import loops

from cases import TOL, ConvCase, edge_case_graph, rel_l2, to_device

pytestmark = pytest.mark.gpu

CASES = [
    (synth.scaled(synth.CONV_NEQUIP, 300, 12_001), 8, "f32"),
    (synth.scaled(synth.CONV_NEQUIP, 300, 12_001), 8, "f64"),
    (synth.scaled(synth.CONV_STREAM, 257, 9_001), 8, "f32"),
    (synth.scaled(synth.CONV_STREAM, 257, 9_001), 16, "f32"),
    (synth.ConvSpec("mixed", 61, 1_777, "5x0e+3x1o+7x2e+2x3o", 3, 3), 5, "f64"),
    (synth.ConvSpec("mul80", 41, 997, "80x0e+80x1o", 1, 1), 3, "f32"),
    (synth.ConvSpec("mul4", 53, 1_201, "4x0e+4x1o", 2, 2), 1, "f32"),
    # MACE-like irreps (4,352 weights per edge): Theta is copied to LDS per path group (and per
    # channel tile in the forward), R * weight_numel alone would not fit a workgroup's LDS
    (synth.scaled(synth.CONV_MACE, 97, 2_999), 8, "f32"),
    (synth.scaled(synth.CONV_MACE, 97, 2_999), 8, "f64"),
    (synth.scaled(synth.CONV_MACE, 61, 1_501), 16, "f32"),
]


def radial_inputs(case, R, seed):
    npdt = np.float32 if case.dtype == "f32" else np.float64
    st = synth.upstream_streams(seed)  # independent children for rho and Theta
    rho = synth.normal(st["gg_y"], (case.E, R), dtype=npdt)
    theta = synth.normal(st["gg_w"], (R, case.prob.weight_numel), 1.0 / np.sqrt(R * 40.0), dtype=npdt)
    return rho, theta


def run(case, device, rho, theta, ordered):
    import torch
    plan = cg.plan_for(case.spec, case.dtype)
    d = to_device(case, device)
    y = cg.spherical_harmonics(case.spec.lmax_sh, d["vec"])
    o = cg.graph_order(d["row_ptr"]) if ordered else None
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    out = cg.conv_forward_radial(plan, d["row_ptr"], d["col"], d["x"], y, t(rho), t(theta), order=o)
    torch.cuda.synchronize()
    return out, d, y, plan


def oracle(case, rho, theta):
    return loops.conv_forward_radial_rows(case.tab, case.row_ptr, case.col, case.x.astype(np.float64),
                                          case.y_oracle(), rho.astype(np.float64), theta.astype(np.float64),
                                          np.arange(case.N))


@pytest.mark.parametrize("spec,R,dtype", CASES, ids=[f"{c[0].name}-R{c[1]}-{c[2]}" for c in CASES])
def test_radial_forward(device, spec, R, dtype):
    case = ConvCase(spec, dtype, seed=51)
    rho, theta = radial_inputs(case, R, 51)
    out, *_ = run(case, device, rho, theta, ordered=True)
    assert rel_l2(out.cpu().numpy(), oracle(case, rho, theta)) <= TOL[dtype]


@pytest.mark.parametrize("kind", ["empty", "heavy", "isolated"])
def test_radial_edge_cases(device, kind):
    spec = synth.ConvSpec("radial-" + kind, 500, 0, "32x0e+32x1o+32x2e", 2, 2)
    case = ConvCase(spec, "f32", seed=52, graph=edge_case_graph(kind, 500, np.random.default_rng(11)))
    rho, theta = radial_inputs(case, 8, 52)
    out, *_ = run(case, device, rho, theta, ordered=False)
    got = out.cpu().numpy()
    assert np.all(got[np.diff(case.row_ptr) == 0] == 0)
    if case.E:
        assert rel_l2(got, oracle(case, rho, theta)) <= TOL["f32"]


def test_radial_schedule_bitwise_and_matches_materialised_weights(device):
    import torch
    case = ConvCase(synth.scaled(synth.CONV_STREAM, 800, 30_000), "f64", seed=53)
    rho, theta = radial_inputs(case, 8, 53)
    a, d, y, plan = run(case, device, rho, theta, ordered=False)
    b, *_ = run(case, device, rho, theta, ordered=True)
    assert torch.equal(a, b)
    w = torch.from_numpy(rho @ theta).to(device)  # the weights the kernel never stores
    ref = cg.conv_forward(plan, d["row_ptr"], d["col"], d["x"], y, w)
    torch.cuda.synchronize()
    assert rel_l2(a.cpu().numpy(), ref.cpu().numpy()) <= 1e-12
