"""GPU parity on corner shapes of the method, against the oracle (same bars: rel-L2 <= 1e-4 fp32,
<= 1e-10 fp64):

- a scalar convolution (1x0e with l = 0 harmonics: one channel, so 64 edges share a wave);
- multiplicities 1 and 2 next to each other (edge slots of 64 and 32 lanes in one plan);
- the top of the angular range on every side (inputs 2x5o + 1x7e, harmonics and outputs to l = 7);
- a single node whose edges are all self-loops;
- the batched product on one row;
- the uvw convolution (forward and backward) with one channel per irrep.
"""
import numpy as np
import pytest

from clebsch_gordan_tensor_cgtp_amd import binding as cg
from clebsch_gordan_tensor_cgtp_amd import synth
from oracle import irreps as oirreps
from oracle import loops
from oracle import ref
from oracle import sh as osh

from cases import TOL, ConvCase, rel_l2, to_device

pytestmark = pytest.mark.gpu

UVU = {
    "scalar": (synth.ConvSpec("scalar", 37, 501, "1x0e", 0, 0), ("f32", "f64")),
    "mul1-mul2": (synth.ConvSpec("mul1-mul2", 29, 777, "1x0e+2x1o+1x2e", 2, 2), ("f32", "f64")),
    "high-l": (synth.ConvSpec("high-l", 23, 311, "2x5o+1x7e", 7, 7), ("f32", "f64")),
    "single-node": (synth.ConvSpec("single-node", 1, 40, "8x0e+8x1o", 1, 1), ("f32",)),
}
PARAMS = [(k, d) for k, (_, ds) in UVU.items() for d in ds]


@pytest.mark.parametrize("name,dtype", PARAMS)
def test_uvu_corner_forward_backward(device, name, dtype):
    import torch
    spec = UVU[name][0]
    case = ConvCase(spec, dtype, seed=71)
    plan = cg.plan_for(spec, dtype)
    d = to_device(case, device)
    y = cg.spherical_harmonics(spec.lmax_sh, d["vec"])
    out = cg.conv_forward(plan, d["row_ptr"], d["col"], d["x"], y, d["w"])
    tr = cg.graph_transpose(d["row_ptr"], d["col"])
    gx, gy, gw = cg.conv_backward(plan, d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"])
    torch.cuda.synchronize()
    assert rel_l2(out.cpu().numpy(), case.oracle_forward()) <= TOL[dtype]
    dx, eidx, dy, dw = case.oracle_backward()
    assert rel_l2(gx.cpu().numpy(), dx) <= TOL[dtype]
    assert rel_l2(gy.cpu().numpy()[eidx], dy) <= TOL[dtype]
    assert rel_l2(gw.cpu().numpy()[eidx], dw) <= TOL[dtype]


def test_batched_single_row(device):
    import torch
    ins, lmax = "4x0e+4x1o", 2
    out_ir = cg.per_path_out_irreps(ins, lmax, lmax)
    plan = cg.Plan(ins, cg.sh_irreps(lmax), out_ir, "uvu", "f64")
    prob = oirreps.build_problem(ins, oirreps.sh_irreps(lmax), out_ir, "uvu")
    st = synth.streams(72)
    x = synth.normal(st["x"], (1, prob.d_in))
    vec = synth.normal(st["vec"], (1, 3))
    w = synth.normal(st["w"], (1, prob.weight_numel))
    t = lambda a: torch.from_numpy(a).to(device)
    y = cg.spherical_harmonics(lmax, t(vec))
    got = cg.tp_forward(plan, t(x), y, t(w))
    torch.cuda.synchronize()
    want = ref.tp_forward(prob, x, osh.real_sh_all(lmax, vec), w)
    assert rel_l2(got.cpu().numpy(), want) <= TOL["f64"]


def test_uvw_conv_one_channel(device):
    import torch
    ins, lmax, outs = "1x0e+1x1o", 1, "1x0e+1x1o+1x1e"
    prob = oirreps.build_problem(ins, oirreps.sh_irreps(lmax), outs, "uvw")
    plan = cg.Plan(ins, cg.sh_irreps(lmax), outs, "uvw", "f64")
    st = synth.streams(73)
    row_ptr, col = synth.uniform_graph(45, 700, synth.rng(st["graph"]))
    x = synth.normal(st["x"], (45, prob.d_in))
    vec = synth.normal(st["vec"], (700, 3))
    w = synth.normal(st["w"], (prob.weight_numel,))
    g = synth.normal(st["sample"], (45, prob.d_out))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    yd = cg.spherical_harmonics(lmax, t(vec))
    rp, cl = t(row_ptr), t(col)
    out = cg.conv_forward(plan, rp, cl, t(x), yd, t(w))
    tr = cg.graph_transpose(rp, cl)
    gx, gy, gw = cg.conv_backward(plan, rp, cl, tr, t(x), yd, t(w), t(g))
    torch.cuda.synchronize()
    y = osh.real_sh_all(lmax, vec)
    tab = loops.Tables(prob)
    assert rel_l2(out.cpu().numpy(), loops.conv_forward_uvw_rows(tab, row_ptr, col, x, y, w, np.arange(45))) <= TOL["f64"]
    dx, dy, dw = loops.conv_backward_uvw_rows(tab, row_ptr, col, x, y, w, g, np.arange(700), np.arange(45))
    for a, b in ((gx, dx), (gy, dy), (gw, dw)):
        assert rel_l2(a.cpu().numpy(), b) <= TOL["f64"]
