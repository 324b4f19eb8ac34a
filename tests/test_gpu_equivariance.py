"""Equivariance of the HIP path itself (pin G8 applied to the GPU outputs).

The operation exists to keep geometric relations between inputs and outputs
(sciencestack.ai page, "An Efficient Sparse Kernel Generator for
O(3)-Equivariant Deep Networks", Abstract): rotating the node features by
D_in(R) and the edge vectors by R must rotate the output by D_out(R), for
proper and improper R (an improper -R multiplies each irrep by its parity).
Through the backward, the gradients follow: dx by D_in, dY by D_sh, dW
unchanged.  Every quantity below is computed by the library's kernels,
including the spherical harmonics of the rotated edge vectors; only the
Wigner matrices come from the oracle (least squares on its own harmonics).

Bars: rel-L2 <= 1e-4 in fp32 and <= 1e-5 in fp64 between the rotated run and
the rotated result of the plain run.
"""
import numpy as np
import pytest

from clebsch_gordan_tensor_cgtp_amd import binding as cg
from clebsch_gordan_tensor_cgtp_amd import synth
from oracle import irreps as oirreps
from oracle import wigner

from cases import ConvCase, rel_l2

pytestmark = pytest.mark.gpu

BAR = {"f32": 1e-4, "f64": 1e-5}

UVU = {
    "nequip-small": synth.scaled(synth.CONV_NEQUIP, 300, 12_001),
    "mace-small": synth.scaled(synth.CONV_MACE, 97, 2_999),
    "mixed-mul": synth.ConvSpec("mixed", 61, 1_777, "5x0e+3x1o+7x2e+2x3o", 3, 3),
}


def rotation(seed, improper):
    rot = wigner.random_rotation(np.random.default_rng(seed))
    return rot, (-rot if improper else rot)


def dmat(irreps_list, rot, improper):
    return wigner.irreps_d(irreps_list, rot, improper)


def dev(a, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t):
    return t.cpu().numpy().astype(np.float64)


def cast(a, dtype):
    return np.asarray(a, dtype=np.float32 if dtype == "f32" else np.float64)


@pytest.mark.parametrize("improper", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("name", sorted(UVU))
def test_uvu_conv_forward_backward_equivariance(device, name, dtype, improper):
    import torch
    case = ConvCase(UVU[name], dtype, seed=71)
    prob = case.prob
    rot, lin = rotation(5, improper)
    d_in, d_sh, d_out = (dmat(ir, rot, improper) for ir in (prob.ins, prob.sh, prob.out))
    plan = cg.plan_for(case.spec, dtype)
    rp, col = dev(case.row_ptr, device), dev(case.col, device)
    tr = cg.graph_transpose(rp, col)
    x64, v64, g64 = (a.astype(np.float64) for a in (case.x, case.vec, case.g))
    w = dev(case.w, device)

    def run(x, vec, g):
        y = cg.spherical_harmonics(case.spec.lmax_sh, dev(cast(vec, dtype), device))
        xd = dev(cast(x, dtype), device)
        out = cg.conv_forward(plan, rp, col, xd, y, w)
        grads = cg.conv_backward(plan, rp, col, tr, xd, y, w, dev(cast(g, dtype), device))
        torch.cuda.synchronize()
        return [host(out), host(y)] + [host(t) for t in grads]

    out, y, dx, dy, dw = run(x64, v64, g64)
    out2, y2, dx2, dy2, dw2 = run(x64 @ d_in.T, v64 @ lin.T, g64 @ d_out.T)
    assert rel_l2(y2, y @ d_sh.T) <= BAR[dtype]
    assert rel_l2(out2, out @ d_out.T) <= BAR[dtype]
    assert rel_l2(dx2, dx @ d_in.T) <= BAR[dtype]
    assert rel_l2(dy2, dy @ d_sh.T) <= BAR[dtype]
    assert rel_l2(dw2, dw) <= BAR[dtype]


@pytest.mark.parametrize("improper", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_uvu_conv_double_backward_equivariance(device, dtype, improper):
    """Double backward: with the upstream gradients rotated like what they multiply (gg_x by
    D_in, gg_y by D_sh, gg_w unchanged), grad_x, grad_y and grad_grad_out rotate by D_in, D_sh and
    D_out, and grad_w does not change."""
    import torch
    case = ConvCase(UVU["mixed-mul"], dtype, seed=72)
    prob = case.prob
    rot, lin = rotation(6, improper)
    d_in, d_sh, d_out = (dmat(ir, rot, improper) for ir in (prob.ins, prob.sh, prob.out))
    plan = cg.plan_for(case.spec, dtype)
    rp, col = dev(case.row_ptr, device), dev(case.col, device)
    tr = cg.graph_transpose(rp, col)
    rng = np.random.default_rng(8)
    ggx, ggy, ggw = (rng.standard_normal(s) for s in (case.x.shape, (case.E, prob.d_sh), case.w.shape))
    x64, v64, g64 = (a.astype(np.float64) for a in (case.x, case.vec, case.g))
    w = dev(case.w, device)

    def run(x, vec, g, gx, gy):
        y = cg.spherical_harmonics(case.spec.lmax_sh, dev(cast(vec, dtype), device))
        res = cg.conv_double_backward(plan, rp, col, tr, dev(cast(x, dtype), device), y, w,
                                      dev(cast(g, dtype), device), dev(cast(gx, dtype), device),
                                      dev(cast(gy, dtype), device), dev(cast(ggw, dtype), device))
        torch.cuda.synchronize()
        return [host(t) for t in res]

    a = run(x64, v64, g64, ggx, ggy)
    b = run(x64 @ d_in.T, v64 @ lin.T, g64 @ d_out.T, ggx @ d_in.T, ggy @ d_sh.T)
    assert rel_l2(b[0], a[0] @ d_in.T) <= BAR[dtype]
    assert rel_l2(b[1], a[1] @ d_sh.T) <= BAR[dtype]
    assert rel_l2(b[2], a[2]) <= BAR[dtype]
    assert rel_l2(b[3], a[3] @ d_out.T) <= BAR[dtype]


UVW_CONV = ("5x0e+3x1o+7x2e+2x3o", 3, "6x0e+4x1o+3x2e+2x1e+1x3o+17x2o", 61, 1_777)


@pytest.mark.parametrize("improper", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_uvw_conv_forward_backward_equivariance(device, dtype, improper):
    import torch
    ins, lmax, outs, n, e = UVW_CONV
    prob = oirreps.build_problem(ins, oirreps.sh_irreps(lmax), outs, "uvw")
    st = synth.streams(73)
    row_ptr, col = synth.uniform_graph(n, e, synth.rng(st["graph"]))
    x64 = synth.normal(st["x"], (n, prob.d_in))
    v64 = synth.normal(st["vec"], (e, 3))
    g64 = synth.normal(st["sample"], (n, prob.d_out))
    rot, lin = rotation(7, improper)
    d_in, d_sh, d_out = (dmat(ir, rot, improper) for ir in (prob.ins, prob.sh, prob.out))
    plan = cg.Plan(ins, cg.sh_irreps(lmax), outs, "uvw", dtype)
    rp, cl = dev(row_ptr, device), dev(col, device)
    tr = cg.graph_transpose(rp, cl)
    w = dev(cast(synth.normal(st["w"], (prob.weight_numel,)), dtype), device)

    def run(x, vec, g):
        y = cg.spherical_harmonics(lmax, dev(cast(vec, dtype), device))
        xd = dev(cast(x, dtype), device)
        out = cg.conv_forward(plan, rp, cl, xd, y, w)
        grads = cg.conv_backward(plan, rp, cl, tr, xd, y, w, dev(cast(g, dtype), device))
        torch.cuda.synchronize()
        return [host(out)] + [host(t) for t in grads]

    out, dx, dy, dw = run(x64, v64, g64)
    out2, dx2, dy2, dw2 = run(x64 @ d_in.T, v64 @ lin.T, g64 @ d_out.T)
    assert rel_l2(out2, out @ d_out.T) <= BAR[dtype]
    assert rel_l2(dx2, dx @ d_in.T) <= BAR[dtype]
    assert rel_l2(dy2, dy @ d_sh.T) <= BAR[dtype]
    assert rel_l2(dw2, dw) <= BAR[dtype]


@pytest.mark.parametrize("improper", [False, True])
def test_batched_high_l_uvw_equivariance(device, improper):
    """The l <= 7 dense-mixing product (the high-L batch's irreps, 97 rows), forward and backward."""
    import torch
    spec = synth.WORKLOADS["c4"]
    prob = oirreps.build_problem(spec.in_irreps, oirreps.sh_irreps(spec.lmax_sh), spec.out_irreps, "uvw")
    plan = cg.plan_for(spec, "f32")
    st = synth.streams(74)
    B = 97
    x64 = synth.normal(st["x"], (B, prob.d_in))
    v64 = synth.normal(st["vec"], (B, 3))
    g64 = synth.normal(st["sample"], (B, prob.d_out))
    w = dev(cast(synth.normal(st["w"], (prob.weight_numel,), 0.25), "f32"), device)
    rot, lin = rotation(9, improper)
    d_in, d_sh, d_out = (dmat(ir, rot, improper) for ir in (prob.ins, prob.sh, prob.out))

    def run(x, vec, g):
        y = cg.spherical_harmonics(spec.lmax_sh, dev(cast(vec, "f32"), device))
        xd = dev(cast(x, "f32"), device)
        out = cg.tp_forward(plan, xd, y, w)
        grads = cg.tp_backward(plan, xd, y, w, dev(cast(g, "f32"), device))
        torch.cuda.synchronize()
        return [host(out)] + [host(t) for t in grads]

    out, dx, dy, dw = run(x64, v64, g64)
    out2, dx2, dy2, dw2 = run(x64 @ d_in.T, v64 @ lin.T, g64 @ d_out.T)
    assert rel_l2(out2, out @ d_out.T) <= BAR["f32"]
    assert rel_l2(dx2, dx @ d_in.T) <= BAR["f32"]
    assert rel_l2(dy2, dy @ d_sh.T) <= BAR["f32"]
    assert rel_l2(dw2, dw) <= BAR["f32"]
