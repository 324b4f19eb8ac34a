"""The library's launches inside a captured HIP graph (torch.cuda.CUDAGraph on torch's current
stream): the library allocates, clears and synchronises nothing, so a step of forward +
backward can be captured once and replayed.  Each replay is checked bitwise against the eager
result for the inputs it ran on, with new inputs written into the captured buffers and eager
work and synchronisations between the replays; the first eager result is also checked against
the oracle."""
import numpy as np
import pytest

from clebsch_gordan_tensor_cgtp_amd import binding as cg
from clebsch_gordan_tensor_cgtp_amd import synth

from cases import TOL, ConvCase, rel_l2, to_device

pytestmark = pytest.mark.gpu


def test_conv_step_replays_match_eager(device):
    import torch
    case = ConvCase(synth.scaled(synth.CONV_NEQUIP, 400, 16_003), "f32", seed=91)
    plan = cg.plan_for(case.spec, "f32")
    d = to_device(case, device)
    y = cg.spherical_harmonics(case.spec.lmax_sh, d["vec"])
    tr = cg.graph_transpose(d["row_ptr"], d["col"])
    order = cg.graph_order(d["row_ptr"])
    out = torch.empty((case.N, plan.d_out), device=device)
    gx, gy, gw = torch.empty_like(d["x"]), torch.empty_like(y), torch.empty_like(d["w"])

    def step():
        cg.conv_forward(plan, d["row_ptr"], d["col"], d["x"], y, d["w"], out=out, order=order)
        cg.conv_backward(plan, d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"], gx, gy, gw)

    def eager_copy():
        step()
        torch.cuda.synchronize()
        return [t.clone() for t in (out, gx, gy, gw)]

    first = eager_copy()  # also loads the module on this device before capture
    assert rel_l2(first[0].cpu().numpy(), case.oracle_forward()) <= TOL["f32"]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for rep in range(3):
        if rep:
            # new inputs in the captured buffers
            d["x"].copy_(torch.from_numpy(rng.standard_normal(tuple(d["x"].shape)).astype(np.float32)).to(device))
            d["g"].copy_(torch.from_numpy(rng.standard_normal(tuple(d["g"].shape)).astype(np.float32)).to(device))
        want = eager_copy()
        for t in (out, gx, gy, gw):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((out, gx, gy, gw), want):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"


def test_batched_forward_replays_match_eager(device):
    import torch
    ins, lmax = "4x0e+4x1o", 2
    out_ir = cg.per_path_out_irreps(ins, lmax, lmax)
    plan = cg.Plan(ins, cg.sh_irreps(lmax), out_ir, "uvu", "f32")
    B = 1024
    st = synth.streams(92)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    x = t(synth.normal(st["x"], (B, plan.d_x), dtype=np.float32))
    y = cg.spherical_harmonics(lmax, t(synth.normal(st["vec"], (B, 3), dtype=np.float32)))
    w = t(synth.normal(st["w"], (B, plan.weight_numel), dtype=np.float32))
    out = torch.empty((B, plan.d_out), device=device)
    cg.tp_forward(plan, x, y, w, out=out)
    torch.cuda.synchronize()
    want = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(4):
            cg.tp_forward(plan, x, y, w, out=out)
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {rep}"
        cg.tp_forward(plan, x, y, w, out=out)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, want)
