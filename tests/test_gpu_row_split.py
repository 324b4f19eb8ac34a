"""GPU parity of the receiver-owned passes on graphs that split each receiver row over 1, 2
or 4 waves (the forward and the double backward's receiver pass).

The launch picks the split from N, E and the plan (``Plan.row_split``): it doubles while the
launch has fewer than four waves per wave slot of the chip and every part keeps at least 8 edge
groups of the mean row.  601 receivers with mean degrees 20, 40 and 160 land on 1, 2 and 4
parts with 32 channels in fp32; a 16-channel fp64 plan (four edges per wave step) on 2 and 4.
601 is odd, so a 2-part launch ends in a half-used workgroup whose idle waves must still meet the
part-sum barrier.  Bars: rel-L2 <= 1e-4 (fp32), <= 1e-10 (fp64) against the oracle; the
heavy-first schedule gives the same bits as node order.
"""
import numpy as np
import pytest

from clebsch_gordan_tensor_cgtp_amd import binding as cg
from clebsch_gordan_tensor_cgtp_amd import synth

from cases import TOL, ConvCase, rel_l2, to_device
from test_gpu_double_backward import oracle_dbl, run_dbl, upstream

pytestmark = pytest.mark.gpu

N = 601
SMALL16 = synth.ConvSpec("mul16-l1", N, 0, "16x0e+16x1o", 1, 1)
CASES = [  # (spec, mean degree, dtype, expected waves per row)
    (synth.CONV_NEQUIP, 20, "f32", 1),
    (synth.CONV_NEQUIP, 40, "f32", 2),
    (synth.CONV_NEQUIP, 160, "f32", 4),
    (SMALL16, 72, "f64", 2),
    (SMALL16, 160, "f64", 4),
]
IDS = [f"{c[0].name[:12]}-deg{c[1]}-{c[2]}" for c in CASES]


def case_for(spec, degree, dtype, seed):
    return ConvCase(synth.scaled(spec, N, N * degree), dtype, seed=seed)


@pytest.mark.parametrize("spec,degree,dtype,split", CASES, ids=IDS)
def test_forward_split_rows(device, spec, degree, dtype, split):
    import torch
    case = case_for(spec, degree, dtype, 81)
    plan = cg.plan_for(case.spec, dtype)
    assert plan.row_split(case.N, case.E) == split
    d = to_device(case, device)
    y = cg.spherical_harmonics(case.spec.lmax_sh, d["vec"])
    natural = cg.conv_forward(plan, d["row_ptr"], d["col"], d["x"], y, d["w"])
    ordered = cg.conv_forward(plan, d["row_ptr"], d["col"], d["x"], y, d["w"], order=cg.graph_order(d["row_ptr"]))
    torch.cuda.synchronize()
    assert torch.equal(natural, ordered)
    assert rel_l2(natural.cpu().numpy(), case.oracle_forward()) <= TOL[dtype]


@pytest.mark.parametrize("degree,split", [(40, 2), (160, 4)])
def test_double_backward_receiver_pass_split_rows(device, degree, split):
    case = case_for(synth.CONV_NEQUIP, degree, "f32", 82)
    assert cg.plan_for(case.spec, "f32").row_split(case.N, case.E, double_backward=True) == split
    gg = upstream(case, 82)
    got = run_dbl(case, device, gg, order=True, need=(False, False, False, True))
    want = oracle_dbl(case, gg)
    assert rel_l2(got[3].cpu().numpy(), want[3]) <= TOL["f32"]
