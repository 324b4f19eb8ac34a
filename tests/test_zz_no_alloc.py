"""The allocation-free batched backward (cgtp_tp_backward_noalloc) against cgtp_tp_backward.

Both run the same kernels; the only difference is where the temporary memory lives (the
library's fixed device scratch instead of a caller workspace), so the results must agree to the
parity bar (they are in fact bitwise equal).  Two calls in a row, the second with a smaller
batch, so that the second reads a scratch array that still holds the first call's values.  After
the first call on the device, a call must not change the device's free memory.
"""
import ctypes

import numpy as np
import pytest

from clebsch_gordan_tensor_cgtp_amd import binding as cg
from clebsch_gordan_tensor_cgtp_amd import synth

from cases import TOL, rel_l2

pytestmark = pytest.mark.gpu

PLANS = {
    # name: (in irreps, SH lmax, out irreps, batches)
    "high-l": (synth.TP_HIGHL.in_irreps, 7, synth.TP_HIGHL.out_irreps, (3001, 700)),
    "wide-mul": ("32x0e+24x1o", 2, "32x0e+20x1o+17x2e+8x1e", (1500, 333)),
}


def inputs(plan, B, dtype, seed, device):
    import torch
    npdt = np.float32 if dtype == "f32" else np.float64
    st = synth.streams(seed)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    x = t(synth.normal(st["x"], (B, plan.d_x), dtype=npdt))
    vec = t(synth.normal(st["vec"], (B, 3), dtype=npdt))
    w = t(synth.normal(st["w"], (plan.weight_numel,), 0.25, dtype=npdt))
    g = t(synth.normal(st["sample"], (B, plan.d_out), dtype=npdt))
    return x, vec, w, g


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("name", sorted(PLANS))
def test_noalloc_backward_matches_workspace_backward(device, name, dtype):
    import torch
    ins, lmax, outs, batches = PLANS[name]
    plan = cg.Plan(ins, cg.sh_irreps(lmax), outs, "uvw", dtype)
    for call, B in enumerate(batches):
        print(f"[noalloc] {name} {dtype} call {call} B={B}", flush=True)
        x, vec, w, g = inputs(plan, B, dtype, 100 + call, device)
        y = cg.spherical_harmonics(lmax, vec)
        want = cg.tp_backward(plan, x, y, w, g)
        got = (torch.empty_like(x), torch.empty_like(y), torch.empty_like(w))
        torch.cuda.synchronize()
        if call > 0:
            free0 = torch.cuda.mem_get_info()[0]
        cg.tp_backward_noalloc(plan, x, y, w, g, *got)
        torch.cuda.synchronize()
        if call > 0:
            assert torch.cuda.mem_get_info()[0] == free0
        for a, b in zip(got, want):
            a, b = a.cpu().numpy(), b.cpu().numpy()
            assert rel_l2(a, b) <= TOL[dtype]
            assert np.array_equal(a, b)


def test_noalloc_backward_uvu_and_limits(device):
    """uvu plans need no scratch; a batch whose workspace exceeds the fixed scratch is refused
    before any launch (CGTP_ERR_UNSUPPORTED), and a gradient subset works."""
    import torch
    spec = synth.TP_SMALL
    plan = cg.plan_for(spec, "f32")
    B = 1024
    st = synth.streams(3)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    x = t(synth.normal(st["x"], (B, plan.d_x), dtype=np.float32))
    y = cg.spherical_harmonics(spec.lmax_sh, t(synth.normal(st["vec"], (B, 3), dtype=np.float32)))
    w = t(synth.normal(st["w"], (B, plan.weight_numel), dtype=np.float32))
    g = t(synth.normal(st["sample"], (B, plan.d_out), dtype=np.float32))
    want = cg.tp_backward(plan, x, y, w, g)
    got = (torch.empty_like(x), None, torch.empty_like(w))
    cg.tp_backward_noalloc(plan, x, y, w, g, *got)
    torch.cuda.synchronize()
    assert np.array_equal(got[0].cpu().numpy(), want[0].cpu().numpy())
    assert np.array_equal(got[2].cpu().numpy(), want[2].cpu().numpy())
    # the wide route's workspace grows with B: a large batch is refused, with nothing launched
    wide = cg.Plan(*PLANS["wide-mul"][:1], cg.sh_irreps(2), PLANS["wide-mul"][2], "uvw", "f32")
    big = 2_000_000
    assert cg.tp_backward_workspace_size(wide, big) > 64 << 20
    fake = ctypes.c_void_p(1 << 20)
    st_ = cg.lib().cgtp_tp_backward_noalloc(wide.handle, big, fake, fake, fake, 1, fake, fake, fake, fake,
                                            ctypes.c_void_p(0))
    assert st_ == cg.STATUS_CODES["CGTP_ERR_UNSUPPORTED"]
    assert "scratch" in cg.last_error()
