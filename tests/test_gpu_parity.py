"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: rel-L2 <= 1e-4 (fp32), <= 1e-10 (fp64) per output tensor; integer
arrays bit-exact; outputs bitwise repeatable.
"""
import numpy as np
import pytest

from clebsch_gordan_tensor_cgtp_amd import binding as cg
from clebsch_gordan_tensor_cgtp_amd import synth
from oracle import irreps as oirreps
from oracle import loops, ref
from oracle import sh as osh

from cases import TOL, ConvCase, edge_case_graph, rel_l2, to_device

pytestmark = pytest.mark.gpu

SMALL = {
    # name: (spec, dtypes)
    "nequip-small": (synth.scaled(synth.CONV_NEQUIP, 300, 12_001), ("f32", "f64")),
    "stream-small": (synth.scaled(synth.CONV_STREAM, 257, 9_001), ("f32", "f64")),
    "mace-small": (synth.scaled(synth.CONV_MACE, 97, 2_999), ("f32", "f64")),
    "mixed-mul": (synth.ConvSpec("mixed", 61, 1_777, "5x0e+3x1o+7x2e+2x3o", 3, 3), ("f32", "f64")),
    "mul4": (synth.ConvSpec("mul4", 53, 1_201, "4x0e+4x1o", 2, 2), ("f32",)),
    "mul80": (synth.ConvSpec("mul80", 41, 997, "80x0e+80x1o", 1, 1), ("f32",)),
}
CASES = [(k, d) for k, (_, ds) in SMALL.items() for d in ds]


def run_gpu(case, device, need=(True, True, True)):
    import torch
    plan = cg.plan_for(case.spec, case.dtype)
    d = to_device(case, device)
    y = cg.spherical_harmonics(case.spec.lmax_sh, d["vec"])
    out = cg.conv_forward(plan, d["row_ptr"], d["col"], d["x"], y, d["w"])
    tr = cg.graph_transpose(d["row_ptr"], d["col"])
    grads = cg.conv_backward(plan, d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"], need=need)
    torch.cuda.synchronize()
    return d, y, out, tr, grads


@pytest.mark.parametrize("lmax", range(8))
@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_spherical_harmonics(device, lmax, dtype):
    import torch
    vec = synth.normal(synth.streams(lmax)["vec"], (4099, 3), dtype=np.float32 if dtype == "f32" else np.float64)
    got = cg.spherical_harmonics(lmax, torch.from_numpy(vec).to(device)).cpu().numpy()
    want = osh.real_sh_all(lmax, vec.astype(np.float64))
    assert rel_l2(got, want) <= TOL[dtype]
    assert np.abs(got - want).max() <= (1e-5 if dtype == "f32" else 1e-12) * max(1, lmax)


@pytest.mark.parametrize("kind", ["uniform", "empty", "heavy", "isolated", "selfdup"])
def test_transpose_bit_exact(device, kind):
    import torch
    rng = np.random.default_rng(3)
    if kind == "uniform":
        row_ptr, col = synth.uniform_graph(1000, 40_000, rng)
    else:
        row_ptr, col = edge_case_graph(kind, 700, rng)
    t = lambda a: torch.from_numpy(a).to(device)
    trp, te, td = (a.cpu().numpy() for a in cg.graph_transpose(t(row_ptr), t(col)))
    order = np.argsort(col, kind="stable")
    want_ptr = np.concatenate([[0], np.cumsum(np.bincount(col, minlength=len(row_ptr) - 1))])
    dst = np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr))
    assert np.array_equal(trp, want_ptr)
    assert np.array_equal(te, order)
    assert np.array_equal(td, dst[order])


@pytest.mark.parametrize("kind", ["uniform", "powerlaw", "heavy", "empty"])
def test_graph_order_and_ordered_forward(device, kind):
    """Heavy-first schedule: bit-exact vs a numpy stable sort; the forward result is unchanged bitwise."""
    import torch
    rng = np.random.default_rng(8)
    if kind == "uniform":
        graph = synth.uniform_graph(3000, 90_000, rng)
    elif kind == "powerlaw":
        graph = synth.powerlaw_graph(4000, 120_000, 2.0, 500, rng)
    else:
        graph = edge_case_graph(kind, 900, rng)
    row_ptr, col = graph
    deg = np.diff(row_ptr).astype(np.int64)
    bucket = np.floor(np.log2(deg + 1)).astype(np.int64)
    want = np.argsort(-bucket, kind="stable")
    rp = torch.from_numpy(row_ptr).to(device)
    order = cg.graph_order(rp).cpu().numpy()
    assert np.array_equal(order, want)
    spec = synth.ConvSpec("order-" + kind, len(row_ptr) - 1, len(col), "32x0e+32x1o+32x2e", 2, 2)
    case = ConvCase(spec, "f32", seed=3, graph=graph)
    plan = cg.plan_for(spec, "f32")
    d = to_device(case, device)
    y = cg.spherical_harmonics(2, d["vec"])
    a = cg.conv_forward(plan, d["row_ptr"], d["col"], d["x"], y, d["w"])
    b = cg.conv_forward(plan, d["row_ptr"], d["col"], d["x"], y, d["w"], order=torch.from_numpy(order).to(device))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("name,dtype", CASES)
def test_conv_forward_backward_small(device, name, dtype):
    spec = SMALL[name][0]
    case = ConvCase(spec, dtype, seed=1)
    d, y, out, tr, (gx, gy, gw) = run_gpu(case, device)
    assert rel_l2(y.cpu().numpy(), case.y_oracle()) <= TOL[dtype]
    assert rel_l2(out.cpu().numpy(), case.oracle_forward()) <= TOL[dtype]
    dx, eidx, dy, dw = case.oracle_backward()
    assert np.array_equal(eidx, np.arange(case.E))
    assert rel_l2(gx.cpu().numpy(), dx) <= TOL[dtype]
    assert rel_l2(gy.cpu().numpy(), dy) <= TOL[dtype]
    assert rel_l2(gw.cpu().numpy(), dw) <= TOL[dtype]


@pytest.mark.parametrize("kind", ["empty", "heavy", "isolated", "selfdup"])
def test_conv_edge_cases(device, kind):
    spec = synth.ConvSpec("edge-" + kind, 700, 0, "32x0e+32x1o+32x2e", 2, 2)
    graph = edge_case_graph(kind, 700, np.random.default_rng(5))
    case = ConvCase(spec, "f32", seed=2, graph=graph)
    d, y, out, tr, (gx, gy, gw) = run_gpu(case, device)
    out_h = out.cpu().numpy()
    want = case.oracle_forward()
    deg = np.diff(case.row_ptr)
    assert np.all(out_h[deg == 0] == 0)
    if case.E == 0:
        assert np.all(out_h == 0) and np.all(gx.cpu().numpy() == 0)
        return
    assert rel_l2(out_h, want) <= TOL["f32"]
    dx, eidx, dy, dw = case.oracle_backward()
    assert rel_l2(gx.cpu().numpy(), dx) <= TOL["f32"]
    assert rel_l2(gy.cpu().numpy(), dy) <= TOL["f32"]
    assert rel_l2(gw.cpu().numpy(), dw) <= TOL["f32"]


@pytest.mark.parametrize("kind", ["empty", "heavy", "isolated", "selfdup"])
@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_split_plan_edge_cases(device, kind, dtype):
    """A plan split into several path groups (128 channels of l <= 3, SH l <= 3): its receiver
    pass takes two edges per loop iteration and its sender pass loads the next edge's operands as
    the current edge frees them; rows of 0, 1 and 2 edges, a 5,000-edge row, self-loops and
    duplicates exercise the ends of both loops."""
    spec = synth.ConvSpec("split-edge-" + kind, 300, 0, "128x0e+128x1o+128x2e+128x3o", 3, 3)
    graph = edge_case_graph(kind, 300, np.random.default_rng(6))
    case = ConvCase(spec, dtype, seed=3, graph=graph)
    assert "e += 2 * stride" in cg.plan_for(spec, dtype).source  # the two-edge receiver loop
    print(f"[split edge] {kind} {dtype} E={case.E}", flush=True)
    d, y, out, tr, (gx, gy, gw) = run_gpu(case, device)
    out_h = out.cpu().numpy()
    deg = np.diff(case.row_ptr)
    assert np.all(out_h[deg == 0] == 0)
    if case.E == 0:
        assert np.all(out_h == 0) and np.all(gx.cpu().numpy() == 0)
        return
    assert rel_l2(out_h, case.oracle_forward()) <= TOL[dtype]
    dx, _, dy, dw = case.oracle_backward()
    assert rel_l2(gx.cpu().numpy(), dx) <= TOL[dtype]
    assert rel_l2(gy.cpu().numpy(), dy) <= TOL[dtype]
    assert rel_l2(gw.cpu().numpy(), dw) <= TOL[dtype]


def test_backward_optional_outputs(device):
    import torch
    case = ConvCase(synth.scaled(synth.CONV_NEQUIP, 100, 3_000), "f32", seed=4)
    d, y, out, tr, full = run_gpu(case, device)
    for need in [(True, False, False), (False, True, False), (False, False, True)]:
        part = cg.conv_backward(cg.plan_for(case.spec, "f32"), d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"],
                                need=need)
        torch.cuda.synchronize()
        for a, b, n in zip(full, part, need):
            if n:
                assert torch.equal(a, b)
            else:
                assert b is None


def test_determinism_bitwise(device):
    import torch
    case = ConvCase(synth.scaled(synth.CONV_NEQUIP, 400, 20_000), "f32", seed=6)
    r1 = run_gpu(case, device)
    r2 = run_gpu(case, device)
    assert torch.equal(r1[2], r2[2])
    for a, b in zip(r1[4], r2[4]):
        assert torch.equal(a, b)


def test_no_device_allocation(device):
    """The library allocates nothing: with caller-owned outputs memory_allocated is unchanged."""
    import torch
    case = ConvCase(synth.scaled(synth.CONV_NEQUIP, 200, 8_000), "f32", seed=7)
    plan = cg.plan_for(case.spec, "f32")
    d = to_device(case, device)
    y = torch.empty((case.E, plan.d_sh), dtype=torch.float32, device=device)
    out = torch.empty((case.N, plan.d_out), dtype=torch.float32, device=device)
    tr = (torch.empty(case.N + 1, dtype=torch.int32, device=device),
          torch.empty(case.E, dtype=torch.int32, device=device), torch.empty(case.E, dtype=torch.int32, device=device))
    gx, gy, gw = torch.empty_like(d["x"]), torch.empty_like(y), torch.empty_like(d["w"])

    def calls():
        cg.spherical_harmonics(2, d["vec"], out=y)
        cg.conv_forward(plan, d["row_ptr"], d["col"], d["x"], y, d["w"], out=out)
        cg.graph_transpose(d["row_ptr"], d["col"], *tr)
        cg.conv_backward(plan, d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"], gx, gy, gw)

    calls()  # first call on the device loads the plan's code object
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(device)
    free_before = torch.cuda.mem_get_info(device)[0]
    for _ in range(3):
        calls()
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated(device) == before
    assert torch.cuda.mem_get_info(device)[0] >= free_before - (2 << 20)


# --------------------------------------------------------------------------- batched product

@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("in_irreps,lmax,B", [("4x0e+4x1o", 2, 1024), ("32x0e+32x1o+32x2e", 2, 777),
                                              ("5x0e+3x1o+7x2e+2x3o", 3, 301)])
def test_tp_forward_uvu(device, dtype, in_irreps, lmax, B):
    import torch
    out_ir = oirreps.per_path_out_irreps(in_irreps, lmax, lmax)
    prob = oirreps.build_problem(in_irreps, oirreps.sh_irreps(lmax), out_ir, "uvu")
    plan = cg.plan_create(in_irreps, oirreps.sh_irreps(lmax), out_ir, "uvu", dtype)
    st = synth.streams(11)
    npdt = np.float32 if dtype == "f32" else np.float64
    x = synth.normal(st["x"], (B, prob.d_in), dtype=npdt)
    vec = synth.normal(st["vec"], (B, 3), dtype=npdt)
    w = synth.normal(st["w"], (B, prob.weight_numel), dtype=npdt)
    t = lambda a: torch.from_numpy(a).to(device)
    y = cg.spherical_harmonics(lmax, t(vec))
    out = cg.tp_forward(plan, t(x), y, t(w)).cpu().numpy()
    want = ref.tp_forward(prob, x, osh.real_sh_all(lmax, vec.astype(np.float64)), w)
    assert rel_l2(out, want) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("in_irreps,lmax,B", [("4x0e+4x1o", 2, 1024), ("32x0e+32x1o+32x2e", 2, 777),
                                              ("5x0e+3x1o+7x2e+2x3o", 3, 301), ("128x0e+128x1o+128x2e+128x3o", 3, 97),
                                              ("80x0e+80x1o", 1, 33)])
def test_tp_backward_uvu(device, dtype, in_irreps, lmax, B):
    """Batched backward vs the oracle's convolution backward on the identity graph (row b is its
    own sender and receiver); optional outputs give the same bits."""
    import torch
    out_ir = oirreps.per_path_out_irreps(in_irreps, lmax, lmax)
    prob = oirreps.build_problem(in_irreps, oirreps.sh_irreps(lmax), out_ir, "uvu")
    plan = cg.plan_create(in_irreps, oirreps.sh_irreps(lmax), out_ir, "uvu", dtype)
    st = synth.streams(12)
    npdt = np.float32 if dtype == "f32" else np.float64
    x = synth.normal(st["x"], (B, prob.d_in), dtype=npdt)
    vec = synth.normal(st["vec"], (B, 3), dtype=npdt)
    w = synth.normal(st["w"], (B, prob.weight_numel), dtype=npdt)
    g = synth.normal(st["sample"], (B, prob.d_out), dtype=npdt)
    t = lambda a: torch.from_numpy(a).to(device)
    y = cg.spherical_harmonics(lmax, t(vec))
    gx, gy, gw = cg.tp_backward(plan, t(x), y, t(w), t(g))
    torch.cuda.synchronize()
    ident = np.arange(B + 1)
    want = ref.conv_backward(prob, ident, np.arange(B), x, osh.real_sh_all(lmax, vec.astype(np.float64)), w, g)
    for got, exp in zip((gx, gy, gw), want):
        assert rel_l2(got.cpu().numpy(), exp) <= TOL[dtype]
    for k in range(3):
        part = cg.tp_backward(plan, t(x), y, t(w), t(g), need=tuple(i == k for i in range(3)))
        torch.cuda.synchronize()
        assert torch.equal(part[k], (gx, gy, gw)[k])


# --------------------------------------------------------------------------- uvw (dense mixing on MFMA)

def _uvw_case(in_irreps, lmax, out_irreps, B, dtype, seed=13):
    prob = oirreps.build_problem(in_irreps, oirreps.sh_irreps(lmax), out_irreps, "uvw")
    st = synth.streams(seed)
    npdt = np.float32 if dtype == "f32" else np.float64
    x = synth.normal(st["x"], (B, prob.d_in), dtype=npdt)
    vec = synth.normal(st["vec"], (B, 3), dtype=npdt)
    # W_p ~ N(0,1)/sqrt(mul_in * paths into the output irrep)
    fan = {}
    for p in prob.paths:
        fan[p.slot] = fan.get(p.slot, 0) + prob.ins[p.i1].mul
    w = synth.normal(st["w"], (prob.weight_numel,), dtype=np.float64)
    for p in prob.paths:
        n = prob.ins[p.i1].mul * prob.out[p.slot].mul
        w[p.w_off:p.w_off + n] /= np.sqrt(fan[p.slot])
    return prob, x, vec, w.astype(npdt)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("in_irreps,lmax,out_irreps,B", [
    (synth.TP_HIGHL.in_irreps, 7, synth.TP_HIGHL.out_irreps, 333),
    ("3x0e+5x1o+2x2e", 2, "4x0e+7x1o+3x2e+2x1e+16x2o", 77),
    ("16x0e+16x1o", 1, "16x0e+16x1o+16x1e", 1),
    # output multiplicities above 16: 16-wide output tiles, ragged last tile, mixed tile counts
    ("20x0e+5x1o", 1, "33x0e+17x1o+3x1e", 77),
    ("8x0e+8x1o+8x2e", 2, "32x0e+32x1o+32x2e", 300),
])
def test_tp_forward_uvw(device, dtype, in_irreps, lmax, out_irreps, B):
    import torch
    prob, x, vec, w = _uvw_case(in_irreps, lmax, out_irreps, B, dtype)
    plan = cg.plan_create(in_irreps, oirreps.sh_irreps(lmax), out_irreps, "uvw", dtype)
    t = lambda a: torch.from_numpy(a).to(device)
    y = cg.spherical_harmonics(lmax, t(vec))
    out = cg.tp_forward(plan, t(x), y, t(w)).cpu().numpy()
    want = loops.uvw_forward(loops.Tables(prob), x.astype(np.float64),
                             osh.real_sh_all(lmax, vec.astype(np.float64)), w.astype(np.float64))
    assert rel_l2(out, want) <= TOL[dtype]


def test_tp_forward_uvw_full_size_sampled(device):
    """The high-L workload at its full batch (50,000 rows), checked on a seeded row sample."""
    import torch
    spec = synth.TP_HIGHL
    prob, x, vec, w = _uvw_case(spec.in_irreps, spec.lmax_sh, spec.out_irreps, spec.batch, "f32", seed=0)
    plan = cg.plan_for(spec, "f32")
    t = lambda a: torch.from_numpy(a).to(device)
    y = cg.spherical_harmonics(spec.lmax_sh, t(vec))
    out = cg.tp_forward(plan, t(x), y, t(w))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1).choice(spec.batch, 2048, replace=False))
    rows = np.unique(np.concatenate([rows, [0, spec.batch - 1]]))
    want = loops.uvw_forward(loops.Tables(prob), x[rows].astype(np.float64),
                             osh.real_sh_all(spec.lmax_sh, vec[rows].astype(np.float64)), w.astype(np.float64))
    assert rel_l2(out.cpu().numpy()[rows], want) <= TOL["f32"]


# --------------------------------------------------------------------------- uvw batched backward

UVB_CASES = [
    ("3x0e+2x1o+2x2e", 2, "2x0e+3x1o+2x2e+1x1e+2x2o", 1000, ("f32", "f64")),
    ("16x0e+16x1o+16x2e", 2, "16x0e+16x1o+16x2e+16x1e+16x2o", 777, ("f32", "f64")),
    ("5x0e+3x1o+7x2e+2x3o", 3, "6x0e+4x1o+3x2e+2x1e+1x3o+9x2o", 301, ("f32",)),
    ("+".join(f"16x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(6)), 5,
     "+".join(f"16x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(6)), 200, ("f32",)),
    # multiplicities above 16: the convolution backward on the identity graph
    ("20x0e+5x1o", 1, "33x0e+17x1o+3x1e", 77, ("f32", "f64")),
    ("32x0e+32x1o", 1, "32x0e+32x1o+32x1e", 300, ("f32",)),
]
WIDE = UVB_CASES[-2]


def _uvb_run(device, ins, lmax, outs, B, dtype, seed=61, need=(True, True, True)):
    import torch
    prob = oirreps.build_problem(ins, oirreps.sh_irreps(lmax), outs, "uvw")
    plan = cg.plan_create(ins, oirreps.sh_irreps(lmax), outs, "uvw", dtype)
    st = synth.streams(seed)
    npdt = np.float32 if dtype == "f32" else np.float64
    x = synth.normal(st["x"], (B, prob.d_in), dtype=npdt)
    vec = synth.normal(st["vec"], (B, 3), dtype=npdt)
    w = synth.normal(st["w"], (prob.weight_numel,), 0.25, dtype=npdt)
    g = synth.normal(st["sample"], (B, prob.d_out), dtype=npdt)
    t = lambda a: torch.from_numpy(a).to(device)
    y = cg.spherical_harmonics(lmax, t(vec))
    got = cg.tp_backward(plan, t(x), y, t(w), t(g), need=need)
    torch.cuda.synchronize()
    return prob, plan, x, vec, w, g, got


@pytest.mark.parametrize("ins,lmax,outs,B,dtype", [(c[0], c[1], c[2], c[3], d) for c in UVB_CASES for d in c[4]])
def test_tp_backward_uvw(device, ins, lmax, outs, B, dtype):
    prob, plan, x, vec, w, g, (gx, gy, gw) = _uvb_run(device, ins, lmax, outs, B, dtype)
    y = osh.real_sh_all(lmax, vec.astype(np.float64))
    f64 = lambda a: np.asarray(a, np.float64)
    dx, dy, dw = loops.uvw_backward(loops.Tables(prob), f64(x), y, f64(w), f64(g), np.arange(B), np.arange(B))
    assert rel_l2(gx.cpu().numpy(), dx) <= TOL[dtype]
    assert rel_l2(gy.cpu().numpy(), dy) <= TOL[dtype]
    assert rel_l2(gw.cpu().numpy(), dw) <= TOL[dtype]


def test_tp_backward_uvw_wide_subsets_and_empty_batch(device):
    """Multiplicities above 16: each gradient alone gives the bits of the full call, and an empty
    batch gives a zero weight gradient."""
    import torch
    ins, lmax, outs, B, _ = WIDE
    full = _uvb_run(device, ins, lmax, outs, B, "f32")[-1]
    for k in range(3):
        need = tuple(j == k for j in range(3))
        part = _uvb_run(device, ins, lmax, outs, B, "f32", need=need)[-1]
        assert torch.equal(part[k], full[k])
    plan = cg.plan_create(ins, oirreps.sh_irreps(lmax), outs, "uvw", "f32")
    e = lambda *sh: torch.empty(sh, device=device)
    gw = torch.full((plan.weight_numel,), float("nan"), device=device)
    cg.tp_backward(plan, e(0, plan.d_x), e(0, plan.d_sh), e(plan.weight_numel), e(0, plan.d_out),
                   grad_w=gw, need=(False, False, True))
    torch.cuda.synchronize()
    assert torch.count_nonzero(gw).item() == 0


def test_tp_backward_uvw_outputs_and_repeat_bitwise(device):
    import torch
    ins, lmax, outs = "16x0e+16x1o+16x2e", 2, "16x0e+16x1o+16x2e+16x1e+16x2o"
    full = _uvb_run(device, ins, lmax, outs, 4097, "f32")[-1]
    again = _uvb_run(device, ins, lmax, outs, 4097, "f32")[-1]
    for a, b in zip(full, again):
        assert torch.equal(a, b)
    for k in range(3):
        part = _uvb_run(device, ins, lmax, outs, 4097, "f32", need=tuple(i == k for i in range(3)))[-1]
        assert torch.equal(part[k], full[k])
        assert all(part[i] is None for i in range(3) if i != k)


def test_tp_backward_uvw_full_size_sampled(device):
    """The high-L batch (50,000 rows, l <= 7): dx, dY on sampled rows, dW over every row."""
    spec = synth.TP_HIGHL
    prob = oirreps.build_problem(spec.in_irreps, oirreps.sh_irreps(spec.lmax_sh), spec.out_irreps, "uvw")
    B = spec.batch
    _, plan, x, vec, w, g, (gx, gy, gw) = _uvb_run(device, spec.in_irreps, spec.lmax_sh, spec.out_irreps, B, "f32",
                                                   seed=62)
    rows = np.unique(np.concatenate([np.random.default_rng(63).choice(B, 200, replace=False), [0, B - 1]]))
    f64 = lambda a: np.asarray(a, np.float64)
    y = osh.real_sh_all(spec.lmax_sh, vec.astype(np.float64))
    dx, dy, dw = loops.uvw_backward(loops.Tables(prob), f64(x), y, f64(w), f64(g), rows, np.arange(B))
    assert rel_l2(gx.cpu().numpy()[rows], dx) <= TOL["f32"]
    assert rel_l2(gy.cpu().numpy()[rows], dy) <= TOL["f32"]
    assert rel_l2(gw.cpu().numpy(), dw) <= TOL["f32"]
