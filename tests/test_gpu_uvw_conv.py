"""GPU parity of the convolution in uvw mode (shared weights, MFMA multiplicity mixing).

Bars: rel-L2 <= 1e-4 (fp32), <= 1e-10 (fp64) against the oracle (oracle.ref.conv_forward /
oracle.loops.conv_forward_uvw_rows, pinned by a dense einsum, the identity graph, linearity and
equivariance); the receiver schedule does not change a bit; receivers without edges get zeros.
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
    "high-l": (LADDER5, 5, LADDER5, 37, 401, ("f32", "f64")),   # slots span several launches
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
            "w": synth.normal(st["w"], (prob.weight_numel,), dtype=npdt)}


def run_gpu(c, device, ordered=False):
    import torch
    plan = cg.Plan(c["ins"], cg.sh_irreps(c["lmax"]), c["outs"], "uvw", c["dtype"])
    t = {k: torch.from_numpy(np.ascontiguousarray(c[k])).to(device) for k in ("row_ptr", "col", "x", "vec", "w")}
    y = cg.spherical_harmonics(c["lmax"], t["vec"])
    order = cg.graph_order(t["row_ptr"]) if ordered else None
    out = cg.conv_forward(plan, t["row_ptr"], t["col"], t["x"], y, t["w"], order=order)
    torch.cuda.synchronize()
    return out


def oracle(c):
    y = osh.real_sh_all(c["lmax"], c["vec"].astype(np.float64))
    n = len(c["row_ptr"]) - 1
    return loops.conv_forward_uvw_rows(loops.Tables(c["prob"]), c["row_ptr"], c["col"], c["x"].astype(np.float64), y,
                                       c["w"].astype(np.float64), np.arange(n))


@pytest.mark.parametrize("name,dtype", PARAMS)
def test_uvw_conv_parity(device, name, dtype):
    c = make_case(name, dtype, seed=41)
    got = run_gpu(c, device, ordered=True).cpu().numpy()
    assert rel_l2(got, oracle(c)) <= TOL[dtype]


@pytest.mark.parametrize("kind", ["empty", "heavy", "isolated", "selfdup"])
def test_uvw_conv_edge_cases(device, kind):
    c = make_case("nequip-32", "f32", seed=42, graph=edge_case_graph(kind, 333, np.random.default_rng(9)))
    got = run_gpu(c, device).cpu().numpy()
    deg = np.diff(c["row_ptr"])
    assert np.all(got[deg == 0] == 0)
    if len(c["col"]):
        assert rel_l2(got, oracle(c)) <= TOL["f32"]


def test_uvw_conv_schedule_and_repeat_bitwise(device):
    import torch
    c = make_case("nequip-32", "f32", seed=43,
                  graph=synth.powerlaw_graph(1000, 30_000, 2.0, 400, np.random.default_rng(3)))
    a = run_gpu(c, device, ordered=False)
    b = run_gpu(c, device, ordered=True)
    again = run_gpu(c, device, ordered=True)
    assert torch.equal(a, b) and torch.equal(b, again)
    assert rel_l2(a.cpu().numpy(), oracle(c)) <= TOL["f32"]
