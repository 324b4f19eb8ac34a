"""The C ABI on the CPU: every declared symbol is exported, the planner's
bookkeeping and CG blocks agree with the oracle (two independent codes), and
argument errors come back as status codes before any GPU call."""
import ctypes
import os
import re

import numpy as np
import pytest

from clebsch_gordan_tensor_cgtp_amd import binding as cg
from clebsch_gordan_tensor_cgtp_amd import synth
from oracle import cg as ocg
from oracle import irreps as oirreps

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cgtp.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cgtp_[a-z_]+)\s*\(", text)))


def test_header_declares_what_binding_knows():
    assert set(declared_functions()) == set(cg.EXPORTS)


def declared_arities():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b(?:cgtp_status|const char \*)\s*(cgtp_[a-z_]+)\s*\(([^)]*)\)", text):
        args = [a for a in m.group(2).split(",") if a.strip() and a.strip() != "void"]
        out[m.group(1)] = len(args)
    return out


def test_binding_declares_every_argument():
    """Every export taking arguments has ctypes argtypes of the header's arity (so 64-bit sizes
    are passed as 64-bit values, never as C int)."""
    lib = cg.lib()
    ar = declared_arities()
    assert set(ar) == set(declared_functions())
    for name, n in ar.items():
        if n:
            assert getattr(lib, name).argtypes is not None and len(getattr(lib, name).argtypes) == n, name


def test_library_exports_every_declared_symbol():
    lib = cg.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


# ---------------------------------------------------------------------------- bookkeeping (G12)

BOOK = {
    # workload: (paths, nnz, d_x, d_sh, d_out, weights per edge/row or shared)
    "c1": (9, 59, 16, 9, 116, 36),
    "c2": (15, 137, 288, 9, 1632, 480),
    "c3": (34, 611, 2048, 16, 19968, 4352),
    "c4": (154, 12868, 1024, 64, 1024, 39424),
    "c5": (15, 137, 576, 9, 3264, 960),
}


@pytest.mark.parametrize("name", sorted(BOOK))
def test_bookkeeping_planner_and_oracle(name):
    spec = synth.WORKLOADS[name]
    plan = cg.plan_for(spec, "f32")
    got = (plan.num_paths, plan.nnz_total, plan.d_x, plan.d_sh, plan.d_out, plan.weight_numel)
    assert got == BOOK[name]
    out = spec.out_irreps if getattr(spec, "mode", "uvu") == "uvw" else \
        oirreps.per_path_out_irreps(spec.in_irreps, spec.lmax_sh, getattr(spec, "lmax_out", spec.lmax_sh))
    prob = oirreps.build_problem(spec.in_irreps, oirreps.sh_irreps(spec.lmax_sh), out,
                                 getattr(spec, "mode", "uvu"))
    assert (len(prob.paths), prob.d_in, prob.d_sh, prob.d_out, prob.weight_numel) == \
        (BOOK[name][0],) + BOOK[name][2:]
    for p, op in enumerate(prob.paths):
        info = plan.path(p)
        assert (info["i1"], info["i2"], info["slot"], info["l1"], info["l2"], info["l3"], info["p3"],
                info["w_off"]) == (op.i1, op.i2, op.slot, op.l1, op.l2, op.l3, op.p3, op.w_off)


def test_planner_cg_matches_oracle_cg(tmp_path, monkeypatch):
    """G11: the planner's recursion and the oracle's exact Racah sum give the same blocks."""
    monkeypatch.setenv("CGTP_CACHE_DIR", str(tmp_path))  # keep this large module out of the shared cache
    ins = "+".join(f"1x{l}{p}" for l in range(8) for p in "eo")
    out = "+".join(f"1x{l}{p}" for l in range(8) for p in "eo")
    plan = cg.plan_create(ins, oirreps.sh_irreps(7), out, "uvw", "f64")
    seen = set()
    for p in range(plan.num_paths):
        info = plan.path(p)
        key = (info["l1"], info["l2"], info["l3"])
        ijk, vals = plan.coefficients(p)
        want = ocg.nonzeros(*key)
        assert [tuple(r) for r in ijk] == [(i, j, k) for i, j, k, _ in want], key
        assert np.max(np.abs(vals - np.array([c for *_, c in want]))) <= 1e-15, key
        seen.add(key)
    assert len(seen) > 100


def test_generated_source_has_literal_nonzeros_and_no_atomics():
    """The nonzeros are compile-time literals (rounded to the kernel dtype) and nothing is atomic."""
    for dtype, rnd in (("f32", lambda v: float(np.float32(v))), ("f64", float)):
        plan = cg.plan_for(synth.WORKLOADS["c2"], dtype)
        src = plan.source
        assert "atomic" not in src.lower()
        lits = {float.fromhex(m) for m in re.findall(r"(-?0x[0-9a-f]+(?:\.[0-9a-f]*)?p[-+]?\d+)", src)}
        for p in range(plan.num_paths):
            _, vals = plan.coefficients(p)
            for v in vals:
                assert rnd(v) in lits, (dtype, p, v)


def test_row_split_rule():
    """Waves per receiver row: doubled while the launch has under four waves per wave slot
    (1024 SIMDs x the occupancy target) and each part keeps >= 8 edge groups of the mean row;
    plans with several path groups or channel tiles never split."""
    c2 = cg.plan_for(synth.WORKLOADS["c2"], "f32")   # 32 channels: 2 edges per wave step, 4 waves/SIMD
    assert c2.row_split(5000, 200_000) == 2
    assert c2.row_split(601, 601 * 20) == 1 and c2.row_split(601, 601 * 40) == 2
    assert c2.row_split(601, 601 * 160) == 4
    assert c2.row_split(20_000, 800_000) == 1        # 20,000 waves already >= 4 x 4096 slots
    assert c2.row_split(10_000, 400_000) == 2
    assert c2.row_split(1, 0) == 1 and c2.row_split(0, 0) == 1
    assert c2.row_split(5000, 200_000, double_backward=True) == 2   # 2 waves/SIMD: 8192 slots
    assert c2.row_split(9000, 360_000, double_backward=True) == 1
    c5 = cg.plan_for(synth.WORKLOADS["c5"], "f32")   # 64 channels: one edge per wave step
    assert c5.row_split(200_000, 10_000_000) == 1
    assert c5.row_split(2000, 100_000) == 4
    c3 = cg.plan_for(synth.WORKLOADS["c3"], "f32")   # three path groups x two channel tiles
    assert c3.row_split(100, 100_000) == 1
    src = c2.source
    assert "cgtp_conv_fwd_split2(" in src and "cgtp_conv_dbwd_recv_split4(" in src
    assert "cgtp_conv_fwd_split2(" not in c3.source
    with pytest.raises(cg.CgtpError, match="pass must be"):
        v = ctypes.c_int32()
        cg._check(cg.lib().cgtp_conv_row_split(c2.handle, 10, 10, 2, ctypes.byref(v)))


# ---------------------------------------------------------------------------- error paths

def test_plan_errors():
    L = cg.lib()
    h = ctypes.c_void_p()
    bad = [
        ("32x0e+", "1x0e", "32x0e", 0, 0, cg.STATUS_CODES["CGTP_ERR_IRREPS"]),
        ("32x0q", "1x0e", "32x0e", 0, 0, cg.STATUS_CODES["CGTP_ERR_IRREPS"]),
        ("32x8e", "1x0e", "32x8e", 0, 0, cg.STATUS_CODES["CGTP_ERR_IRREPS"]),
        ("32x0e", "2x0e", "32x0e", 0, 0, cg.STATUS_CODES["CGTP_ERR_IRREPS"]),     # SH mul must be 1
        ("32x0e", "1x0e", "16x0e", 0, 0, cg.STATUS_CODES["CGTP_ERR_IRREPS"]),     # uvu mul mismatch
        ("32x0e", "1x0e", "32x1o", 0, 0, cg.STATUS_CODES["CGTP_ERR_IRREPS"]),     # unreachable output
        ("8x1o", "1x1o", "8x0e+8x0e", 0, 0, cg.STATUS_CODES["CGTP_ERR_IRREPS"]),  # 2 slots, 1 path
        ("32x0e", "1x0e", "32x0e", 7, 0, cg.STATUS_CODES["CGTP_ERR_INVALID_ARG"]),
        ("32x0e", "1x0e", "32x0e", 0, 9, cg.STATUS_CODES["CGTP_ERR_INVALID_ARG"]),
    ]
    for a, b, c, mode, dt, want in bad:
        st = L.cgtp_plan_create(a.encode(), b.encode(), c.encode(), mode, dt, ctypes.byref(h))
        assert st == want, (a, b, c, mode, dt, st, cg.last_error())
        assert cg.last_error()
    assert L.cgtp_plan_create(None, b"1x0e", b"1x0e", 0, 0, ctypes.byref(h)) == \
        cg.STATUS_CODES["CGTP_ERR_INVALID_ARG"]


def test_call_errors_before_any_gpu_work():
    L = cg.lib()
    plan = cg.plan_for(synth.WORKLOADS["c2"], "f32")
    uvw = cg.plan_for(synth.WORKLOADS["c4"], "f32")
    inval = cg.STATUS_CODES["CGTP_ERR_INVALID_ARG"]
    unsup = cg.STATUS_CODES["CGTP_ERR_UNSUPPORTED"]
    fake = ctypes.c_void_p(1 << 20)            # aligned, never dereferenced: every call below fails first
    odd = ctypes.c_void_p((1 << 20) + 2)       # misaligned for float
    null = ctypes.c_void_p(0)
    s = ctypes.c_void_p(0)
    assert L.cgtp_conv_forward(None, 4, 4, fake, fake, fake, fake, fake, fake, s) == inval
    assert L.cgtp_conv_forward(plan.handle, -1, 4, fake, fake, fake, fake, fake, fake, s) == inval
    assert L.cgtp_conv_forward(plan.handle, 4, 1 << 31, fake, fake, fake, fake, fake, fake, s) == inval
    assert L.cgtp_conv_forward(plan.handle, 4, 4, null, fake, fake, fake, fake, fake, s) == inval
    assert L.cgtp_conv_forward(plan.handle, 4, 4, fake, fake, odd, fake, fake, fake, s) == inval
    # output overlapping an input
    assert L.cgtp_conv_forward(plan.handle, 4, 4, fake, ctypes.c_void_p(1 << 22), ctypes.c_void_p(1 << 24),
                               fake, fake, ctypes.c_void_p((1 << 24) + 64), s) == inval
    # uvw convolution: shared weights must be given, outputs must not overlap them
    assert L.cgtp_conv_forward(uvw.handle, 4, 4, fake, fake, fake, fake, null, fake, s) == inval
    assert L.cgtp_conv_forward(uvw.handle, 4, 0, fake, null, null, null, null, fake, s) == inval
    assert L.cgtp_conv_forward(uvw.handle, 4, 4, fake, fake, ctypes.c_void_p(1 << 22), ctypes.c_void_p(1 << 24),
                               ctypes.c_void_p(1 << 26), ctypes.c_void_p((1 << 26) + 64), s) == inval
    # the batched uvw forward takes any output multiplicity (16-wide output tiles); its backward
    # stops at 16 (below)
    wide = ctypes.c_void_p()
    assert L.cgtp_plan_create(b"16x0e", b"1x0e", b"32x0e", 1, 0, ctypes.byref(wide)) == 0
    # batched backward: uvu needs shared=0; the uvw backward is not built
    z = ctypes.c_size_t(0)
    assert L.cgtp_tp_backward(plan.handle, 4, fake, fake, fake, 1, fake, fake, fake, fake, null, z, s) == inval
    assert L.cgtp_tp_backward(uvw.handle, 4, fake, fake, fake, 0, fake, fake, fake, fake, null, z, s) == inval
    assert L.cgtp_tp_backward(plan.handle, 4, fake, fake, fake, 0, null, fake, null, null, null, z, s) == inval
    assert L.cgtp_tp_backward(plan.handle, 0, null, null, null, 0, null, null, null, null, null, z, s) == 0
    # uvw: the shared-weight gradient needs the workspace, sized by the query
    nb = ctypes.c_size_t()
    assert L.cgtp_tp_backward_workspace_size(uvw.handle, 50_000, ctypes.byref(nb)) == 0
    nblocks = (50_000 + 15) // 16
    bpc = -(-nblocks // 256)
    assert nb.value == -(-nblocks // bpc) * uvw.weight_numel * 4   # at most 256 chunks of 16-row blocks
    assert L.cgtp_tp_backward_workspace_size(plan.handle, 50_000, ctypes.byref(nb)) == 0 and nb.value == 0
    assert L.cgtp_tp_backward(uvw.handle, 4, fake, fake, fake, 1, ctypes.c_void_p(1 << 26), null, null,
                              ctypes.c_void_p(1 << 28), null, z, s) == inval
    # wider plans run the convolution backward on the identity graph: the workspace holds its part
    # (16x0e -> 32x0e, l = 0: G 4 x 16 floats padded to 256 bytes, one 512-weight dW partial) and
    # the index array 0..B, and is needed for every gradient
    assert L.cgtp_tp_backward_workspace_size(wide, 4, ctypes.byref(nb)) == 0 and nb.value == 256 + 2048 + 20
    assert L.cgtp_tp_backward(wide, 4, fake, fake, fake, 1, fake, fake, fake, fake, null, z, s) == inval
    assert L.cgtp_tp_backward(wide, 4, fake, fake, fake, 1, fake, fake, null, null, ctypes.c_void_p(1 << 28),
                              ctypes.c_size_t(256 + 2048 + 19), s) == inval
    assert L.cgtp_plan_destroy(wide) == 0
    assert L.cgtp_tp_forward(plan.handle, 4, fake, fake, fake, 1, fake, s) == inval   # uvu needs shared=0
    assert L.cgtp_tp_forward(uvw.handle, 4, fake, fake, fake, 0, fake, s) == inval    # uvw needs shared=1
    assert L.cgtp_spherical_harmonics(8, 0, 4, fake, fake, s) == inval
    assert L.cgtp_spherical_harmonics(2, 3, 4, fake, fake, s) == inval
    assert L.cgtp_graph_transpose(4, 4, null, fake, fake, fake, fake, s) == inval
    # backward: plan, N, E, row_ptr, col, t_row_ptr, t_edge, t_dst, x, y, w, g, gx, gy, gw, stream
    assert L.cgtp_conv_backward(plan.handle, 4, 4, fake, fake, null, fake, fake, fake, fake, fake, fake,
                                fake, fake, fake, s) == inval
    assert L.cgtp_conv_backward(plan.handle, 4, 4, fake, fake, fake, fake, fake, null, fake, fake, fake,
                                fake, fake, fake, s) == inval
    assert L.cgtp_conv_backward(uvw.handle, 4, 4, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                fake, fake, fake, s) == unsup
    # uvw convolution backward: the workspace is checked (size, alignment, overlap) before any GPU call
    cuvw = cg.plan_for(synth.EXTRA_WORKLOADS["c2uvw"], "f32")
    wsz = ctypes.c_size_t()
    assert L.cgtp_conv_backward_workspace_size(cuvw.handle, 4, 4, ctypes.byref(wsz)) == 0 and wsz.value > 0
    big = ctypes.c_void_p(1 << 30)

    def ws_call(workspace, nbytes, grad_w=ctypes.c_void_p(1 << 28), order=null):
        # plan, N, E, row_ptr, col, order, t_row_ptr, t_edge, t_dst, x, y, w, g, gx, gy, gw, ws, bytes, stream
        st = L.cgtp_conv_backward_ws(cuvw.handle, 4, 4, fake, fake, order, fake, fake, fake, fake, fake, fake,
                                     fake, null, null, grad_w, workspace, ctypes.c_size_t(nbytes), s)
        return st, cg.last_error()
    assert ws_call(big, wsz.value - 1) == (inval, "workspace too small (see cgtp_conv_backward_workspace_size)")
    assert ws_call(null, wsz.value) == (inval, "workspace is NULL")
    assert ws_call(ctypes.c_void_p((1 << 30) + 64), wsz.value) == (inval, "workspace is not aligned to 256 bytes")
    assert ws_call(big, wsz.value, grad_w=ctypes.c_void_p((1 << 30) + 256)) == (inval, "grad_w overlaps workspace")
    assert ws_call(big, wsz.value, order=ctypes.c_void_p((1 << 20) + 2)) == (inval, "order is not aligned to 4 bytes")
    assert L.cgtp_conv_backward_ws(cuvw.handle, 4, 4, fake, fake, null, fake, fake, fake, fake, fake, fake, fake,
                                   null, null, null, null, z, s) == 0            # nothing requested
    # zero-sized work is a no-op that succeeds without touching memory
    assert L.cgtp_tp_forward(plan.handle, 0, null, null, null, 0, null, s) == 0
    assert L.cgtp_spherical_harmonics(2, 0, 0, null, null, s) == 0
    assert L.cgtp_conv_forward(plan.handle, 0, 0, null, null, null, null, null, null, s) == 0


def test_conv_uvw_backward_workspace_and_modules():
    """Workspace of the uvw convolution backward: G (N x sum_p mul_in (2 l3 + 1), padded to 256
    bytes) plus one dW partial per 16-receiver tile; its two modules build on the host."""
    plan = cg.plan_for(synth.EXTRA_WORKLOADS["c2uvw"], "f32")
    dg = sum(plan.path(p)["mul_in"] * (2 * plan.path(p)["l3"] + 1) for p in range(plan.num_paths))
    for n in (1, 17, 5000):
        want = -(-n * dg * 4 // 256) * 256 + -(-n // 16) * plan.weight_numel * 4
        assert cg.conv_backward_workspace_size(plan, n, 40 * n) == want
    assert cg.conv_backward_workspace_size(plan, 0, 0) == 0
    assert cg.conv_backward_workspace_size(cg.plan_for(synth.WORKLOADS["c2"], "f32"), 5000, 200_000) == 0
    with pytest.raises(cg.CgtpError, match="CGTP_ERR_UNSUPPORTED"):
        cg.plan_for(synth.WORKLOADS["c2"], "f32").conv_uvw_backward_source(0)
    src_gw = plan.conv_uvw_backward_source(0)
    src_xy = plan.conv_uvw_backward_source(1)
    assert "cgtp_conv_uvw_bwd_g" in src_gw and "cgtp_conv_uvw_bwd_w" in src_gw and "cgtp_reduce_chunks" in src_gw
    assert "cgtp_conv_uvw_bwd_xy" in src_xy
    # the sender pass has unit weights: it reads no weight and writes no weight gradient
    assert "&w[" not in src_xy and "dw[" not in src_xy
    for src in (src_gw, src_xy):
        assert "atomic" not in src.lower()
    # the radial projection in uvw mode: the forward kernel of radial channel rr scales the SH
    # values by rho as it loads them; its backward workspace is G, R x tiles dTheta partials and
    # two SH-sized rows per edge, each part 256-byte aligned
    assert "cgtp_conv_uvw_rad" in src_gw and "rho[(size_t)" in src_gw
    pad = lambda b: (b + 255) // 256 * 256
    N, E, R = 5000, 200_000, 8
    tiles, es = (N + 15) // 16, 4
    gb = cg.conv_backward_workspace_size(plan, N, E) - tiles * plan.weight_numel * es
    assert cg.conv_backward_radial_workspace_size(plan, N, E, R) == (
        gb + pad(R * tiles * plan.weight_numel * es) + 2 * pad(E * plan.d_sh * es))
    assert cg.conv_backward_radial_workspace_size(plan, 0, 0, R) == 0


def test_uvw_batched_backward_module_has_no_atomics_and_no_lane_shuffles():
    """The batched uvw backward (dx/dY and dW kernels) builds on the host; like every generated
    kernel it issues no atomic, and its lane sums over xor 16 / 32 are permlane exchanges."""
    plan = cg.Plan("4x0e+3x1o+2x2e", cg.sh_irreps(2), "5x0e+3x1o+2x2e+1x1e", "uvw", "f32")
    src = plan.uvw_backward_source()
    assert "cgtp_tp_uvw_bwd_xy" in src and "cgtp_tp_uvw_bwd_w" in src
    # (its wave-scope fences name memory orders, __ATOMIC_RELEASE / _ACQUIRE, and order nothing
    # but the compiler's placement of the LDS transpose)
    assert not re.search(r"__hip_atomic|atomic(add|sub|cas|exch|max|min|inc|dec|and|or|xor)|atomic_fetch", src, re.I)
    assert "xsum16(" in src and "xsum32(" in src and "__shfl" not in src


def test_compiled_code_does_not_depend_on_what_the_process_loaded_first(tmp_path):
    """The generated module is compiled by the ROCm installation's hipRTC in a link namespace of
    its own, so a process that imported torch first (which brings its own hipRTC and compiler
    library under the same soname) writes the same code object under the same cache key."""
    import subprocess
    import sys
    prog = ("import sys\n"
            "if sys.argv[1] == 'torch': import torch\n"
            "from clebsch_gordan_tensor_cgtp_amd import binding as cg\n"
            "cg.Plan('4x0e+4x1o', cg.sh_irreps(2), cg.per_path_out_irreps('4x0e+4x1o', 2, 2), 'uvu', 'f32')\n")
    dirs = []
    for first in ("torch", "plain"):
        d = tmp_path / first
        d.mkdir()
        env = dict(os.environ, CGTP_CACHE_DIR=str(d), PYTHONPATH=ROOT)
        subprocess.run([sys.executable, "-c", prog, first], check=True, env=env, cwd=ROOT, timeout=600)
        dirs.append(d)
    a = sorted(p.name for p in dirs[0].iterdir() if p.suffix == ".hsaco")
    b = sorted(p.name for p in dirs[1].iterdir() if p.suffix == ".hsaco")
    assert a == b and len(a) == 1
    assert (dirs[0] / a[0]).read_bytes() == (dirs[1] / b[0]).read_bytes()


@pytest.mark.parametrize("irreps,dtype", [("128x7o", "f64"), ("256x7o", "f32")])
def test_uvw_convolution_rejects_paths_beyond_workgroup_lds(irreps, dtype, tmp_path, monkeypatch):
    """A uvw path whose T staging for one 16-receiver tile (16 x mul_in x (2 l3 + 1) elements)
    exceeds the 160 KB of LDS of one workgroup cannot be split further: the plan still builds (the
    batched forward tiles its output channels), while the convolution entry points return
    CGTP_ERR_UNSUPPORTED with the reason before any GPU call."""
    monkeypatch.setenv("CGTP_CACHE_DIR", str(tmp_path))
    plan = cg.plan_create(irreps, "1x0e", irreps, "uvw", dtype)
    L = cg.lib()
    fake = ctypes.c_void_p(1 << 20)
    null = ctypes.c_void_p(0)
    s = ctypes.c_void_p(0)
    unsup = cg.STATUS_CODES["CGTP_ERR_UNSUPPORTED"]
    assert L.cgtp_conv_forward(plan.handle, 4, 4, fake, fake, fake, fake, fake, fake, s) == unsup
    assert "LDS" in cg.last_error()
    assert L.cgtp_conv_backward_ws(plan.handle, 4, 4, fake, fake, null, fake, fake, fake, fake, fake, fake, fake,
                                   fake, fake, fake, fake, ctypes.c_size_t(1 << 30), s) == unsup
    assert L.cgtp_tp_backward(plan.handle, 4, fake, fake, fake, 1, fake, fake, fake, fake, fake,
                              ctypes.c_size_t(1 << 30), s) == unsup
    with pytest.raises(cg.CgtpError, match="CGTP_ERR_UNSUPPORTED"):
        plan.conv_uvw_backward_source(0)
    # the uvw radial projection runs on the same convolution kernels: refused the same way
    assert L.cgtp_conv_forward_radial(plan.handle, 4, 4, fake, fake, null, fake, fake, 2, fake, fake, fake, s) == unsup
    assert "LDS" in cg.last_error()
    assert L.cgtp_conv_backward_radial(plan.handle, 4, 4, fake, fake, fake, fake, fake, fake, fake, 2, fake, fake,
                                       fake, fake, fake, fake, fake, fake, ctypes.c_size_t(1 << 30), s) == unsup
    with pytest.raises(cg.CgtpError, match="CGTP_ERR_UNSUPPORTED"):
        plan.radial_source(2)
    plan.close()


def test_compile_after_the_environment_moved(tmp_path):
    """hipRTC runs in a link namespace of its own, whose C library keeps its own pointer to the
    environment.  A process that changes its environment after the first plan (here: enough new
    variables to move the environment array) must still compile the next module."""
    import subprocess
    import sys
    # the environment is moved once before the first plan (so the namespace copies a heap array)
    # and many times after it (freeing that array); the freed memory is then overwritten
    prog = ("import os, sys\n"
            "from clebsch_gordan_tensor_cgtp_amd import binding as cg\n"
            "for i in range(300): os.environ[f'CGTP_TEST_PRE_{i}'] = 'x'\n"
            "cg.Plan('2x0e', '1x0e', '2x0e', 'uvu', 'f32')\n"
            "for i in range(3000): os.environ[f'CGTP_TEST_PAD_{i}'] = 'x' * 64\n"
            "junk = [bytearray(b'\\xff' * n) for n in range(1024, 65536, 512) for _ in range(4)]\n"
            "os.environ['CGTP_CACHE_DIR'] = sys.argv[1]\n"
            "p = cg.Plan('3x1o', '1x0e+1x1o', '3x1o+3x0e+3x1e+3x2e', 'uvu', 'f32')\n"
            "print(p.num_paths)\n")
    env = dict(os.environ, CGTP_CACHE_DIR=str(tmp_path / "first"), PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", prog, str(tmp_path / "second")], env=env, cwd=ROOT, timeout=600,
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip() == "4"
    assert any(p.suffix == ".hsaco" for p in (tmp_path / "second").iterdir())


def test_radial_theta_copies_fit_per_path_group(tmp_path, monkeypatch):
    """The radial kernels copy to LDS only the Theta columns one workgroup reads: a channel tile
    of one path group in the forward, one path group in the backward.  The MACE-like plan (4,352
    weights per edge) at R = 8 needs 139 KB for the whole of Theta but a few tens of KB per
    unit, so both kernels are generated; R = 64 overflows even one unit and is refused before
    any code is generated or any GPU call is made."""
    monkeypatch.setenv("CGTP_CACHE_DIR", str(tmp_path))
    plan = cg.plan_for(synth.WORKLOADS["c3"], "f32")
    src = plan.radial_source(8)
    assert "cgtp_conv_fwd_radial(" in src and "cgtp_conv_bwd_radial(" in src
    sizes = [int(n) for n in re.findall(r"__shared__ T thl\[(\d+)\]", src)]
    assert len(sizes) == 2 and max(sizes) < 8 * plan.weight_numel
    # every staged column is a Theta element of a path of the group (row r, column w_p + c)
    assert "theta[(size_t)r * WROW + " in src
    with pytest.raises(cg.CgtpError, match="CGTP_ERR_UNSUPPORTED"):
        plan.radial_source(64)
    assert "LDS" in cg.last_error()
    fake = ctypes.c_void_p(1 << 20)
    s = ctypes.c_void_p(0)
    unsup = cg.STATUS_CODES["CGTP_ERR_UNSUPPORTED"]
    assert cg.lib().cgtp_conv_forward_radial(plan.handle, 4, 4, fake, fake, None, fake, fake, 64, fake, fake,
                                             ctypes.c_void_p(1 << 24), s) == unsup
