"""Pins of the oracle's operations (oracle/ref.py, oracle/cpu_loops.c).

G8  equivariance under proper and improper rotations (forward and backward)
G9  brute force: a dense einsum with the fully assembled coupling tensor
G10 trilinear identity and finite differences for the backward
plus: the explicit C loops agree with the numpy definitions, and planted
mistakes in the oracle (a transposed index, a dropped term, a wrong sign)
are caught by these pins.
"""
import numpy as np
import pytest

from oracle import irreps, loops, ref, wigner
from oracle import sh as osh
from oracle.cg import real_cg_block

IN_MIXED = "2x0e+3x1o+2x2e+1x3o"


def problem(in_irreps=IN_MIXED, lmax_sh=3, lmax_out=3, mode="uvu", out=None):
    out = out or irreps.per_path_out_irreps(in_irreps, lmax_sh, lmax_out)
    return irreps.build_problem(in_irreps, irreps.sh_irreps(lmax_sh), out, mode)


def small_graph(rng, n_nodes, n_edges):
    recv = rng.integers(0, n_nodes, n_edges)
    send = rng.integers(0, n_nodes, n_edges)
    order = np.argsort(recv, kind="stable")
    row_ptr = np.concatenate([[0], np.cumsum(np.bincount(recv, minlength=n_nodes))])
    return row_ptr, send[order]


def conv_inputs(prob, rng, n_nodes=7, n_edges=30):
    row_ptr, col = small_graph(rng, n_nodes, n_edges)
    x = rng.standard_normal((n_nodes, prob.d_in))
    vec = rng.standard_normal((n_edges, 3))
    w = rng.standard_normal((n_edges, prob.weight_numel))
    g = rng.standard_normal((n_nodes, prob.d_out))
    return row_ptr, col, x, vec, w, g


def dense_tensor(prob):
    """The assembled coupling tensor P[x, y, w, out] (uvu) with P = C on every nonzero."""
    oa, ob, oo = irreps.offsets(prob.ins), irreps.offsets(prob.sh), irreps.offsets(prob.out)
    t = np.zeros((prob.d_in, prob.d_sh, prob.weight_numel, prob.d_out))
    for p in prob.paths:
        c = real_cg_block(p.l1, p.l2, p.l3)
        n1, n2, n3 = c.shape
        mi, mo = prob.ins[p.i1].mul, prob.out[p.slot].mul
        for u in range(mi):
            xs = slice(oa[p.i1] + u * n1, oa[p.i1] + (u + 1) * n1)
            ys = slice(ob[p.i2], ob[p.i2] + n2)
            if prob.mode == "uvu":
                os_ = slice(oo[p.slot] + u * n3, oo[p.slot] + (u + 1) * n3)
                t[xs, ys, p.w_off + u, os_] += c
            else:
                for w_ in range(mo):
                    os_ = slice(oo[p.slot] + w_ * n3, oo[p.slot] + (w_ + 1) * n3)
                    t[xs, ys, p.w_off + u * mo + w_, os_] += c
    return t


# ------------------------------------------------------------------------------ G9 brute force

@pytest.mark.parametrize("in_irreps,lmax_sh,lmax_out", [
    ("4x0e+4x1o", 2, 2), ("3x0e+3x1o+3x2e", 2, 2), (IN_MIXED, 3, 3), ("2x1o+1x2e", 1, 3)])
def test_uvu_forward_and_backward_brute_force(in_irreps, lmax_sh, lmax_out):
    prob = problem(in_irreps, lmax_sh, lmax_out)
    rng = np.random.default_rng(0)
    row_ptr, col, x, vec, w, g = conv_inputs(prob, rng)
    y = rng.standard_normal((len(col), prob.d_sh))  # any y: the operation is bilinear in x, y
    t = dense_tensor(prob)
    dst = ref.receivers_of(row_ptr)
    msg = np.einsum("abvo,ea,eb,ev->eo", t, x[col], y, w)
    want = np.zeros((len(row_ptr) - 1, prob.d_out))
    np.add.at(want, dst, msg)
    assert np.allclose(ref.conv_forward(prob, row_ptr, col, x, y, w), want, atol=1e-12)
    dx, dy, dw = ref.conv_backward(prob, row_ptr, col, x, y, w, g)
    gd = g[dst]
    want_dxs = np.einsum("abvo,eb,ev,eo->ea", t, y, w, gd)
    want_dx = np.zeros_like(x)
    np.add.at(want_dx, col, want_dxs)
    assert np.allclose(dx, want_dx, atol=1e-12)
    assert np.allclose(dy, np.einsum("abvo,ea,ev,eo->eb", t, x[col], w, gd), atol=1e-12)
    assert np.allclose(dw, np.einsum("abvo,ea,eb,eo->ev", t, x[col], y, gd), atol=1e-12)


def test_uvw_forward_brute_force():
    ins = "3x0e+2x1o+2x2e"
    prob = irreps.build_problem(ins, irreps.sh_irreps(2), "2x0e+3x1o+2x2e+1x1e+2x2o", "uvw")
    rng = np.random.default_rng(1)
    x = rng.standard_normal((11, prob.d_in))
    y = rng.standard_normal((11, prob.d_sh))
    w = rng.standard_normal(prob.weight_numel)
    t = dense_tensor(prob)
    want = np.einsum("abvo,ra,rb,v->ro", t, x, y, w)
    assert np.allclose(ref.tp_forward(prob, x, y, w), want, atol=1e-12)


def test_tp_uvu_is_conv_on_identity_graph():
    prob = problem("4x0e+4x1o", 2, 2)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((9, prob.d_in))
    y = rng.standard_normal((9, prob.d_sh))
    w = rng.standard_normal((9, prob.weight_numel))
    ident = np.arange(10)
    assert np.allclose(ref.tp_forward(prob, x, y, w),
                       ref.conv_forward(prob, ident, np.arange(9), x, y, w), atol=1e-14)


# ------------------------------------------------------------------------------ G8 equivariance

def _rotate_case(prob, improper, seed=4):
    rng = np.random.default_rng(seed)
    row_ptr, col, x, vec, w, g = conv_inputs(prob, rng)
    rot = wigner.random_rotation(rng)
    lin = -rot if improper else rot
    d_in = wigner.irreps_d(prob.ins, rot, improper)
    d_sh = wigner.irreps_d(prob.sh, rot, improper)
    d_out = wigner.irreps_d(prob.out, rot, improper)
    y = osh.real_sh_all(prob.sh[-1].l, vec)
    y_rot = osh.real_sh_all(prob.sh[-1].l, vec @ lin.T)
    assert np.allclose(y_rot, y @ d_sh.T, atol=1e-11)
    return row_ptr, col, x, y, w, g, d_in, d_sh, d_out, y_rot


@pytest.mark.parametrize("improper", [False, True])
def test_conv_equivariance(improper):
    prob = problem()
    row_ptr, col, x, y, w, g, d_in, d_sh, d_out, y_rot = _rotate_case(prob, improper)
    out = ref.conv_forward(prob, row_ptr, col, x, y, w)
    out_rot = ref.conv_forward(prob, row_ptr, col, x @ d_in.T, y_rot, w)
    assert np.abs(out_rot - out @ d_out.T).max() < 1e-10 * max(1, np.abs(out).max())
    dx, dy, dw = ref.conv_backward(prob, row_ptr, col, x, y, w, g)
    dx2, dy2, dw2 = ref.conv_backward(prob, row_ptr, col, x @ d_in.T, y_rot, w, g @ d_out.T)
    assert np.allclose(dx2, dx @ d_in.T, atol=1e-10)
    assert np.allclose(dy2, dy @ d_sh.T, atol=1e-10)
    assert np.allclose(dw2, dw, atol=1e-10)


@pytest.mark.parametrize("improper", [False, True])
def test_uvw_equivariance(improper):
    ins = "2x0e+2x1o+2x2e+1x3o"
    out_irreps = "3x0e+2x1o+2x2e+1x3o+2x1e+1x2o"
    prob = irreps.build_problem(ins, irreps.sh_irreps(3), out_irreps, "uvw")
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, prob.d_in))
    vec = rng.standard_normal((6, 3))
    w = rng.standard_normal(prob.weight_numel)
    rot = wigner.random_rotation(rng)
    lin = -rot if improper else rot
    d_in = wigner.irreps_d(prob.ins, rot, improper)
    d_out = wigner.irreps_d(prob.out, rot, improper)
    out = ref.tp_forward(prob, x, osh.real_sh_all(3, vec), w)
    out_rot = ref.tp_forward(prob, x @ d_in.T, osh.real_sh_all(3, vec @ lin.T), w)
    assert np.allclose(out_rot, out @ d_out.T, atol=1e-10)


# ------------------------------------------------------------------------------ G10 backward

def test_trilinear_identity():
    prob = problem()
    rng = np.random.default_rng(5)
    row_ptr, col, x, vec, w, g = conv_inputs(prob, rng, 9, 40)
    y = rng.standard_normal((len(col), prob.d_sh))
    out = ref.conv_forward(prob, row_ptr, col, x, y, w)
    dx, dy, dw = ref.conv_backward(prob, row_ptr, col, x, y, w, g)
    s = np.sum(g * out)
    for a, b in ((dx, x), (dy, y), (dw, w)):
        assert abs(np.sum(a * b) - s) <= 1e-12 * max(1.0, abs(s)) * 10


def test_finite_differences():
    prob = problem("2x0e+2x1o+1x2e", 2, 2)
    rng = np.random.default_rng(6)
    row_ptr, col, x, vec, w, g = conv_inputs(prob, rng, 5, 14)
    y = rng.standard_normal((len(col), prob.d_sh))
    dx, dy, dw = ref.conv_backward(prob, row_ptr, col, x, y, w, g)

    def loss(x_, y_, w_):
        return np.sum(g * ref.conv_forward(prob, row_ptr, col, x_, y_, w_))

    h = 1e-6
    for arr, grad, which in ((x, dx, 0), (y, dy, 1), (w, dw, 2)):
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p = [x, y, w]
            args_m = [x, y, w]
            args_p[which], args_m[which] = ap, am
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-6 * max(1.0, abs(grad[idx]))


# ------------------------------------------------------------------------------ C loops == numpy

@pytest.mark.parametrize("in_f32", [False, True])
def test_cpu_loops_match_numpy(in_f32):
    prob = problem()
    tab = loops.Tables(prob)
    rng = np.random.default_rng(8)
    row_ptr, col, x, vec, w, g = conv_inputs(prob, rng, 12, 70)
    y = rng.standard_normal((len(col), prob.d_sh))
    dt = np.float32 if in_f32 else np.float64
    x, y, w, g = (a.astype(dt) for a in (x, y, w, g))
    n = len(row_ptr) - 1
    out = ref.conv_forward(prob, row_ptr, col, x, y, w)
    dx, dy, dw = ref.conv_backward(prob, row_ptr, col, x, y, w, g)
    assert np.allclose(loops.uvu_forward(tab, row_ptr, col, x, y, w), out, atol=1e-12)
    rows = np.array([5, 0, 11, 3])
    assert np.allclose(loops.conv_forward_rows(tab, row_ptr, col, x, y, w, rows), out[rows], atol=1e-12)
    eidx, dy_s, dw_s = loops.conv_backward_edge_rows(tab, row_ptr, col, x, y, w, g, np.arange(n))
    assert np.array_equal(eidx, np.arange(len(col)))
    assert np.allclose(dy_s, dy, atol=1e-12) and np.allclose(dw_s, dw, atol=1e-12)
    senders = np.array([2, 7, 0, 11])
    assert np.allclose(loops.conv_backward_x_rows(tab, row_ptr, col, y, w, g, senders), dx[senders],
                       atol=1e-12)


def test_cpu_loops_uvw_match_numpy():
    ins = "3x0e+2x1o+2x2e"
    prob = irreps.build_problem(ins, irreps.sh_irreps(2), "2x0e+3x1o+2x2e+1x1e+2x2o", "uvw")
    rng = np.random.default_rng(10)
    x = rng.standard_normal((13, prob.d_in))
    y = rng.standard_normal((13, prob.d_sh))
    w = rng.standard_normal(prob.weight_numel)
    assert np.allclose(loops.uvw_forward(loops.Tables(prob), x, y, w), ref.tp_forward(prob, x, y, w),
                       atol=1e-12)


# ------------------------------------------------------------------------------ planted mistakes

def _mutated(kind):
    real = ref.nonzeros

    def nz(l1, l2, l3):
        z = list(real(l1, l2, l3))
        if (l1, l2, l3) != (1, 1, 2):
            return z
        if kind == "transpose":   # swap the roles of the input and output components
            return [(k % (2 * l1 + 1), j, i % (2 * l3 + 1), c) for i, j, k, c in z]
        if kind == "drop":
            return z[1:]
        if kind == "sign":
            return [(i, j, k, -c if n == 0 else c) for n, (i, j, k, c) in enumerate(z)]
        raise ValueError(kind)
    return nz


@pytest.mark.parametrize("kind", ["transpose", "drop", "sign"])
def test_planted_mistake_is_caught_by_equivariance(monkeypatch, kind):
    prob = problem("2x0e+2x1o", 2, 2)
    row_ptr, col, x, y, w, g, d_in, d_sh, d_out, y_rot = _rotate_case(prob, False, seed=12)
    monkeypatch.setattr(ref, "nonzeros", _mutated(kind))
    out = ref.conv_forward(prob, row_ptr, col, x, y, w)
    out_rot = ref.conv_forward(prob, row_ptr, col, x @ d_in.T, y_rot, w)
    assert np.abs(out_rot - out @ d_out.T).max() > 1e-3


# ------------------------------------------------------------------------------ double backward

def _dbl_inputs(prob, rng, n_nodes=6, n_edges=21):
    row_ptr, col, x, vec, w, g = conv_inputs(prob, rng, n_nodes, n_edges)
    y = rng.standard_normal((len(col), prob.d_sh))
    ggx = rng.standard_normal(x.shape)
    ggy = rng.standard_normal(y.shape)
    ggw = rng.standard_normal(w.shape)
    return row_ptr, col, x, y, w, g, ggx, ggy, ggw


@pytest.mark.parametrize("in_irreps,lmax_sh,lmax_out", [("3x0e+3x1o+3x2e", 2, 2), ("2x1o+1x2e", 1, 3)])
def test_double_backward_matches_autograd_of_dense_einsum(in_irreps, lmax_sh, lmax_out):
    """Brute force: torch autograd (CPU, float64) differentiates twice through the dense coupling."""
    import torch
    prob = problem(in_irreps, lmax_sh, lmax_out)
    rng = np.random.default_rng(11)
    row_ptr, col, x, y, w, g, ggx, ggy, ggw = _dbl_inputs(prob, rng)
    t = torch.from_numpy(dense_tensor(prob))
    dst = torch.from_numpy(ref.receivers_of(row_ptr))
    colt = torch.from_numpy(np.asarray(col, np.int64))
    X, Y, W, G = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, y, w, g))

    def forward(x_, y_, w_):
        msg = torch.einsum("abvo,ea,eb,ev->eo", t, x_[colt], y_, w_)
        return torch.zeros(len(row_ptr) - 1, prob.d_out, dtype=torch.float64).index_add(0, dst, msg)

    first = torch.autograd.grad((G * forward(X, Y, W)).sum(), (X, Y, W), create_graph=True)
    l2 = sum((torch.from_numpy(u) * v).sum() for u, v in zip((ggx, ggy, ggw), first))
    want = torch.autograd.grad(l2, (X, Y, W, G))
    got = ref.conv_double_backward(prob, row_ptr, col, x, y, w, g, ggx, ggy, ggw)
    for a, b in zip(got, want):
        assert np.allclose(a, b.numpy(), atol=1e-11, rtol=1e-11)


def test_double_backward_finite_differences():
    prob = problem("2x0e+2x1o+1x2e", 2, 2)
    rng = np.random.default_rng(12)
    row_ptr, col, x, y, w, g, ggx, ggy, ggw = _dbl_inputs(prob, rng, 5, 13)
    got = ref.conv_double_backward(prob, row_ptr, col, x, y, w, g, ggx, ggy, ggw)

    def l2(x_, y_, w_, g_):
        dx, dy, dw = ref.conv_backward(prob, row_ptr, col, x_, y_, w_, g_)
        return np.sum(ggx * dx) + np.sum(ggy * dy) + np.sum(ggw * dw)

    h = 1e-6
    base = [x, y, w, g]
    for which in range(4):
        for _ in range(5):
            arr = base[which]
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            args_p, args_m = list(base), list(base)
            args_p[which], args_m[which] = arr.copy(), arr.copy()
            args_p[which][idx] += h
            args_m[which][idx] -= h
            fd = (l2(*args_p) - l2(*args_m)) / (2 * h)
            assert abs(fd - got[which][idx]) < 1e-6 * max(1.0, abs(got[which][idx]))


def test_double_backward_euler_identities():
    """L2 = A + B + C is linear in each operand: <d/dx, x> = B + C, <d/dy, y> = A + C,
    <d/dW, W> = A + B, <d/dg, g> = A + B + C with A = <ggx, dx>, B = <ggy, dy>, C = <ggw, dW>."""
    prob = problem()
    rng = np.random.default_rng(13)
    row_ptr, col, x, y, w, g, ggx, ggy, ggw = _dbl_inputs(prob, rng, 8, 33)
    dx1, dy1, dw1 = ref.conv_backward(prob, row_ptr, col, x, y, w, g)
    A, B, C = np.sum(ggx * dx1), np.sum(ggy * dy1), np.sum(ggw * dw1)
    dx, dy, dw, dg = ref.conv_double_backward(prob, row_ptr, col, x, y, w, g, ggx, ggy, ggw)
    scale = max(1.0, abs(A) + abs(B) + abs(C))
    for got, want in ((np.sum(dx * x), B + C), (np.sum(dy * y), A + C), (np.sum(dw * w), A + B),
                      (np.sum(dg * g), A + B + C)):
        assert abs(got - want) <= 1e-11 * scale


@pytest.mark.parametrize("improper", [False, True])
def test_double_backward_equivariance(improper):
    prob = problem()
    row_ptr, col, x, y, w, g, d_in, d_sh, d_out, y_rot = _rotate_case(prob, improper)
    rng = np.random.default_rng(14)
    ggx = rng.standard_normal(x.shape)
    ggy = rng.standard_normal(y.shape)
    ggw = rng.standard_normal(w.shape)
    base = ref.conv_double_backward(prob, row_ptr, col, x, y, w, g, ggx, ggy, ggw)
    rot = ref.conv_double_backward(prob, row_ptr, col, x @ d_in.T, y_rot, w, g @ d_out.T, ggx @ d_in.T,
                                   ggy @ d_sh.T, ggw)
    for got, want in zip(rot, (base[0] @ d_in.T, base[1] @ d_sh.T, base[2], base[3] @ d_out.T)):
        assert np.allclose(got, want, atol=1e-10)


@pytest.mark.parametrize("in_f32", [False, True])
def test_cpu_loops_double_backward_match_numpy(in_f32):
    prob = problem()
    rng = np.random.default_rng(15)
    row_ptr, col, x, y, w, g, ggx, ggy, ggw = _dbl_inputs(prob, rng, 9, 40)
    if in_f32:
        x, y, w, g, ggx, ggy, ggw = (a.astype(np.float32) for a in (x, y, w, g, ggx, ggy, ggw))
    want = ref.conv_double_backward(prob, row_ptr, col, x, y, w, g, ggx, ggy, ggw)
    tab = loops.Tables(prob)
    rows = np.array([4, 0, 7, 2])
    senders = np.array([3, 8, 1])
    eidx, dx, dy, dw, dg = loops.conv_double_backward_rows(tab, row_ptr, col, x, y, w, g, ggx, ggy, ggw,
                                                           rows, senders)
    assert np.allclose(dg, want[3][rows], atol=1e-12)
    assert np.allclose(dy, want[1][eidx], atol=1e-12)
    assert np.allclose(dw, want[2][eidx], atol=1e-12)
    assert np.allclose(dx, want[0][senders], atol=1e-12)



# ------------------------------------------------------------------------------ uvw convolution

def _uvw_conv_problem():
    return irreps.build_problem("3x0e+2x1o+2x2e", irreps.sh_irreps(2), "2x0e+3x1o+2x2e+1x1e+2x2o", "uvw")


def test_uvw_conv_brute_force_and_identity_graph():
    prob = _uvw_conv_problem()
    rng = np.random.default_rng(16)
    row_ptr, col = small_graph(rng, 7, 31)
    x = rng.standard_normal((7, prob.d_in))
    y = rng.standard_normal((31, prob.d_sh))
    w = rng.standard_normal(prob.weight_numel)
    t = dense_tensor(prob)
    msg = np.einsum("abvo,ea,eb,v->eo", t, x[col], y, w)
    want = np.zeros((7, prob.d_out))
    np.add.at(want, ref.receivers_of(row_ptr), msg)
    assert np.allclose(ref.conv_forward(prob, row_ptr, col, x, y, w), want, atol=1e-12)
    ident = np.arange(32)
    assert np.allclose(ref.conv_forward(prob, ident, np.arange(31), x[col], y, w),
                       ref.tp_forward(prob, x[col], y, w), atol=1e-13)


def test_uvw_conv_is_mixing_of_unit_weight_uvu_messages():
    """Linearity: the uvw convolution equals W applied to the per-path sums of unit-weight messages."""
    prob = _uvw_conv_problem()
    rng = np.random.default_rng(17)
    row_ptr, col = small_graph(rng, 6, 25)
    x = rng.standard_normal((6, prob.d_in))
    y = rng.standard_normal((25, prob.d_sh))
    w = rng.standard_normal(prob.weight_numel)
    got = ref.conv_forward(prob, row_ptr, col, x, y, w)
    dst = ref.receivers_of(row_ptr)
    oa, ob, oo = irreps.offsets(prob.ins), irreps.offsets(prob.sh), irreps.offsets(prob.out)
    want = np.zeros_like(got)
    for p in prob.paths:
        c = real_cg_block(p.l1, p.l2, p.l3)
        mi, mo = prob.ins[p.i1].mul, prob.out[p.slot].mul
        n1, n2, n3 = c.shape
        xb = x[col][:, oa[p.i1]:oa[p.i1] + mi * n1].reshape(-1, mi, n1)
        yb = y[:, ob[p.i2]:ob[p.i2] + n2]
        t = np.zeros((6, mi, n3))
        np.add.at(t, dst, np.einsum("ijk,eui,ej->euk", c, xb, yb))
        wp = w[p.w_off:p.w_off + mi * mo].reshape(mi, mo)
        want[:, oo[p.slot]:oo[p.slot] + mo * n3] += np.einsum("nuk,uv->nvk", t, wp).reshape(6, -1)
    assert np.allclose(got, want, atol=1e-12)


@pytest.mark.parametrize("improper", [False, True])
def test_uvw_conv_equivariance(improper):
    prob = irreps.build_problem("2x0e+2x1o+2x2e+1x3o", irreps.sh_irreps(3), "3x0e+2x1o+2x2e+1x3o+2x1e+1x2o", "uvw")
    rng = np.random.default_rng(18)
    row_ptr, col = small_graph(rng, 6, 20)
    x = rng.standard_normal((6, prob.d_in))
    vec = rng.standard_normal((20, 3))
    w = rng.standard_normal(prob.weight_numel)
    rot = wigner.random_rotation(rng)
    lin = -rot if improper else rot
    d_in = wigner.irreps_d(prob.ins, rot, improper)
    d_out = wigner.irreps_d(prob.out, rot, improper)
    out = ref.conv_forward(prob, row_ptr, col, x, osh.real_sh_all(3, vec), w)
    out_rot = ref.conv_forward(prob, row_ptr, col, x @ d_in.T, osh.real_sh_all(3, vec @ lin.T), w)
    assert np.allclose(out_rot, out @ d_out.T, atol=1e-10)


@pytest.mark.parametrize("in_f32", [False, True])
def test_cpu_loops_uvw_conv_match_numpy(in_f32):
    prob = _uvw_conv_problem()
    rng = np.random.default_rng(19)
    row_ptr, col = small_graph(rng, 9, 44)
    x = rng.standard_normal((9, prob.d_in))
    y = rng.standard_normal((44, prob.d_sh))
    w = rng.standard_normal(prob.weight_numel)
    if in_f32:
        x, y, w = (a.astype(np.float32) for a in (x, y, w))
    want = ref.conv_forward(prob, row_ptr, col, x, y, w)
    rows = np.array([5, 0, 8, 3])
    got = loops.conv_forward_uvw_rows(loops.Tables(prob), row_ptr, col, x, y, w, rows)
    assert np.allclose(got, want[rows], atol=1e-12)



# ------------------------------------------------------------------------------ radial projection

def test_radial_conv_brute_force_and_linearity():
    """W_e = rho_e Theta: equals the dense einsum with that W, is linear in Theta, and a rho that is
    one-hot on radial channel r selects Theta's row r as every edge's weights."""
    prob = problem("3x0e+3x1o+3x2e", 2, 2)
    rng = np.random.default_rng(20)
    row_ptr, col, x, vec, w, g = conv_inputs(prob, rng, 7, 29)
    y = rng.standard_normal((29, prob.d_sh))
    rho = rng.standard_normal((29, 5))
    theta = rng.standard_normal((5, prob.weight_numel))
    got = ref.conv_forward_radial(prob, row_ptr, col, x, y, rho, theta)
    t = dense_tensor(prob)
    msg = np.einsum("abvo,ea,eb,er,rv->eo", t, x[col], y, rho, theta)
    want = np.zeros((7, prob.d_out))
    np.add.at(want, ref.receivers_of(row_ptr), msg)
    assert np.allclose(got, want, atol=1e-12)
    theta2 = rng.standard_normal(theta.shape)
    both = ref.conv_forward_radial(prob, row_ptr, col, x, y, rho, theta + 2.0 * theta2)
    assert np.allclose(both, got + 2.0 * ref.conv_forward_radial(prob, row_ptr, col, x, y, rho, theta2), atol=1e-11)
    onehot = np.zeros_like(rho)
    onehot[:, 3] = 1.0
    assert np.allclose(ref.conv_forward_radial(prob, row_ptr, col, x, y, onehot, theta),
                       ref.conv_forward(prob, row_ptr, col, x, y, np.tile(theta[3], (29, 1))), atol=1e-12)


def test_cpu_loops_radial_match_numpy():
    prob = problem()
    rng = np.random.default_rng(21)
    row_ptr, col, x, vec, w, g = conv_inputs(prob, rng, 9, 41)
    y = rng.standard_normal((41, prob.d_sh))
    rho = rng.standard_normal((41, 8))
    theta = rng.standard_normal((8, prob.weight_numel))
    rows = np.array([2, 8, 0, 5])
    want = ref.conv_forward_radial(prob, row_ptr, col, x, y, rho, theta)[rows]
    got = loops.conv_forward_radial_rows(loops.Tables(prob), row_ptr, col, x, y, rho, theta, rows)
    assert np.allclose(got, want, atol=1e-12)



def test_radial_conv_backward_matches_autograd_and_loops():
    """dx, dy, drho, dTheta of sum(g * conv(x, y, rho Theta)): torch autograd (CPU, float64) through
    the dense coupling with W = rho Theta written into the einsum, and the explicit loops."""
    import torch
    prob = problem("3x0e+2x1o+3x2e", 2, 2)
    rng = np.random.default_rng(26)
    row_ptr, col, x, vec, w, g = conv_inputs(prob, rng, 8, 33)
    y = rng.standard_normal((33, prob.d_sh))
    rho = rng.standard_normal((33, 5))
    theta = rng.standard_normal((5, prob.weight_numel))
    t = torch.from_numpy(dense_tensor(prob))
    dst = torch.from_numpy(ref.receivers_of(row_ptr))
    colt = torch.from_numpy(np.asarray(col, np.int64))
    X, Y, Rho, Th = (torch.tensor(a, requires_grad=True) for a in (x, y, rho, theta))
    msg = torch.einsum("abvo,ea,eb,er,rv->eo", t, X[colt], Y, Rho, Th)
    out = torch.zeros(8, prob.d_out, dtype=torch.float64).index_add(0, dst, msg)
    want = torch.autograd.grad((torch.from_numpy(g) * out).sum(), (X, Y, Rho, Th))
    got = ref.conv_backward_radial(prob, row_ptr, col, x, y, rho, theta, g)
    for a, b in zip(got, want):
        assert np.allclose(a, b.numpy(), atol=1e-10)
    rows, senders = np.array([6, 0, 3]), np.array([7, 2, 0, 5])
    eidx, dx, dy, drho, dtheta = loops.conv_backward_radial_rows(loops.Tables(prob), row_ptr, col, x, y, rho, theta,
                                                                 g, rows, senders)
    assert np.allclose(dx, got[0][senders], atol=1e-11)
    assert np.allclose(dy, got[1][eidx], atol=1e-11)
    assert np.allclose(drho, got[2][eidx], atol=1e-11)
    assert np.allclose(dtheta, got[3], atol=1e-10)


def test_radial_conv_backward_one_hot_and_adjoint():
    """A rho one-hot on channel r gives dTheta zero outside row r and equal there to the sum of the
    stored-weight gradients over all edges, and drho[e][r] = <dW_e, Theta[r]>; for any direction V,
    <dTheta, V> = <g, conv(x, y, rho V)> (the forward is linear in Theta)."""
    prob = problem("2x0e+3x1o+2x2e", 2, 2)
    rng = np.random.default_rng(27)
    row_ptr, col, x, vec, w, g = conv_inputs(prob, rng, 6, 25)
    y = rng.standard_normal((25, prob.d_sh))
    theta = rng.standard_normal((4, prob.weight_numel))
    onehot = np.zeros((25, 4))
    onehot[:, 2] = 1.0
    dx, dy, drho, dtheta = ref.conv_backward_radial(prob, row_ptr, col, x, y, onehot, theta, g)
    _, _, dw = ref.conv_backward(prob, row_ptr, col, x, y, np.tile(theta[2], (25, 1)), g)
    assert np.allclose(dtheta[[0, 1, 3]], 0.0) and np.allclose(dtheta[2], dw.sum(axis=0), atol=1e-11)
    assert np.allclose(drho, dw @ theta.T, atol=1e-11)
    rho = rng.standard_normal((25, 4))
    v = rng.standard_normal(theta.shape)
    _, _, _, dtheta = ref.conv_backward_radial(prob, row_ptr, col, x, y, rho, theta, g)
    lhs = float(np.sum(dtheta * v))
    rhs = float(np.sum(g * ref.conv_forward_radial(prob, row_ptr, col, x, y, rho, v)))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(rhs))


def _uvw_radial_case(seed, n_nodes, n_edges, R):
    prob = _uvw_conv_problem()
    rng = np.random.default_rng(seed)
    row_ptr, col = small_graph(rng, n_nodes, n_edges)
    x = rng.standard_normal((n_nodes, prob.d_in))
    y = rng.standard_normal((n_edges, prob.d_sh))
    rho = rng.standard_normal((n_edges, R))
    theta = rng.standard_normal((R, prob.weight_numel))
    g = rng.standard_normal((n_nodes, prob.d_out))
    return prob, rng, row_ptr, col, x, y, rho, theta, g


def test_radial_uvw_conv_brute_force_linearity_and_one_hot():
    """uvw with W_e = rho_e Theta (each edge its own W_p[u][w] blocks): the dense einsum with that W,
    linear in Theta, and a rho one-hot on channel r equals the shared-weight uvw convolution with
    Theta's row r."""
    prob, rng, row_ptr, col, x, y, rho, theta, g = _uvw_radial_case(28, 7, 31, 4)
    got = ref.conv_forward_radial(prob, row_ptr, col, x, y, rho, theta)
    msg = np.einsum("abvo,ea,eb,er,rv->eo", dense_tensor(prob), x[col], y, rho, theta)
    want = np.zeros((7, prob.d_out))
    np.add.at(want, ref.receivers_of(row_ptr), msg)
    assert np.allclose(got, want, atol=1e-12)
    theta2 = rng.standard_normal(theta.shape)
    both = ref.conv_forward_radial(prob, row_ptr, col, x, y, rho, theta - 3.0 * theta2)
    assert np.allclose(both, got - 3.0 * ref.conv_forward_radial(prob, row_ptr, col, x, y, rho, theta2), atol=1e-11)
    onehot = np.zeros_like(rho)
    onehot[:, 1] = 1.0
    assert np.allclose(ref.conv_forward_radial(prob, row_ptr, col, x, y, onehot, theta),
                       ref.conv_forward(prob, row_ptr, col, x, y, theta[1]), atol=1e-12)


def test_radial_uvw_conv_backward_matches_autograd_one_hot_and_adjoint():
    """dx, dy, drho, dTheta of sum(g * conv(x, y, rho Theta)) in uvw mode: torch autograd (CPU,
    float64) through the dense coupling; a rho one-hot on channel r gives the shared-weight uvw
    gradients (dTheta zero outside row r); <dTheta, V> = <g, conv(x, y, rho V)>."""
    import torch
    prob, rng, row_ptr, col, x, y, rho, theta, g = _uvw_radial_case(29, 8, 33, 5)
    t = torch.from_numpy(dense_tensor(prob))
    dst = torch.from_numpy(ref.receivers_of(row_ptr))
    colt = torch.from_numpy(np.asarray(col, np.int64))
    X, Y, Rho, Th = (torch.tensor(a, requires_grad=True) for a in (x, y, rho, theta))
    msg = torch.einsum("abvo,ea,eb,er,rv->eo", t, X[colt], Y, Rho, Th)
    out = torch.zeros(8, prob.d_out, dtype=torch.float64).index_add(0, dst, msg)
    want = torch.autograd.grad((torch.from_numpy(g) * out).sum(), (X, Y, Rho, Th))
    got = ref.conv_backward_radial(prob, row_ptr, col, x, y, rho, theta, g)
    for a, b in zip(got, want):
        assert np.allclose(a, b.numpy(), atol=1e-10)
    onehot = np.zeros_like(rho)
    onehot[:, 3] = 1.0
    dx, dy, drho, dtheta = ref.conv_backward_radial(prob, row_ptr, col, x, y, onehot, theta, g)
    sx, sy, sw = ref.conv_backward_uvw(prob, row_ptr, col, x, y, theta[3], g)
    assert np.allclose(dx, sx, atol=1e-11) and np.allclose(dy, sy, atol=1e-11)
    assert np.allclose(dtheta[[0, 1, 2, 4]], 0.0) and np.allclose(dtheta[3], sw, atol=1e-11)
    v = rng.standard_normal(theta.shape)
    lhs = float(np.sum(got[3] * v))
    rhs = float(np.sum(g * ref.conv_forward_radial(prob, row_ptr, col, x, y, rho, v)))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(rhs))


# ------------------------------------------------------------------------------ batched backward

def _uvw_tp_problem():
    return irreps.build_problem("3x0e+2x1o+2x2e", irreps.sh_irreps(2), "2x0e+3x1o+2x2e+1x1e+2x2o", "uvw")


def test_tp_backward_uvw_matches_autograd_of_dense_einsum():
    import torch
    prob = _uvw_tp_problem()
    rng = np.random.default_rng(22)
    x = rng.standard_normal((9, prob.d_in))
    y = rng.standard_normal((9, prob.d_sh))
    w = rng.standard_normal(prob.weight_numel)
    g = rng.standard_normal((9, prob.d_out))
    t = torch.from_numpy(dense_tensor(prob))
    X, Y, W = (torch.tensor(a, requires_grad=True) for a in (x, y, w))
    out = torch.einsum("abvo,ra,rb,v->ro", t, X, Y, W)
    want = torch.autograd.grad((torch.from_numpy(g) * out).sum(), (X, Y, W))
    got = ref.tp_backward(prob, x, y, w, g)
    for a, b in zip(got, want):
        assert np.allclose(a, b.numpy(), atol=1e-11)


def test_tp_backward_uvw_trilinear_and_finite_differences():
    prob = _uvw_tp_problem()
    rng = np.random.default_rng(23)
    x = rng.standard_normal((7, prob.d_in))
    y = rng.standard_normal((7, prob.d_sh))
    w = rng.standard_normal(prob.weight_numel)
    g = rng.standard_normal((7, prob.d_out))
    dx, dy, dw = ref.tp_backward(prob, x, y, w, g)
    s = np.sum(g * ref.tp_forward(prob, x, y, w))
    for a, b in ((dx, x), (dy, y), (dw, w)):
        assert abs(np.sum(a * b) - s) <= 1e-11 * max(1.0, abs(s))
    h = 1e-6
    base = [x, y, w]
    for which, grad in enumerate((dx, dy, dw)):
        for _ in range(4):
            arr = base[which]
            idx = tuple(rng.integers(0, n) for n in arr.shape)
            ap, am = list(base), list(base)
            ap[which], am[which] = arr.copy(), arr.copy()
            ap[which][idx] += h
            am[which][idx] -= h
            fd = (np.sum(g * ref.tp_forward(prob, *ap)) - np.sum(g * ref.tp_forward(prob, *am))) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-6 * max(1.0, abs(grad[idx]))



@pytest.mark.parametrize("in_f32", [False, True])
def test_cpu_loops_uvw_backward_match_numpy(in_f32):
    prob = irreps.build_problem("2x0e+3x1o+2x2e+1x3o", irreps.sh_irreps(3), "3x0e+2x1o+2x2e+1x3o+2x1e+1x2o", "uvw")
    rng = np.random.default_rng(24)
    x = rng.standard_normal((13, prob.d_in))
    y = rng.standard_normal((13, prob.d_sh))
    w = rng.standard_normal(prob.weight_numel)
    g = rng.standard_normal((13, prob.d_out))
    if in_f32:
        x, y, w, g = (a.astype(np.float32) for a in (x, y, w, g))
    want = ref.tp_backward(prob, x, y, w, g)
    rows = np.array([4, 0, 12, 7])
    dx, dy, dw = loops.uvw_backward(loops.Tables(prob), x, y, w, g, rows, np.arange(13))
    assert np.allclose(dx, want[0][rows], atol=1e-12)
    assert np.allclose(dy, want[1][rows], atol=1e-12)
    assert np.allclose(dw, want[2], atol=1e-11)



def test_uvw_conv_backward_matches_autograd_and_loops():
    import torch
    prob = _uvw_conv_problem()
    rng = np.random.default_rng(25)
    row_ptr, col = small_graph(rng, 7, 27)
    x = rng.standard_normal((7, prob.d_in))
    y = rng.standard_normal((27, prob.d_sh))
    w = rng.standard_normal(prob.weight_numel)
    g = rng.standard_normal((7, prob.d_out))
    t = torch.from_numpy(dense_tensor(prob))
    dst = torch.from_numpy(ref.receivers_of(row_ptr))
    colt = torch.from_numpy(np.asarray(col, np.int64))
    X, Y, W = (torch.tensor(a, requires_grad=True) for a in (x, y, w))
    msg = torch.einsum("abvo,ea,eb,v->eo", t, X[colt], Y, W)
    out = torch.zeros(7, prob.d_out, dtype=torch.float64).index_add(0, dst, msg)
    want = torch.autograd.grad((torch.from_numpy(g) * out).sum(), (X, Y, W))
    got = ref.conv_backward_uvw(prob, row_ptr, col, x, y, w, g)
    for a, b in zip(got, want):
        assert np.allclose(a, b.numpy(), atol=1e-11)
    edges, senders = np.array([3, 0, 26, 11]), np.array([6, 1, 4])
    dx, dy, dw = loops.conv_backward_uvw_rows(loops.Tables(prob), row_ptr, col, x, y, w, g, edges, senders)
    assert np.allclose(dx, got[0][senders], atol=1e-12)
    assert np.allclose(dy, got[1][edges], atol=1e-12)
    assert np.allclose(dw, got[2], atol=1e-11)


# ------------------------------------------------------------------------------ uvw double backward

def _uvw_dbl_inputs(prob, rng, n_nodes=7, n_edges=27):
    row_ptr, col = small_graph(rng, n_nodes, n_edges)
    x, ggx = rng.standard_normal((2, n_nodes, prob.d_in))
    y, ggy = rng.standard_normal((2, n_edges, prob.d_sh))
    w, ggw = rng.standard_normal((2, prob.weight_numel))
    g = rng.standard_normal((n_nodes, prob.d_out))
    return row_ptr, col, x, y, w, g, ggx, ggy, ggw


@pytest.mark.parametrize("ins,lmax,outs", [
    ("3x0e+2x1o+2x2e", 2, "2x0e+3x1o+2x2e+1x1e+2x2o"),
    ("2x0e+1x1o+2x2e+1x3o", 3, "1x0e+2x1o+1x2e+2x3o+1x1e"),
    ("17x0e+3x1o", 1, "18x1o+2x0e+19x1e")])
def test_uvw_double_backward_matches_autograd_of_dense_einsum(ins, lmax, outs):
    """Brute force: torch autograd (CPU, float64) differentiates twice through the dense coupling
    of the uvw convolution (shared weights, multiplicity mixing inside the coupling tensor)."""
    import torch
    prob = irreps.build_problem(ins, irreps.sh_irreps(lmax), outs, "uvw")
    rng = np.random.default_rng(41)
    row_ptr, col, x, y, w, g, ggx, ggy, ggw = _uvw_dbl_inputs(prob, rng)
    t = torch.from_numpy(dense_tensor(prob))
    dst = torch.from_numpy(ref.receivers_of(row_ptr))
    colt = torch.from_numpy(np.asarray(col, np.int64))
    X, Y, W, G = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, y, w, g))

    def forward(x_, y_, w_):
        msg = torch.einsum("abvo,ea,eb,v->eo", t, x_[colt], y_, w_)
        return torch.zeros(len(row_ptr) - 1, prob.d_out, dtype=torch.float64).index_add(0, dst, msg)

    first = torch.autograd.grad((G * forward(X, Y, W)).sum(), (X, Y, W), create_graph=True)
    l2 = sum((torch.from_numpy(u) * v).sum() for u, v in zip((ggx, ggy, ggw), first))
    want = torch.autograd.grad(l2, (X, Y, W, G))
    got = ref.conv_double_backward_uvw(prob, row_ptr, col, x, y, w, g, ggx, ggy, ggw)
    for a, b in zip(got, want):
        assert np.allclose(a, b.numpy(), atol=1e-11, rtol=1e-11)


def test_uvw_double_backward_euler_identities_and_finite_differences():
    """L2 = A + B + C with A = <ggx, dx>, B = <ggy, dy>, C = <ggw, dW> is linear in each operand:
    <d/dx, x> = B + C, <d/dy, y> = A + C, <d/dW, W> = A + B, <d/dg, g> = A + B + C; and central
    differences of L2 (through the first-order oracle) match the derivatives."""
    prob = _uvw_conv_problem()
    rng = np.random.default_rng(42)
    row_ptr, col, x, y, w, g, ggx, ggy, ggw = _uvw_dbl_inputs(prob, rng, 6, 23)
    dx1, dy1, dw1 = ref.conv_backward_uvw(prob, row_ptr, col, x, y, w, g)
    A, B, C = np.sum(ggx * dx1), np.sum(ggy * dy1), np.sum(ggw * dw1)
    got = ref.conv_double_backward_uvw(prob, row_ptr, col, x, y, w, g, ggx, ggy, ggw)
    scale = max(1.0, abs(A) + abs(B) + abs(C))
    for d, v, want in zip(got, (x, y, w, g), (B + C, A + C, A + B, A + B + C)):
        assert abs(np.sum(d * v) - want) <= 1e-11 * scale

    def l2(x_, y_, w_, g_):
        a, b, c = ref.conv_backward_uvw(prob, row_ptr, col, x_, y_, w_, g_)
        return np.sum(ggx * a) + np.sum(ggy * b) + np.sum(ggw * c)

    h = 1e-6
    base = [x, y, w, g]
    for which in range(4):
        for _ in range(4):
            arr = base[which]
            idx = tuple(rng.integers(0, s) for s in arr.shape)
            plus, minus = list(base), list(base)
            plus[which], minus[which] = arr.copy(), arr.copy()
            plus[which][idx] += h
            minus[which][idx] -= h
            fd = (l2(*plus) - l2(*minus)) / (2 * h)
            assert abs(fd - got[which][idx]) < 1e-6 * max(1.0, abs(got[which][idx]))


@pytest.mark.parametrize("improper", [False, True])
def test_uvw_double_backward_equivariance(improper):
    """Rotating x, the edge vectors and g (and the upstream gradients like what they multiply)
    rotates d/dx, d/dy and d/dg and leaves d/dW unchanged."""
    prob = _uvw_conv_problem()
    rng = np.random.default_rng(43)
    row_ptr, col, x, _, w, g, ggx, ggy, ggw = _uvw_dbl_inputs(prob, rng)
    vec = rng.standard_normal((len(col), 3))
    rot = wigner.random_rotation(rng)
    lin = -rot if improper else rot
    d_in, d_sh, d_out = (wigner.irreps_d(ir, rot, improper) for ir in (prob.ins, prob.sh, prob.out))
    lmax = prob.sh[-1].l
    y, y_rot = osh.real_sh_all(lmax, vec), osh.real_sh_all(lmax, vec @ lin.T)
    a = ref.conv_double_backward_uvw(prob, row_ptr, col, x, y, w, g, ggx, ggy @ np.eye(prob.d_sh), ggw)
    b = ref.conv_double_backward_uvw(prob, row_ptr, col, x @ d_in.T, y_rot, w, g @ d_out.T, ggx @ d_in.T,
                                     ggy @ d_sh.T, ggw)
    assert np.allclose(b[0], a[0] @ d_in.T, atol=1e-10)
    assert np.allclose(b[1], a[1] @ d_sh.T, atol=1e-10)
    assert np.allclose(b[2], a[2], atol=1e-10)
    assert np.allclose(b[3], a[3] @ d_out.T, atol=1e-10)
