"""The operations, written as their plain definitions in numpy (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: "An Efficient Sparse Kernel Generator for O(3)-Equivariant Deep
Networks" (sciencestack.ai page).  Abstract and Figure 1: the CG tensor
product contracts the block-sparse tensor with two dense vectors and then
applies a structured weight; Figure 4: use case A (a batch of independent
rows) and use case B (graph convolution: node features combined with edge
features, messages summed into the receiving node).  The abstract also names
the gradient of the product.  The Sobek page (Abstract) states the same
convolution without edge-sized intermediates; it does not change the values.

Every function loops over paths and CG nonzeros in the order the paths are
enumerated and is vectorised over rows/edges and channels only.  All
arithmetic is float64.  For path p = (i1, i2, l3) with real CG block C_p and
a nonzero C_p[i, j, k] (the readings are in ``oracle.irreps``/``oracle.cg``):

uvu   out[r, o_q + u(2l3+1) + k] += W[r, w_p + u] * C x[s, a + u(2l1+1) + i] * y[r, b + j]
uvw   out[r, o_q + w(2l3+1) + k] += sum_u W_p[u, w] * C x[s, a + u(2l1+1) + i] * y[r, b + j]

For the batched product s = r; for the convolution the row r is an edge e in
receiver-CSR order, s = col[e] its sender and the sum runs over the edges of
each receiver n.  No extra path normalisation factor is applied.
"""
import numpy as np

from .cg import nonzeros
from .irreps import Problem, offsets


def _layout(prob: Problem):
    return offsets(prob.ins), offsets(prob.sh), offsets(prob.out)


def _path_terms(prob: Problem):
    """Yield (path, a, b, o, mul_in, mul_out, nz) with block offsets."""
    oa, ob, oo = _layout(prob)
    for p in prob.paths:
        yield (p, oa[p.i1], ob[p.i2], oo[p.slot], prob.ins[p.i1].mul, prob.out[p.slot].mul,
               nonzeros(p.l1, p.l2, p.l3))


def edge_messages(prob: Problem, xs: np.ndarray, y: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Per-row tensor product: xs[r] is the input row used by row r (uvu only)."""
    assert prob.mode == "uvu"
    rows = xs.shape[0]
    msg = np.zeros((rows, prob.d_out))
    for p, a, b, o, mul, _, nz in _path_terms(prob):
        n1, n3 = 2 * p.l1 + 1, 2 * p.l3 + 1
        xb = xs[:, a:a + mul * n1].reshape(rows, mul, n1)
        wb = w[:, p.w_off:p.w_off + mul]                        # (rows, mul)
        ob = msg[:, o:o + mul * n3].reshape(rows, mul, n3)      # view into msg
        for i, j, k, c in nz:
            ob[:, :, k] += wb * (c * xb[:, :, i] * y[:, b + j][:, None])
    return msg


def tp_forward(prob: Problem, x, y, w):
    """Batched CG tensor product, use case A.  uvu: w (B, P*mul); uvw: w shared, flat."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    w = np.asarray(w, np.float64)
    if prob.mode == "uvu":
        return edge_messages(prob, x, y, w)
    rows = x.shape[0]
    out = np.zeros((rows, prob.d_out))
    for p, a, b, o, mul_in, mul_out, nz in _path_terms(prob):
        n1, n3 = 2 * p.l1 + 1, 2 * p.l3 + 1
        xb = x[:, a:a + mul_in * n1].reshape(rows, mul_in, n1)
        wp = w[p.w_off:p.w_off + mul_in * mul_out].reshape(mul_in, mul_out)
        t = np.zeros((rows, mul_in, n3))
        for i, j, k, c in nz:
            t[:, :, k] += c * xb[:, :, i] * y[:, b + j][:, None]
        ob = out[:, o:o + mul_out * n3].reshape(rows, mul_out, n3)
        ob += np.einsum("ruk,uw->rwk", t, wp)
    return out


def receivers_of(row_ptr: np.ndarray) -> np.ndarray:
    """Receiver index of every edge of a receiver-sorted CSR."""
    row_ptr = np.asarray(row_ptr, np.int64)
    return np.repeat(np.arange(len(row_ptr) - 1), np.diff(row_ptr))


def conv_forward(prob: Problem, row_ptr, col, x, y, w):
    """Fused convolution, use case B: out[n] = sum over edges e of n of TP(x[col[e]], y[e], W_e).

    uvu: W_e = W[e] (per-edge weights).  uvw: W_e = W, the shared [P][mul_in][mul_out] block for
    every edge (the fully connected multiplicity mixing of the Sobek page, Abstract, inside the
    convolution)."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    w = np.asarray(w, np.float64)
    col = np.asarray(col, np.int64)
    n_nodes = len(row_ptr) - 1
    msg = edge_messages(prob, x[col], y, w) if prob.mode == "uvu" else tp_forward(prob, x[col], y, w)
    out = np.zeros((n_nodes, prob.d_out))
    np.add.at(out, receivers_of(row_ptr), msg)
    return out


def conv_backward_uvw(prob: Problem, row_ptr, col, x, y, w, g):
    """Gradients of sum(g * conv_forward(...)) for a uvw plan (shared W): every edge is a row of
    the batched product with x[col[e]], y[e] and g[receiver(e)]; dY is that row's gradient, dW the
    sum over the edges and dx the sum over each sender's edges."""
    x, y, w, g = (np.asarray(a, np.float64) for a in (x, y, w, g))
    col = np.asarray(col, np.int64)
    dxs, dy, dw = tp_backward(prob, x[col], y, w, g[receivers_of(row_ptr)])
    dx = np.zeros_like(x)
    np.add.at(dx, col, dxs)
    return dx, dy, dw


def conv_backward(prob: Problem, row_ptr, col, x, y, w, g):
    """Gradients of sum(g * conv_forward(...)) with respect to x, y and W.

    For each path and nonzero (i, j, k, c), with n the receiver and s the
    sender of edge e:
      dW[e, w_p + u]   += c * x[s,u,i] * y[e,j] * g[n,u,k]
      dY[e, b + j]     += c * W[e,p,u] * x[s,u,i] * g[n,u,k]   (summed over u)
      dx[s, a + u..+i] += c * W[e,p,u] * y[e,j] * g[n,u,k]     (summed over e)
    """
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    w = np.asarray(w, np.float64)
    g = np.asarray(g, np.float64)
    col = np.asarray(col, np.int64)
    dst = receivers_of(row_ptr)
    n_edges = len(col)
    xs, gs = x[col], g[dst]
    dxs = np.zeros_like(xs)
    dy = np.zeros_like(y)
    dw = np.zeros_like(w)
    for p, a, b, o, mul, _, nz in _path_terms(prob):
        n1, n3 = 2 * p.l1 + 1, 2 * p.l3 + 1
        xb = xs[:, a:a + mul * n1].reshape(n_edges, mul, n1)
        dxb = dxs[:, a:a + mul * n1].reshape(n_edges, mul, n1)
        gb = gs[:, o:o + mul * n3].reshape(n_edges, mul, n3)
        wb = w[:, p.w_off:p.w_off + mul]
        for i, j, k, c in nz:
            yj = y[:, b + j][:, None]
            dw[:, p.w_off:p.w_off + mul] += c * xb[:, :, i] * yj * gb[:, :, k]
            dy[:, b + j] += np.sum(c * wb * xb[:, :, i] * gb[:, :, k], axis=1)
            dxb[:, :, i] += c * wb * yj * gb[:, :, k]
    dx = np.zeros_like(x)
    np.add.at(dx, col, dxs)
    return dx, dy, dw


def conv_double_backward(prob: Problem, row_ptr, col, x, y, w, g, ggx, ggy, ggw):
    """Second-order gradients of the convolution (uvu).

    Sources: sciencestack.ai page, Abstract (the higher partial derivatives used
    for interatomic forces); OpenEquivariance discussion page (a convolution
    double backward with four results); Sobek page, Abstract (forward, backward
    and double backward of the same operator).

    With (dx, dy, dW) = conv_backward(x, y, W, g) and upstream gradients
    (ggx, ggy, ggw) for them, the scalar is
        L2 = <ggx, dx> + <ggy, dy> + <ggw, dW>
           = sum over edges e = (s -> n), paths p, channels u, nonzeros (i, j, k, c) of
             c * g[n,u,k] * (ggx[s,u,i] y[e,j] W[e,p,u] + x[s,u,i] ggy[e,j] W[e,p,u]
                             + x[s,u,i] y[e,j] ggw[e,p,u])
    and the four results are its derivatives, term by term:
      d/dx[s,u,i]   = sum c g_k (ggy_j W + y_j ggw)          (summed over the edges of s)
      d/dy[e,j]     = sum_u c g_k (ggx_i W + x_i ggw)
      d/dW[e,p,u]   = sum c g_k (ggx_i y_j + x_i ggy_j)
      d/dg[n,u,k]   = sum c (ggx_i y_j W + x_i ggy_j W + x_i y_j ggw)   (summed over the edges of n)
    Returns (dx, dy, dw, dg), float64.
    """
    x, y, w, g, ggx, ggy, ggw = (np.asarray(a, np.float64) for a in (x, y, w, g, ggx, ggy, ggw))
    col = np.asarray(col, np.int64)
    dst = receivers_of(row_ptr)
    n_edges = len(col)
    xs, gxs, gs = x[col], ggx[col], g[dst]
    dxs = np.zeros_like(xs)
    dy = np.zeros_like(y)
    dw = np.zeros_like(w)
    dgs = np.zeros((n_edges, prob.d_out))
    for p, a, b, o, mul, _, nz in _path_terms(prob):
        n1, n3 = 2 * p.l1 + 1, 2 * p.l3 + 1
        xb = xs[:, a:a + mul * n1].reshape(n_edges, mul, n1)
        gxb = gxs[:, a:a + mul * n1].reshape(n_edges, mul, n1)
        dxb = dxs[:, a:a + mul * n1].reshape(n_edges, mul, n1)
        gb = gs[:, o:o + mul * n3].reshape(n_edges, mul, n3)
        dgb = dgs[:, o:o + mul * n3].reshape(n_edges, mul, n3)
        wb = w[:, p.w_off:p.w_off + mul]
        gwb = ggw[:, p.w_off:p.w_off + mul]
        for i, j, k, c in nz:
            yj = y[:, b + j][:, None]
            gyj = ggy[:, b + j][:, None]
            dxb[:, :, i] += c * gb[:, :, k] * (gyj * wb + yj * gwb)
            dy[:, b + j] += np.sum(c * gb[:, :, k] * (gxb[:, :, i] * wb + xb[:, :, i] * gwb), axis=1)
            dw[:, p.w_off:p.w_off + mul] += c * gb[:, :, k] * (gxb[:, :, i] * yj + xb[:, :, i] * gyj)
            dgb[:, :, k] += c * (gxb[:, :, i] * yj * wb + xb[:, :, i] * gyj * wb + xb[:, :, i] * yj * gwb)
    dx = np.zeros_like(x)
    np.add.at(dx, col, dxs)
    dg = np.zeros_like(g)
    np.add.at(dg, dst, dgs)
    return dx, dy, dw, dg


def conv_double_backward_uvw(prob: Problem, row_ptr, col, x, y, w, g, ggx, ggy, ggw):
    """Second-order gradients of the convolution with shared weights (uvw).

    Sources as for the uvu double backward; the Sobek page (Abstract) carries both operator
    families, the fully connected one included, through the double backward.  With
    (dx, dy, dW) = conv_backward_uvw(x, y, W, g) and upstream gradients (ggx, ggy, ggw),
        L2 = <ggx, dx> + <ggy, dy> + <ggw, dW>
           = sum over edges e = (s -> n), paths p, channels u, w, nonzeros (i, j, k, c) of
             c * g[n,w,k] * (W_p[u,w] (ggx[s,u,i] y[e,j] + x[s,u,i] ggy[e,j]) + ggw_p[u,w] x[s,u,i] y[e,j])
    and, term by term, with G_p[n,u,k] = sum_w W_p[u,w] g[n,w,k] and G'_p the same with ggw:
      d/dx[s,u,i]    = sum c (ggy_j G_k + y_j G'_k)                 (summed over the edges of s)
      d/dy[e,j]      = sum_u c (ggx_i G_k + x_i G'_k)
      d/dW_p[u,w]    = sum_e c g[n,w,k] (ggx_i y_j + x_i ggy_j)
      d/dg[n,w,k]    = sum_e c (sum_u W_p[u,w] (ggx_i y_j + x_i ggy_j) + sum_u ggw_p[u,w] x_i y_j)
    Returns (dx, dy, dw, dg), float64, dw shaped like w."""
    x, y, w, g, ggx, ggy, ggw = (np.asarray(a, np.float64) for a in (x, y, w, g, ggx, ggy, ggw))
    col = np.asarray(col, np.int64)
    dst = receivers_of(row_ptr)
    n_edges = len(col)
    xs, gxs, gs = x[col], ggx[col], g[dst]
    dxs = np.zeros_like(xs)
    dy = np.zeros_like(y)
    dw = np.zeros_like(w)
    dgs = np.zeros((n_edges, prob.d_out))
    for p, a, b, o, mul_in, mul_out, nz in _path_terms(prob):
        n1, n3 = 2 * p.l1 + 1, 2 * p.l3 + 1
        xb = xs[:, a:a + mul_in * n1].reshape(n_edges, mul_in, n1)
        gxb = gxs[:, a:a + mul_in * n1].reshape(n_edges, mul_in, n1)
        dxb = dxs[:, a:a + mul_in * n1].reshape(n_edges, mul_in, n1)
        gb = gs[:, o:o + mul_out * n3].reshape(n_edges, mul_out, n3)
        dgb = dgs[:, o:o + mul_out * n3].reshape(n_edges, mul_out, n3)
        wp = w[p.w_off:p.w_off + mul_in * mul_out].reshape(mul_in, mul_out)
        gwp = ggw[p.w_off:p.w_off + mul_in * mul_out].reshape(mul_in, mul_out)
        dwp = dw[p.w_off:p.w_off + mul_in * mul_out].reshape(mul_in, mul_out)
        G = np.einsum("uw,ewk->euk", wp, gb)
        Gp = np.einsum("uw,ewk->euk", gwp, gb)
        for i, j, k, c in nz:
            yj = y[:, b + j][:, None]
            gyj = ggy[:, b + j][:, None]
            dxb[:, :, i] += c * (gyj * G[:, :, k] + yj * Gp[:, :, k])
            dy[:, b + j] += c * np.sum(gxb[:, :, i] * G[:, :, k] + xb[:, :, i] * Gp[:, :, k], axis=1)
            mixed = gxb[:, :, i] * yj + xb[:, :, i] * gyj           # (e, u)
            dwp += c * np.einsum("eu,ew->uw", mixed, gb[:, :, k])
            dgb[:, :, k] += c * (mixed @ wp + (xb[:, :, i] * yj) @ gwp)
    dx = np.zeros_like(x)
    np.add.at(dx, col, dxs)
    dg = np.zeros_like(g)
    np.add.at(dg, dst, dgs)
    return dx, dy, dw, dg


def edge_messages_uvw(prob: Problem, xs: np.ndarray, y: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Per-row uvw tensor product with a weight block of its own per row: w (rows, weight_numel),
    row r's W_p[u, w] at w[r, w_p + u * mul_out + w] (the fully connected family of the Sobek
    page, Abstract, with edge-conditioned weights)."""
    assert prob.mode == "uvw"
    rows = xs.shape[0]
    msg = np.zeros((rows, prob.d_out))
    for p, a, b, o, mul_in, mul_out, nz in _path_terms(prob):
        n1, n3 = 2 * p.l1 + 1, 2 * p.l3 + 1
        xb = xs[:, a:a + mul_in * n1].reshape(rows, mul_in, n1)
        wp = w[:, p.w_off:p.w_off + mul_in * mul_out].reshape(rows, mul_in, mul_out)
        t = np.zeros((rows, mul_in, n3))
        for i, j, k, c in nz:
            t[:, :, k] += c * xb[:, :, i] * y[:, b + j][:, None]
        msg[:, o:o + mul_out * n3].reshape(rows, mul_out, n3)[...] += np.einsum("ruk,ruw->rwk", t, wp)
    return msg


def edge_backward_uvw(prob: Problem, xs: np.ndarray, y: np.ndarray, w: np.ndarray, gr: np.ndarray):
    """Gradients of sum(gr * edge_messages_uvw(xs, y, w)) with respect to xs, y and the per-row w.
    For each path and nonzero (i, j, k, c), with h[r, u, k] = sum_w W_r,p[u, w] gr[r, w, k]:
      dxs[r, u, i] += c * y[r, j] * h[r, u, k]
      dy[r, j]     += c * sum_u xs[r, u, i] * h[r, u, k]
      dW_r,p[u, w] += c * xs[r, u, i] * y[r, j] * gr[r, w, k]"""
    assert prob.mode == "uvw"
    rows = xs.shape[0]
    dxs = np.zeros_like(xs)
    dy = np.zeros_like(y)
    dw = np.zeros_like(w)
    for p, a, b, o, mul_in, mul_out, nz in _path_terms(prob):
        n1, n3 = 2 * p.l1 + 1, 2 * p.l3 + 1
        xb = xs[:, a:a + mul_in * n1].reshape(rows, mul_in, n1)
        dxb = dxs[:, a:a + mul_in * n1].reshape(rows, mul_in, n1)
        wp = w[:, p.w_off:p.w_off + mul_in * mul_out].reshape(rows, mul_in, mul_out)
        gb = gr[:, o:o + mul_out * n3].reshape(rows, mul_out, n3)
        h = np.einsum("ruw,rwk->ruk", wp, gb)
        t = np.zeros((rows, mul_in, n3))
        for i, j, k, c in nz:
            dxb[:, :, i] += c * y[:, b + j][:, None] * h[:, :, k]
            dy[:, b + j] += c * np.sum(xb[:, :, i] * h[:, :, k], axis=1)
            t[:, :, k] += c * xb[:, :, i] * y[:, b + j][:, None]
        dw[:, p.w_off:p.w_off + mul_in * mul_out] += np.einsum("ruk,rwk->ruw", t, gb).reshape(rows, -1)
    return dxs, dy, dw


def conv_forward_radial(prob: Problem, row_ptr, col, x, y, rho, theta):
    """Convolution whose per-edge weights are a radial projection: W_e = rho[e] @ Theta.

    Source: Sobek page, Abstract (edge-conditioned weights from a radial projection, which the
    streaming formulation reassociates with the coupling and the aggregation so that W_e is
    never stored; both operator families).  rho [E][R] holds each edge's radial features, Theta
    [R][weight_numel] is shared.  The plain definition: form W = rho @ Theta, then the convolution
    with those per-edge weights (uvu: conv_forward; uvw: each edge's own W_p blocks)."""
    w = np.asarray(rho, np.float64) @ np.asarray(theta, np.float64)
    if prob.mode == "uvu":
        return conv_forward(prob, row_ptr, col, x, y, w)
    x = np.asarray(x, np.float64)
    col = np.asarray(col, np.int64)
    out = np.zeros((len(row_ptr) - 1, prob.d_out))
    np.add.at(out, receivers_of(row_ptr), edge_messages_uvw(prob, x[col], np.asarray(y, np.float64), w))
    return out


def conv_backward_radial(prob: Problem, row_ptr, col, x, y, rho, theta, g):
    """Gradients of sum(g * conv_forward_radial(x, y, rho, Theta)) with respect to x, y, rho and
    Theta.

    Sobek page, Abstract: the radial projection is reassociated through the backward as well.  The
    plain definition is the chain rule through W = rho @ Theta (library matmuls):
      (dx, dy, dW) = the convolution's gradients with per-edge weights W,
      drho = dW @ Theta^T,   dTheta = rho^T @ dW."""
    rho = np.asarray(rho, np.float64)
    theta = np.asarray(theta, np.float64)
    if prob.mode == "uvu":
        dx, dy, dw = conv_backward(prob, row_ptr, col, x, y, rho @ theta, g)
    else:
        x, y, g = (np.asarray(a, np.float64) for a in (x, y, g))
        col = np.asarray(col, np.int64)
        dxs, dy, dw = edge_backward_uvw(prob, x[col], y, rho @ theta, g[receivers_of(row_ptr)])
        dx = np.zeros_like(x)
        np.add.at(dx, col, dxs)
    return dx, dy, dw @ theta.T, rho.T @ dw


def tp_backward(prob: Problem, x, y, w, g):
    """Gradients of sum(g * tp_forward(x, y, W)) for the batched product (use case A).

    sciencestack.ai page, Abstract (gradient kernels) and Figure 4A.  uvu: per row, as the
    convolution backward on the identity graph.  uvw (shared W_p [mul_in][mul_out]), for each path
    and nonzero (i, j, k, c):
      dx[b, u, i]   += c * y[b, j] * sum_w W_p[u, w] g[b, w, k]
      dy[b, j]      += c * sum_u x[b, u, i] * sum_w W_p[u, w] g[b, w, k]
      dW_p[u, w]    += c * sum_b x[b, u, i] y[b, j] g[b, w, k]
    Returns (dx, dy, dw) with dw shaped like w."""
    x, y, w, g = (np.asarray(a, np.float64) for a in (x, y, w, g))
    rows = x.shape[0]
    if prob.mode == "uvu":
        ident = np.arange(rows + 1)
        return conv_backward(prob, ident, np.arange(rows), x, y, w, g)
    dx = np.zeros_like(x)
    dy = np.zeros_like(y)
    dw = np.zeros_like(w)
    for p, a, b, o, mul_in, mul_out, nz in _path_terms(prob):
        n1, n3 = 2 * p.l1 + 1, 2 * p.l3 + 1
        xb = x[:, a:a + mul_in * n1].reshape(rows, mul_in, n1)
        dxb = dx[:, a:a + mul_in * n1].reshape(rows, mul_in, n1)
        gb = g[:, o:o + mul_out * n3].reshape(rows, mul_out, n3)
        wp = w[p.w_off:p.w_off + mul_in * mul_out].reshape(mul_in, mul_out)
        gw = np.einsum("uw,rwk->ruk", wp, gb)               # sum_w W_p[u, w] g[b, w, k]
        dwp = dw[p.w_off:p.w_off + mul_in * mul_out].reshape(mul_in, mul_out)
        for i, j, k, c in nz:
            yj = y[:, b + j][:, None]
            dxb[:, :, i] += c * yj * gw[:, :, k]
            dy[:, b + j] += c * np.sum(xb[:, :, i] * gw[:, :, k], axis=1)
            dwp += c * np.einsum("ru,r,rw->uw", xb[:, :, i], y[:, b + j], gb[:, :, k])
    return dx, dy, dw
