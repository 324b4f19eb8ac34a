"""Thin ctypes binding of libcgtp (include/cgtp.h): same names, argument marshalling only.

Every step runs in the library's HIP kernels.  Torch supplies device memory
and the stream (``torch.cuda.current_stream().cuda_stream``); when an output
tensor is not given, it is allocated here with ``torch.empty`` -- the only
allocation on the path, and one the library itself never makes.  If
``libcgtp.so`` is missing the first call raises: there is no fallback.
"""
import ctypes
import os
from functools import lru_cache

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcgtp.so")

CGTP_UVU, CGTP_UVW = 0, 1
CGTP_F32, CGTP_F64 = 0, 1
STATUS = {0: "CGTP_OK", 1: "CGTP_ERR_INVALID_ARG", 2: "CGTP_ERR_IRREPS", 3: "CGTP_ERR_UNSUPPORTED",
          4: "CGTP_ERR_COMPILE", 5: "CGTP_ERR_HIP", 6: "CGTP_ERR_INTERNAL"}
STATUS_CODES = {v: k for k, v in STATUS.items()}

EXPORTS = ("cgtp_plan_create", "cgtp_plan_destroy", "cgtp_plan_info_get", "cgtp_plan_path",
           "cgtp_plan_path_coefficients", "cgtp_plan_source", "cgtp_tp_forward", "cgtp_conv_forward",
           "cgtp_graph_transpose", "cgtp_conv_backward", "cgtp_spherical_harmonics", "cgtp_last_error",
           "cgtp_conv_forward_ordered", "cgtp_graph_order", "cgtp_conv_double_backward", "cgtp_tp_backward",
           "cgtp_conv_forward_radial", "cgtp_plan_radial_prepare", "cgtp_plan_radial_source",
           "cgtp_tp_backward_workspace_size", "cgtp_plan_uvw_backward_prepare", "cgtp_plan_uvw_backward_source",
           "cgtp_conv_backward_workspace_size", "cgtp_conv_backward_ws", "cgtp_plan_conv_uvw_backward_prepare",
           "cgtp_plan_conv_uvw_backward_source", "cgtp_conv_backward_radial", "cgtp_conv_backward_radial_workspace_size",
           "cgtp_conv_row_split", "cgtp_tp_backward_noalloc", "cgtp_conv_backward_receiver",
           "cgtp_conv_backward_receiver_workspace_size", "cgtp_conv_double_backward_workspace_size",
           "cgtp_conv_double_backward_ws")
_STRING_RESULTS = ("cgtp_last_error", "cgtp_plan_source", "cgtp_plan_radial_source", "cgtp_plan_uvw_backward_source",
                   "cgtp_plan_conv_uvw_backward_source")


class CgtpError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class PlanInfo(ctypes.Structure):
    _fields_ = [("d_x", ctypes.c_int32), ("d_sh", ctypes.c_int32), ("d_out", ctypes.c_int32),
                ("num_paths", ctypes.c_int32), ("weight_numel", ctypes.c_int64),
                ("nnz_total", ctypes.c_int32), ("mode", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("fwd_tasks", ctypes.c_int32)]


class PathInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("i1", "i2", "slot", "l1", "l2", "l3", "p3", "x_off", "y_off",
                                              "out_off", "mul_in", "mul_out")] + \
               [("w_off", ctypes.c_int64), ("nnz", ctypes.c_int32)]


_lib = None


def lib():
    """Load libcgtp.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m clebsch_gordan_tensor_cgtp_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.cgtp_last_error.restype = ctypes.c_char_p
        L.cgtp_plan_source.restype = ctypes.c_char_p
        L.cgtp_plan_radial_source.restype = ctypes.c_char_p
        L.cgtp_plan_uvw_backward_source.restype = ctypes.c_char_p
        L.cgtp_plan_conv_uvw_backward_source.restype = ctypes.c_char_p
        L.cgtp_plan_conv_uvw_backward_source.argtypes = [vp, i32]
        L.cgtp_conv_backward_workspace_size.argtypes = [vp, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
        L.cgtp_conv_backward_ws.argtypes = [vp, i64, i64] + [vp] * 14 + [ctypes.c_size_t, vp]
        L.cgtp_conv_backward_radial_workspace_size.argtypes = [vp, i64, i64, i32, ctypes.POINTER(ctypes.c_size_t)]
        L.cgtp_conv_backward_radial.argtypes = [vp, i64, i64] + [vp] * 7 + [i32] + [vp] * 8 + [ctypes.c_size_t, vp]
        L.cgtp_plan_source.argtypes = [vp]
        L.cgtp_conv_row_split.argtypes = [vp, i64, i64, i32, ctypes.POINTER(i32)]
        L.cgtp_plan_create.argtypes = [ctypes.c_char_p] * 3 + [ctypes.c_int, ctypes.c_int, ctypes.POINTER(vp)]
        L.cgtp_plan_destroy.argtypes = [vp]
        L.cgtp_plan_info_get.argtypes = [vp, ctypes.POINTER(PlanInfo)]
        L.cgtp_plan_path.argtypes = [vp, i32, ctypes.POINTER(PathInfo)]
        L.cgtp_plan_path_coefficients.argtypes = [vp, i32, i32, vp, vp, ctypes.POINTER(i32)]
        L.cgtp_tp_forward.argtypes = [vp, i64, vp, vp, vp, ctypes.c_int, vp, vp]
        L.cgtp_tp_backward.argtypes = [vp, i64, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.cgtp_tp_backward_noalloc.argtypes = [vp, i64, vp, vp, vp, ctypes.c_int, vp, vp, vp, vp, vp]
        L.cgtp_tp_backward_workspace_size.argtypes = [vp, i64, ctypes.POINTER(ctypes.c_size_t)]
        L.cgtp_conv_backward_receiver.argtypes = [vp, i64, i64] + [vp] * 12 + [ctypes.c_size_t, vp]
        L.cgtp_conv_backward_receiver_workspace_size.argtypes = [vp, i64, i64, ctypes.POINTER(ctypes.c_size_t),
                                                                 ctypes.POINTER(ctypes.c_size_t)]
        L.cgtp_plan_uvw_backward_prepare.argtypes = [vp]
        L.cgtp_plan_uvw_backward_source.argtypes = [vp]
        L.cgtp_plan_conv_uvw_backward_prepare.argtypes = [vp]
        L.cgtp_plan_radial_prepare.argtypes = [vp, i32]
        L.cgtp_plan_radial_source.argtypes = [vp, i32]
        L.cgtp_conv_forward_radial.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp]
        L.cgtp_conv_double_backward.argtypes = [vp, i64, i64] + [vp] * 18
        L.cgtp_conv_double_backward_workspace_size.argtypes = [vp, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
        L.cgtp_conv_double_backward_ws.argtypes = [vp, i64, i64] + [vp] * 18 + [ctypes.c_size_t, vp]
        L.cgtp_conv_forward.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        L.cgtp_conv_forward_ordered.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp]
        L.cgtp_graph_order.argtypes = [i64, vp, vp, vp]
        L.cgtp_graph_transpose.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp]
        L.cgtp_conv_backward.argtypes = [vp, i64, i64] + [vp] * 13
        L.cgtp_spherical_harmonics.argtypes = [i32, ctypes.c_int, i64, vp, vp, vp]
        for name in EXPORTS:
            if name not in _STRING_RESULTS:
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def last_error() -> str:
    return lib().cgtp_last_error().decode()


def _check(status):
    if status != 0:
        raise CgtpError(status, last_error())


# ------------------------------------------------------------------------------------ plans

class Plan:
    def __init__(self, in_irreps, sh_irreps, out_irreps, mode="uvu", dtype="f32"):
        self._h = None
        self.mode, self.dtype = mode, dtype
        self.irreps = (in_irreps, sh_irreps, out_irreps)
        h = ctypes.c_void_p()
        _check(lib().cgtp_plan_create(in_irreps.encode(), sh_irreps.encode(), out_irreps.encode(),
                                      {"uvu": CGTP_UVU, "uvw": CGTP_UVW}[mode],
                                      {"f32": CGTP_F32, "f64": CGTP_F64}[dtype], ctypes.byref(h)))
        self._h = h
        info = PlanInfo()
        _check(lib().cgtp_plan_info_get(h, ctypes.byref(info)))
        self.info = info
        self.d_x, self.d_sh, self.d_out = info.d_x, info.d_sh, info.d_out
        self.num_paths, self.weight_numel, self.nnz_total = info.num_paths, info.weight_numel, info.nnz_total

    @property
    def handle(self):
        return self._h

    @property
    def wide_uvw(self) -> bool:
        """A uvw plan with a multiplicity above 16: its batched backward runs the uvw convolution
        backward on the identity graph (computed once per plan)."""
        if not hasattr(self, "_wide_uvw"):
            self._wide_uvw = self.mode == "uvw" and any(
                max(self.path(p)["mul_in"], self.path(p)["mul_out"]) > 16 for p in range(self.num_paths))
        return self._wide_uvw

    @property
    def torch_dtype(self):
        import torch
        return torch.float32 if self.dtype == "f32" else torch.float64

    def path(self, p: int) -> dict:
        pi = PathInfo()
        _check(lib().cgtp_plan_path(self._h, p, ctypes.byref(pi)))
        return {f: getattr(pi, f) for f, _ in PathInfo._fields_}

    def coefficients(self, p: int):
        """(ijk int32 [nnz,3], values float64 [nnz]) of path p, as the planner computed them."""
        import numpy as np
        n = ctypes.c_int32()
        _check(lib().cgtp_plan_path_coefficients(self._h, p, 0, None, None, ctypes.byref(n)))
        ijk = np.zeros((n.value, 3), dtype=np.int32)
        vals = np.zeros(n.value, dtype=np.float64)
        _check(lib().cgtp_plan_path_coefficients(self._h, p, n.value, ijk.ctypes.data, vals.ctypes.data,
                                                 ctypes.byref(n)))
        return ijk, vals

    def row_split(self, n_nodes: int, n_edges: int, double_backward: bool = False) -> int:
        """Waves per receiver row (1, 2 or 4) of the forward (or of the double backward's receiver
        pass) for a graph of this size; kernels of split rows carry the suffix _split2/_split4."""
        v = ctypes.c_int32()
        _check(lib().cgtp_conv_row_split(self._h, n_nodes, n_edges, 1 if double_backward else 0, ctypes.byref(v)))
        return v.value

    @property
    def source(self) -> str:
        return lib().cgtp_plan_source(self._h).decode()

    def uvw_backward_source(self) -> str:
        """Generate and compile the uvw batched-backward module (host only); its source."""
        _check(lib().cgtp_plan_uvw_backward_prepare(self._h))
        return lib().cgtp_plan_uvw_backward_source(self._h).decode()

    def conv_uvw_backward_source(self, module: int = 0) -> str:
        """Generate and compile the uvw convolution-backward modules (host only); the source of
        module 0 (G and dW kernels) or 1 (the unit-weight sender pass)."""
        _check(lib().cgtp_plan_conv_uvw_backward_prepare(self._h))
        return lib().cgtp_plan_conv_uvw_backward_source(self._h, module).decode()

    def radial_source(self, R: int) -> str:
        """Generate and compile the radial-projection module for R (host only); its source."""
        _check(lib().cgtp_plan_radial_prepare(self._h, R))
        return lib().cgtp_plan_radial_source(self._h, R).decode()

    def close(self):
        if self._h is not None and _lib is not None:
            lib().cgtp_plan_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def plan_create(in_irreps, sh_irreps, out_irreps, mode="uvu", dtype="f32") -> Plan:
    return Plan(in_irreps, sh_irreps, out_irreps, mode, dtype)


def sh_irreps(lmax: int) -> str:
    return "+".join(f"1x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(lmax + 1))


def per_path_out_irreps(in_irreps: str, lmax_sh: int, lmax_out: int) -> str:
    """One output block per coupling path, in path order (string bookkeeping only)."""
    terms = []
    for term in in_irreps.replace(" ", "").split("+"):
        mul, lp = term.split("x")
        l1, p1 = int(lp[:-1]), (1 if lp[-1] == "e" else -1)
        for l2 in range(lmax_sh + 1):
            p3 = p1 * (1 if l2 % 2 == 0 else -1)
            for l3 in range(abs(l1 - l2), min(l1 + l2, lmax_out) + 1):
                terms.append(f"{mul}x{l3}{'e' if p3 == 1 else 'o'}")
    return "+".join(terms)


@lru_cache(maxsize=None)
def plan_for(spec, dtype="f32") -> Plan:
    """The plan of a workload from ``synth.WORKLOADS`` (cached per process)."""
    if hasattr(spec, "n_edges"):
        if spec.mode == "uvw":
            return Plan(spec.in_irreps, sh_irreps(spec.lmax_sh), spec.out_irreps, "uvw", dtype)
        out = per_path_out_irreps(spec.in_irreps, spec.lmax_sh, spec.lmax_out)
        return Plan(spec.in_irreps, sh_irreps(spec.lmax_sh), out, "uvu", dtype)
    if spec.mode == "uvu":
        out = per_path_out_irreps(spec.in_irreps, spec.lmax_sh, spec.lmax_sh)
        return Plan(spec.in_irreps, sh_irreps(spec.lmax_sh), out, "uvu", dtype)
    return Plan(spec.in_irreps, sh_irreps(spec.lmax_sh), spec.out_irreps, "uvw", dtype)


# ------------------------------------------------------------------------------------ calls

def _stream(stream, device=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name, dtype=None, shape=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) torch tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _ptr_or_null(t, name, dtype=None, shape=None):
    return ctypes.c_void_p(0) if t is None else _dev(t, name, dtype, shape)


def tp_forward(plan: Plan, x, y, w, out=None, stream=None):
    import torch
    B = x.shape[0]
    dt = plan.torch_dtype
    if out is None:
        out = torch.empty((B, plan.d_out), dtype=dt, device=x.device)
    shared = 1 if plan.mode == "uvw" else 0
    wshape = (plan.weight_numel,) if shared else (B, plan.weight_numel)
    _check(lib().cgtp_tp_forward(plan.handle, B, _dev(x, "x", dt, (B, plan.d_x)), _dev(y, "y", dt, (B, plan.d_sh)),
                                 _dev(w, "w", dt, wshape), shared, _dev(out, "out", dt, (B, plan.d_out)),
                                 _stream(stream, x.device)))
    return out


def tp_backward_workspace_size(plan: Plan, B: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().cgtp_tp_backward_workspace_size(plan.handle, B, ctypes.byref(n)))
    return n.value


def tp_backward(plan: Plan, x, y, w, grad_out, grad_x=None, grad_y=None, grad_w=None, need=(True, True, True),
                workspace=None, stream=None):
    """Batched product backward: returns (grad_x, grad_y, grad_w); entries not in ``need`` are None.
    uvu: per-row weights; uvw: shared weights (a workspace is allocated here unless given)."""
    import torch
    B = x.shape[0]
    dt = plan.torch_dtype
    dev = x.device
    shared = 1 if plan.mode == "uvw" else 0
    wshape = (plan.weight_numel,) if shared else (B, plan.weight_numel)
    shapes = ((B, plan.d_x), (B, plan.d_sh), wshape)
    res = [None if not nd else (torch.empty(sh, dtype=dt, device=dev) if o is None else o)
           for o, nd, sh in zip((grad_x, grad_y, grad_w), need, shapes)]
    # uvw with every multiplicity <= 16 needs the workspace for grad_w only; wider uvw plans run
    # the convolution backward on the identity graph, which needs it for every gradient
    wide = plan.wide_uvw
    wanted = res[2] is not None or (wide and any(r is not None for r in res))
    nbytes = tp_backward_workspace_size(plan, B) if wanted else 0
    if workspace is None and nbytes:
        es = 4 if plan.dtype == "f32" else 8
        workspace = torch.empty(-(-nbytes // es), dtype=dt, device=dev)
    ws = ctypes.c_void_p(0) if workspace is None else ctypes.c_void_p(workspace.data_ptr())
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().cgtp_tp_backward(plan.handle, B, _dev(x, "x", dt, shapes[0]), _dev(y, "y", dt, shapes[1]),
                                  _dev(w, "w", dt, wshape), shared, _dev(grad_out, "grad_out", dt, (B, plan.d_out)),
                                  *[_ptr_or_null(r, n, dt, sh) for r, n, sh in zip(res, ("grad_x", "grad_y", "grad_w"),
                                                                                   shapes)],
                                  ws, ctypes.c_size_t(wsb), _stream(stream, dev)))
    return tuple(res)


def tp_backward_noalloc(plan: Plan, x, y, w, grad_out, grad_x, grad_y, grad_w, stream=None):
    """cgtp_tp_backward_noalloc: the batched backward with its temporary memory in the library's
    fixed device scratch.  Every output (or None to skip it) is given by the caller; nothing is
    allocated here or in the library."""
    B = x.shape[0]
    dt = plan.torch_dtype
    shared = 1 if plan.mode == "uvw" else 0
    wshape = (plan.weight_numel,) if shared else (B, plan.weight_numel)
    shapes = ((B, plan.d_x), (B, plan.d_sh), wshape)
    _check(lib().cgtp_tp_backward_noalloc(
        plan.handle, B, _dev(x, "x", dt, shapes[0]), _dev(y, "y", dt, shapes[1]), _dev(w, "w", dt, wshape), shared,
        _dev(grad_out, "grad_out", dt, (B, plan.d_out)),
        *[_ptr_or_null(r, n, dt, sh) for r, n, sh in zip((grad_x, grad_y, grad_w), ("grad_x", "grad_y", "grad_w"),
                                                         shapes)], _stream(stream, x.device)))
    return grad_x, grad_y, grad_w


def graph_order(row_ptr, order=None, stream=None):
    """Heavy-first receiver schedule (stable by log2 degree bucket, descending)."""
    import torch
    N = row_ptr.shape[0] - 1
    order = torch.empty(N, dtype=torch.int32, device=row_ptr.device) if order is None else order
    _check(lib().cgtp_graph_order(N, _dev(row_ptr, "row_ptr", torch.int32), _dev(order, "order", torch.int32, (N,)),
                                  _stream(stream, row_ptr.device)))
    return order


def conv_forward(plan: Plan, row_ptr, col, x, y, w, out=None, order=None, stream=None):
    import torch
    N, E = row_ptr.shape[0] - 1, col.shape[0]
    dt = plan.torch_dtype
    if out is None:
        out = torch.empty((N, plan.d_out), dtype=dt, device=x.device)
    wshape = (plan.weight_numel,) if plan.mode == "uvw" else (E, plan.weight_numel)  # uvw: shared weights
    _check(lib().cgtp_conv_forward_ordered(plan.handle, N, E, _dev(row_ptr, "row_ptr", torch.int32),
                                   _dev(col, "col", torch.int32), _ptr_or_null(order, "order", torch.int32, (N,)),
                                   _dev(x, "x", dt, (N, plan.d_x)),
                                   _dev(y, "y", dt, (E, plan.d_sh)), _dev(w, "w", dt, wshape),
                                   _dev(out, "out", dt, (N, plan.d_out)), _stream(stream, x.device)))
    return out


def conv_forward_radial(plan: Plan, row_ptr, col, x, y, rho, theta, out=None, order=None, stream=None):
    """Convolution with W_e = rho[e] @ theta built in the kernel (rho [E][R], theta [R][weight_numel])."""
    import torch
    N, E = row_ptr.shape[0] - 1, col.shape[0]
    R = theta.shape[0]
    dt = plan.torch_dtype
    if out is None:
        out = torch.empty((N, plan.d_out), dtype=dt, device=x.device)
    _check(lib().cgtp_conv_forward_radial(plan.handle, N, E, _dev(row_ptr, "row_ptr", torch.int32),
                                          _dev(col, "col", torch.int32), _ptr_or_null(order, "order", torch.int32, (N,)),
                                          _dev(x, "x", dt, (N, plan.d_x)), _dev(y, "y", dt, (E, plan.d_sh)), R,
                                          _dev(rho, "rho", dt, (E, R)), _dev(theta, "theta", dt, (R, plan.weight_numel)),
                                          _dev(out, "out", dt, (N, plan.d_out)), _stream(stream, x.device)))
    return out


def conv_backward_radial_workspace_size(plan: Plan, N: int, E: int, R: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().cgtp_conv_backward_radial_workspace_size(plan.handle, N, E, R, ctypes.byref(n)))
    return n.value


def conv_backward_radial(plan: Plan, row_ptr, col, transpose, x, y, rho, theta, grad_out, outs=(None, None, None, None),
                         need=(True, True, True, True), workspace=None, stream=None):
    """Backward of the radial-projection convolution: (grad_x, grad_y, grad_rho, grad_theta); entries
    not in ``need`` are None and not computed.  The workspace (uvu: dTheta partials; uvw: those,
    G and two SH-sized rows per edge) is allocated here unless given."""
    import torch
    N, E = row_ptr.shape[0] - 1, col.shape[0]
    R = theta.shape[0]
    dt = plan.torch_dtype
    dev = x.device
    shapes = ((N, plan.d_x), (E, plan.d_sh), (E, R), (R, plan.weight_numel))
    res = [None if not nd else (torch.empty(sh, dtype=dt, device=dev) if o is None else o)
           for o, nd, sh in zip(outs, need, shapes)]
    nbytes = conv_backward_radial_workspace_size(plan, N, E, R) if res[3] is not None or plan.mode == "uvw" else 0
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ws = ctypes.c_void_p(0) if workspace is None else ctypes.c_void_p(workspace.data_ptr())
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    t_row_ptr, t_edge, t_dst = transpose
    names = ("grad_x", "grad_y", "grad_rho", "grad_theta")
    _check(lib().cgtp_conv_backward_radial(
        plan.handle, N, E, _dev(row_ptr, "row_ptr", torch.int32), _dev(col, "col", torch.int32),
        _dev(t_row_ptr, "t_row_ptr", torch.int32, (N + 1,)), _dev(t_edge, "t_edge", torch.int32, (E,)),
        _dev(t_dst, "t_dst", torch.int32, (E,)), _dev(x, "x", dt, (N, plan.d_x)), _dev(y, "y", dt, (E, plan.d_sh)), R,
        _dev(rho, "rho", dt, (E, R)), _dev(theta, "theta", dt, (R, plan.weight_numel)),
        _dev(grad_out, "grad_out", dt, (N, plan.d_out)),
        *[_ptr_or_null(r, nm, dt, sh) for r, nm, sh in zip(res, names, shapes)],
        ws, ctypes.c_size_t(wsb), _stream(stream, dev)))
    return tuple(res)


def graph_transpose(row_ptr, col, t_row_ptr=None, t_edge=None, t_dst=None, stream=None):
    import torch
    N, E = row_ptr.shape[0] - 1, col.shape[0]
    dev = row_ptr.device
    t_row_ptr = torch.empty(N + 1, dtype=torch.int32, device=dev) if t_row_ptr is None else t_row_ptr
    t_edge = torch.empty(E, dtype=torch.int32, device=dev) if t_edge is None else t_edge
    t_dst = torch.empty(E, dtype=torch.int32, device=dev) if t_dst is None else t_dst
    _check(lib().cgtp_graph_transpose(N, E, _dev(row_ptr, "row_ptr", torch.int32), _dev(col, "col", torch.int32),
                                      _dev(t_row_ptr, "t_row_ptr", torch.int32, (N + 1,)),
                                      _dev(t_edge, "t_edge", torch.int32, (E,)),
                                      _dev(t_dst, "t_dst", torch.int32, (E,)), _stream(stream, dev)))
    return t_row_ptr, t_edge, t_dst


def conv_backward_workspace_size(plan: Plan, N: int, E: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().cgtp_conv_backward_workspace_size(plan.handle, N, E, ctypes.byref(n)))
    return n.value


def conv_backward(plan: Plan, row_ptr, col, transpose, x, y, w, grad_out, grad_x=None, grad_y=None, grad_w=None,
                  need=(True, True, True), order=None, workspace=None, stream=None):
    """Returns (grad_x, grad_y, grad_w); entries not in ``need`` are None and not computed.
    uvw plans: shared weights, a workspace (allocated here unless given) and an optional
    receiver schedule ``order`` for the weight-gradient pass."""
    import torch
    N, E = row_ptr.shape[0] - 1, col.shape[0]
    dt = plan.torch_dtype
    dev = x.device
    t_row_ptr, t_edge, t_dst = transpose
    uvw = plan.mode == "uvw"
    wshape = (plan.weight_numel,) if uvw else (E, plan.weight_numel)
    if need[0] and grad_x is None:
        grad_x = torch.empty((N, plan.d_x), dtype=dt, device=dev)
    if need[1] and grad_y is None:
        grad_y = torch.empty((E, plan.d_sh), dtype=dt, device=dev)
    if need[2] and grad_w is None:
        grad_w = torch.empty(wshape, dtype=dt, device=dev)
    gx = grad_x if need[0] else None
    gy = grad_y if need[1] else None
    gw = grad_w if need[2] else None
    if uvw:
        nbytes = conv_backward_workspace_size(plan, N, E)
        if workspace is None and nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        ws = ctypes.c_void_p(0) if workspace is None else ctypes.c_void_p(workspace.data_ptr())
        wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib().cgtp_conv_backward_ws(
            plan.handle, N, E, _dev(row_ptr, "row_ptr", torch.int32), _dev(col, "col", torch.int32),
            _ptr_or_null(order, "order", torch.int32, (N,)),
            _dev(t_row_ptr, "t_row_ptr", torch.int32, (N + 1,)), _dev(t_edge, "t_edge", torch.int32, (E,)),
            _dev(t_dst, "t_dst", torch.int32, (E,)), _dev(x, "x", dt, (N, plan.d_x)),
            _dev(y, "y", dt, (E, plan.d_sh)), _dev(w, "w", dt, wshape), _dev(grad_out, "grad_out", dt, (N, plan.d_out)),
            _ptr_or_null(gx, "grad_x", dt, (N, plan.d_x)), _ptr_or_null(gy, "grad_y", dt, (E, plan.d_sh)),
            _ptr_or_null(gw, "grad_w", dt, wshape), ws, ctypes.c_size_t(wsb), _stream(stream, dev)))
        return gx, gy, gw
    _check(lib().cgtp_conv_backward(
        plan.handle, N, E, _dev(row_ptr, "row_ptr", torch.int32), _dev(col, "col", torch.int32),
        _dev(t_row_ptr, "t_row_ptr", torch.int32, (N + 1,)), _dev(t_edge, "t_edge", torch.int32, (E,)),
        _dev(t_dst, "t_dst", torch.int32, (E,)), _dev(x, "x", dt, (N, plan.d_x)), _dev(y, "y", dt, (E, plan.d_sh)),
        _dev(w, "w", dt, (E, plan.weight_numel)), _dev(grad_out, "grad_out", dt, (N, plan.d_out)),
        _ptr_or_null(gx, "grad_x", dt, (N, plan.d_x)), _ptr_or_null(gy, "grad_y", dt, (E, plan.d_sh)),
        _ptr_or_null(gw, "grad_w", dt, (E, plan.weight_numel)), _stream(stream, dev)))
    return gx, gy, gw


def conv_backward_receiver_workspace_size(plan: Plan, N: int, E: int):
    """(bytes for one edge range holding every edge, the least workspace the call accepts)."""
    full, least = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().cgtp_conv_backward_receiver_workspace_size(plan.handle, N, E, ctypes.byref(full), ctypes.byref(least)))
    return full.value, least.value


def conv_backward_receiver(plan: Plan, row_ptr, col, transpose, x, y, w, grad_out, grad_x=None, grad_y=None,
                           grad_w=None, need=(True, True, True), workspace=None, stream=None):
    """The convolution backward in receiver order (cgtp_conv_backward_receiver): returns (grad_x,
    grad_y, grad_w); entries not in ``need`` are None and not computed.  grad_x needs a workspace
    (uint8 device tensor); the edges are taken in ranges of as many dx rows as it holds.  One that
    holds every edge is allocated here unless given."""
    import torch
    N, E = row_ptr.shape[0] - 1, col.shape[0]
    dt = plan.torch_dtype
    dev = x.device
    t_row_ptr, t_edge, _ = transpose
    if need[0] and grad_x is None:
        grad_x = torch.empty((N, plan.d_x), dtype=dt, device=dev)
    if need[1] and grad_y is None:
        grad_y = torch.empty((E, plan.d_sh), dtype=dt, device=dev)
    if need[2] and grad_w is None:
        grad_w = torch.empty((E, plan.weight_numel), dtype=dt, device=dev)
    gx = grad_x if need[0] else None
    gy = grad_y if need[1] else None
    gw = grad_w if need[2] else None
    if gx is not None and workspace is None and E > 0:
        workspace = torch.empty(conv_backward_receiver_workspace_size(plan, N, E)[0], dtype=torch.uint8, device=dev)
    ws = ctypes.c_void_p(0) if workspace is None else ctypes.c_void_p(workspace.data_ptr())
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().cgtp_conv_backward_receiver(
        plan.handle, N, E, _dev(row_ptr, "row_ptr", torch.int32), _dev(col, "col", torch.int32),
        _dev(t_row_ptr, "t_row_ptr", torch.int32, (N + 1,)), _dev(t_edge, "t_edge", torch.int32, (E,)),
        _dev(x, "x", dt, (N, plan.d_x)), _dev(y, "y", dt, (E, plan.d_sh)), _dev(w, "w", dt, (E, plan.weight_numel)),
        _dev(grad_out, "grad_out", dt, (N, plan.d_out)), _ptr_or_null(gx, "grad_x", dt, (N, plan.d_x)),
        _ptr_or_null(gy, "grad_y", dt, (E, plan.d_sh)), _ptr_or_null(gw, "grad_w", dt, (E, plan.weight_numel)),
        ws, ctypes.c_size_t(wsb), _stream(stream, dev)))
    return gx, gy, gw


def conv_double_backward_workspace_size(plan: Plan, N: int, E: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().cgtp_conv_double_backward_workspace_size(plan.handle, N, E, ctypes.byref(n)))
    return n.value


def conv_double_backward(plan: Plan, row_ptr, col, transpose, x, y, w, grad_out, gg_x, gg_y, gg_w, order=None,
                         outs=(None, None, None, None), need=(True, True, True, True), workspace=None, stream=None):
    """Second-order gradients (grad_x, grad_y, grad_w, grad_grad_out) of
    <gg_x, dx> + <gg_y, dy> + <gg_w, dW>, where (dx, dy, dW) = conv_backward(x, y, w, grad_out).
    An upstream gradient given as None is passed as zeros.  Entries not in ``need`` are None
    and not computed.  uvw plans (shared weights) run cgtp_conv_double_backward_ws with a
    workspace, allocated here unless given."""
    import torch
    N, E = row_ptr.shape[0] - 1, col.shape[0]
    dt = plan.torch_dtype
    dev = x.device
    wshape = (plan.weight_numel,) if plan.mode == "uvw" else (E, plan.weight_numel)
    shapes = ((N, plan.d_x), (E, plan.d_sh), wshape, (N, plan.d_out))
    gg = [torch.zeros(sh, dtype=dt, device=dev) if t is None else t for t, sh in zip((gg_x, gg_y, gg_w), shapes)]
    res = [None if not nd else (torch.empty(sh, dtype=dt, device=dev) if o is None else o)
           for o, nd, sh in zip(outs, need, shapes)]
    t_row_ptr, t_edge, t_dst = transpose
    names = ("grad_x", "grad_y", "grad_w", "grad_grad_out")
    if plan.mode == "uvw":
        nbytes = conv_double_backward_workspace_size(plan, N, E)
        if workspace is None and nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        ws = ctypes.c_void_p(0) if workspace is None else ctypes.c_void_p(workspace.data_ptr())
        wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib().cgtp_conv_double_backward_ws(
            plan.handle, N, E, _dev(row_ptr, "row_ptr", torch.int32), _dev(col, "col", torch.int32),
            _ptr_or_null(order, "order", torch.int32, (N,)),
            _dev(t_row_ptr, "t_row_ptr", torch.int32, (N + 1,)), _dev(t_edge, "t_edge", torch.int32, (E,)),
            _dev(t_dst, "t_dst", torch.int32, (E,)), _dev(x, "x", dt, shapes[0]), _dev(y, "y", dt, shapes[1]),
            _dev(w, "w", dt, shapes[2]), _dev(grad_out, "grad_out", dt, shapes[3]),
            _dev(gg[0], "gg_x", dt, shapes[0]), _dev(gg[1], "gg_y", dt, shapes[1]), _dev(gg[2], "gg_w", dt, shapes[2]),
            *[_ptr_or_null(r, nm, dt, sh) for r, nm, sh in zip(res, names, shapes)], ws, ctypes.c_size_t(wsb),
            _stream(stream, dev)))
        return tuple(res)
    _check(lib().cgtp_conv_double_backward(
        plan.handle, N, E, _dev(row_ptr, "row_ptr", torch.int32), _dev(col, "col", torch.int32),
        _ptr_or_null(order, "order", torch.int32, (N,)),
        _dev(t_row_ptr, "t_row_ptr", torch.int32, (N + 1,)), _dev(t_edge, "t_edge", torch.int32, (E,)),
        _dev(t_dst, "t_dst", torch.int32, (E,)), _dev(x, "x", dt, shapes[0]), _dev(y, "y", dt, shapes[1]),
        _dev(w, "w", dt, shapes[2]), _dev(grad_out, "grad_out", dt, shapes[3]),
        _dev(gg[0], "gg_x", dt, shapes[0]), _dev(gg[1], "gg_y", dt, shapes[1]), _dev(gg[2], "gg_w", dt, shapes[2]),
        *[_ptr_or_null(r, nm, dt, sh) for r, nm, sh in zip(res, names, shapes)], _stream(stream, dev)))
    return tuple(res)


def spherical_harmonics(lmax: int, vec, out=None, stream=None):
    import torch
    E = vec.shape[0]
    dt = vec.dtype
    if dt not in (torch.float32, torch.float64):
        raise TypeError("vec must be float32 or float64")
    if out is None:
        out = torch.empty((E, (lmax + 1) ** 2), dtype=dt, device=vec.device)
    _check(lib().cgtp_spherical_harmonics(lmax, CGTP_F64 if dt == torch.float64 else CGTP_F32, E,
                                          _dev(vec, "vec", dt, (E, 3)), _dev(out, "y", dt, (E, (lmax + 1) ** 2)),
                                          _stream(stream, vec.device)))
    return out
