"""Benchmark of the fused CGTP convolution on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c5|c2|c3|...] [--no-cpu]
                    [--double-backward]

The default workload is the largest single-GPU convolution: the power-law graph
with 200,000 nodes and 10,000,000 edges, 64x(0e,1o,2e) features, SH l <= 2,
fp32, forward + backward with no edge-sized intermediates (Sobek page,
Abstract: the edge-scaling regime).

One step = one pass of the hot path over the synthetic graph: the fused
convolution forward (cgtp_conv_forward_ordered, heavy-first receiver schedule)
followed by the fused backward (cgtp_conv_backward: grad_x, grad_y, grad_w).
Per-graph set-up (plan and hipRTC, spherical harmonics of the edge vectors,
the sender transpose, the receiver schedule) runs before the timed region.  All inputs are resident in HBM when timing starts.

Prints one JSON line with the throughput in edges/s (forward + backward per
edge), the roofline of the dominant kernel (HIP events on the launch stream)
and the CPU oracle's rate on the host cores (``cpu_baseline``).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "edges/sec fused CGTP conv fwd (+bwd) and % of HBM / FP32 roofline"
HBM_PEAK_GBS = 8000.0
# workspace of the receiver-order backward: a fixed bound, independent of the edge count (the edges
# are taken in ranges of as many dx rows as it holds)
RECEIVER_WORKSPACE_BYTES = 4 << 30


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c5", choices=["c1", "c2", "c3", "c4", "c5", "c2uvw", "c1big", "c4wide"])
    ap.add_argument("--backward", action="store_true",
                    help="batched workloads: also time cgtp_tp_backward; uvw convolution: also cgtp_conv_backward_ws")
    ap.add_argument("--dtype", default="f32", choices=["f32", "f64"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--backward-schedule", default="sender", choices=["receiver", "sender"],
                    help="uvu convolution backward: receiver order with a bounded workspace "
                         "(cgtp_conv_backward_receiver) or sender order (cgtp_conv_backward)")
    ap.add_argument("--receiver-workspace-gib", type=float, default=RECEIVER_WORKSPACE_BYTES / 2**30,
                    help="workspace of the receiver-order backward (GiB; the call splits the edges into "
                         "as many ranges as it needs)")
    ap.add_argument("--natural-order", action="store_true",
                    help="start receivers in node order instead of the heavy-first schedule")
    ap.add_argument("--radial", type=int, default=0, metavar="R",
                    help="time the forward with radially projected weights W_e = rho_e Theta (R features per edge)")
    ap.add_argument("--double-backward", action="store_true",
                    help="time the convolution double backward (both passes) instead of forward + backward")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (calibrates the HBM byte counters)")
    ap.add_argument("--nodes", type=int, default=0,
                    help="convolution workloads: the same recipe with this many receivers (sweeps; with --edges)")
    ap.add_argument("--edges", type=int, default=0, help="convolution workloads: edge count of the --nodes variant")
    return ap.parse_args()


def copy_probe():
    """A plain copy of known size: 1 GiB read + 1 GiB written per launch, 5 launches."""
    import torch
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read_per_launch": a.numel() * 4,
                      "copy_probe_bytes_written_per_launch": b.numel() * 4, "launches": 5}), flush=True)


def algorithmic_bytes(plan, N, E, es):
    """Compulsory HBM bytes per launch: every input read once, every output written once."""
    fwd = (N + 1) * 4 + E * 4 + es * (N * plan.d_x + E * plan.d_sh + E * plan.weight_numel + N * plan.d_out)
    bwd = ((N + 1) * 4 + 2 * E * 4
           + es * (N * plan.d_x + E * plan.d_sh + E * plan.weight_numel + N * plan.d_out)
           + es * (N * plan.d_x + E * plan.d_sh + E * plan.weight_numel))
    return fwd, bwd


def algorithmic_bytes_dbl(plan, N, E, es):
    """Compulsory bytes of the two double-backward passes: inputs read once, outputs written once.
    Receiver pass: row_ptr, col, x, gg_x, y, gg_y, w, gg_w -> grad_grad_out.  Sender pass:
    t_row_ptr, t_edge, t_dst, x, gg_x, y, gg_y, w, gg_w, grad_out -> grad_x, grad_y, grad_w."""
    ops = 2 * N * plan.d_x + 2 * E * plan.d_sh + 2 * E * plan.weight_numel
    recv = (N + 1) * 4 + E * 4 + es * (ops + N * plan.d_out)
    send = (N + 1) * 4 + 2 * E * 4 + es * (ops + N * plan.d_out) + es * (N * plan.d_x + E * plan.d_sh
                                                                         + E * plan.weight_numel)
    return recv, send


def cpu_baseline_dbl(spec, seed, host_graph, max_seconds=30.0):
    """The oracle's double backward (explicit fp64 loops, OpenMP) on the sub-graph of a contiguous
    receiver slice holding ~5% of the edges, random values (timing only): all four results of the
    sub-graph, i.e. the same per-edge work as the full operation.  Rate = sub-graph edges per second."""
    from oracle import irreps as oirreps
    from oracle import loops
    row_ptr, col = (np.asarray(a, dtype=np.int64) for a in host_graph)
    N, E = len(row_ptr) - 1, len(col)
    out_ir = oirreps.per_path_out_irreps(spec.in_irreps, spec.lmax_sh, spec.lmax_out)
    prob = oirreps.build_problem(spec.in_irreps, oirreps.sh_irreps(spec.lmax_sh), out_ir, "uvu")
    tab = loops.Tables(prob)
    threads = loops.default_threads()
    rng = np.random.default_rng(seed + 98)
    target = max(2_000, E // 20)
    start = int(rng.integers(0, max(1, N // 2)))
    stop = min(max(int(np.searchsorted(row_ptr, row_ptr[start] + target)), start + 1), N)
    e0, e1 = int(row_ptr[start]), int(row_ptr[stop])
    n_e = e1 - e0
    sub_ptr = row_ptr[start:stop + 1] - e0
    uniq, inv = np.unique(col[e0:e1], return_inverse=True)
    x, ggx = rng.standard_normal((2, len(uniq), prob.d_in))
    y, ggy = rng.standard_normal((2, n_e, prob.d_sh))
    w, ggw = rng.standard_normal((2, n_e, prob.weight_numel))
    g = rng.standard_normal((stop - start, prob.d_out))
    rows, senders = np.arange(stop - start), np.arange(len(uniq))
    t0 = time.perf_counter()
    reps = 0
    while True:
        loops.conv_double_backward_rows(tab, sub_ptr, inv, x, y, w, g, ggx, ggy, ggw, rows, senders, threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= 10.0 or el >= max_seconds:
            break
    return {"value": n_e * reps / el, "unit": "edges/s", "cores": threads, "kind": "oracle",
            "sample": f"receivers [{start},{stop}) = {n_e} of {E} edges and their {len(uniq)} senders: all four "
                      f"double-backward results of that sub-graph; fp64 explicit loops, mean of {reps} rep(s)"}


def bench_double_backward(a, spec, plan, d, host_graph, device):
    import torch
    from clebsch_gordan_tensor_cgtp_amd import binding as cg
    from clebsch_gordan_tensor_cgtp_amd import synth
    N, E = d["row_ptr"].shape[0] - 1, d["col"].shape[0]
    es = 4 if a.dtype == "f32" else 8
    npdt = np.float32 if a.dtype == "f32" else np.float64
    up = synth.upstream_streams(a.seed)

    def dev(t):
        return torch.from_numpy(np.ascontiguousarray(t)).to(device) if isinstance(t, np.ndarray) else t

    gg = [dev(synth.normal(up["gg_x"], (N, plan.d_x), dtype=npdt, device=device)),
          dev(synth.normal(up["gg_y"], (E, plan.d_sh), dtype=npdt, device=device)),
          dev(synth.normal(up["gg_w"], (E, plan.weight_numel), dtype=npdt, device=device))]
    y = cg.spherical_harmonics(spec.lmax_sh, d["vec"])
    tr = cg.graph_transpose(d["row_ptr"], d["col"])
    order = cg.graph_order(d["row_ptr"]) if not a.natural_order else None
    outs = (torch.empty_like(d["x"]), torch.empty_like(y), torch.empty_like(d["w"]),
            torch.empty((N, plan.d_out), dtype=plan.torch_dtype, device=device))

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        cg.conv_double_backward(plan, d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"], *gg, order=order,
                                outs=outs, need=(False, False, False, True))
        if ev is not None:
            ev[1].record()
        cg.conv_double_backward(plan, d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"], *gg, order=order,
                                outs=outs, need=(True, True, True, False))
        if ev is not None:
            ev[2].record()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    t0 = time.perf_counter()
    for k in range(a.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    recv_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    send_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms_per_step = wall * 1e3 / a.steps
    recv_b, send_b = algorithmic_bytes_dbl(plan, N, E, es)
    recv_k = split_kernel("cgtp_conv_dbwd_recv", plan.row_split(N, E, double_backward=True))
    dom = ("cgtp_conv_dbwd_send", send_ms, send_b) if send_ms >= recv_ms else (recv_k, recv_ms, recv_b)
    oth = (recv_k, recv_ms, recv_b) if dom[0] == "cgtp_conv_dbwd_send" else ("cgtp_conv_dbwd_send", send_ms, send_b)
    achieved = dom[2] / (dom[1] * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": E / (ms_per_step * 1e-3), "unit": "edges/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": a.dtype, "data": "synthetic",
        "config": {"workload": spec.name, "N": N, "E": E, "in_irreps": spec.in_irreps, "sh_lmax": spec.lmax_sh,
                   "paths": plan.num_paths, "d_out": plan.d_out,
                   "step": "conv_double_backward (grad_x, grad_y, grad_w, grad_grad_out)",
                   "receiver_schedule": "natural" if a.natural_order else "heavy-first",
                   "recv_ms": recv_ms, "send_ms": send_ms},
        "roofline": {"bound": "hbm", "kernel": dom[0], "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(plan, spec, a.dtype, dom[0]),
                     "algorithmic_bytes_per_launch": dom[2], "avg_launch_ms": dom[1],
                     "other": {"kernel": oth[0], "achieved": oth[2] / (oth[1] * 1e-3) / 1e9}},
        "cpu_baseline": None,
    }
    if not a.no_cpu:
        line["cpu_baseline"] = cpu_baseline_dbl(spec, a.seed, host_graph)
    print(json.dumps(line), flush=True)


def uvw_conv_flops(plan, N, E):
    """Fixed counting convention for the uvw convolution: per edge the sparse contraction
    sum_p mul_in * 2 * nnz_p (VALU), per receiver the mixing sum_p 2 * mul_in * mul_out * (2l3+1)
    (MFMA)."""
    sparse = dense = 0
    for p in range(plan.num_paths):
        info = plan.path(p)
        sparse += info["mul_in"] * 2 * info["nnz"]
        dense += 2 * info["mul_in"] * info["mul_out"] * (2 * info["l3"] + 1)
    return E * sparse, N * dense


def cpu_baseline_uvw_conv(plan_prob, spec, seed, host_graph, max_seconds=30.0, backward=False):
    """The oracle's explicit uvw loops on every edge of a contiguous receiver slice (~5% of the
    edges), summed per receiver; with ``backward`` also the explicit uvw backward loops on the
    slice's edges as rows (dx and dY per edge, dW over the slice).  Random values (timing only).
    Rate = slice edges per second."""
    from oracle import irreps as oirreps
    from oracle import loops
    row_ptr, col = (np.asarray(a, dtype=np.int64) for a in host_graph)
    N, E = len(row_ptr) - 1, len(col)
    prob = oirreps.build_problem(spec.in_irreps, oirreps.sh_irreps(spec.lmax_sh), spec.out_irreps, "uvw")
    tab = loops.Tables(prob)
    threads = loops.default_threads()
    rng = np.random.default_rng(seed + 97)
    target = max(2_000, E // 20)
    start = int(rng.integers(0, max(1, N // 2)))
    stop = min(max(int(np.searchsorted(row_ptr, row_ptr[start] + target)), start + 1), N)
    x = rng.standard_normal((N, prob.d_in))
    y = rng.standard_normal((E, prob.d_sh))
    w = rng.standard_normal(prob.weight_numel)
    rows = np.arange(start, stop)
    n_e = int(row_ptr[stop] - row_ptr[start])
    edges = np.arange(row_ptr[start], row_ptr[stop])
    dst = np.repeat(np.arange(N), np.diff(row_ptr))
    g = rng.standard_normal((N, prob.d_out))
    t0 = time.perf_counter()
    reps = 0
    while True:
        loops.conv_forward_uvw_rows(tab, row_ptr, col, x, y, w, rows, threads)
        if backward:
            xe, ye, ge = x[col[edges]], y[edges], g[dst[edges]]
            loops.uvw_backward(tab, xe, ye, w, ge, np.arange(n_e), np.arange(n_e), threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= 10.0 or el >= max_seconds:
            break
    what = "uvw convolution output and backward (dx, dY, dW) of the slice's edges" if backward else \
        "uvw convolution output of that slice"
    return {"value": n_e * reps / el, "unit": "edges/s", "cores": threads, "kind": "oracle",
            "sample": f"receivers [{start},{stop}) = {n_e} of {E} edges: {what}; "
                      f"fp64 explicit loops, mean of {reps} rep(s)"}


def bench_conv_uvw(a, spec, plan, d, host_graph, device):
    """uvw convolution: one step = conv_forward (with --backward: + the backward's dx/dY pass,
    G = W^T g and the unit-weight sender pass, and its dW pass, per-tile partials and their
    reduction; both through cgtp_conv_backward_ws with a preallocated workspace)."""
    import torch
    from clebsch_gordan_tensor_cgtp_amd import binding as cg
    N, E = d["row_ptr"].shape[0] - 1, d["col"].shape[0]
    es = 4 if a.dtype == "f32" else 8
    y = cg.spherical_harmonics(spec.lmax_sh, d["vec"])
    order = cg.graph_order(d["row_ptr"]) if not a.natural_order else None
    out = torch.empty((N, plan.d_out), dtype=plan.torch_dtype, device=device)
    backward = a.backward
    if a.double_backward:
        return bench_conv_uvw_double_backward(a, spec, plan, d, y, order, device)
    if backward:
        plan.conv_uvw_backward_source(0)  # JIT outside the timed region
        tr = cg.graph_transpose(d["row_ptr"], d["col"])
        ws = torch.empty(cg.conv_backward_workspace_size(plan, N, E), dtype=torch.uint8, device=device)
        gx, gy, gw = torch.empty_like(d["x"]), torch.empty_like(y), torch.empty_like(d["w"])

    def step(ev):
        ev[0].record()
        cg.conv_forward(plan, d["row_ptr"], d["col"], d["x"], y, d["w"], out=out, order=order)
        ev[1].record()
        if backward:
            cg.conv_backward(plan, d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"], gx, gy, gw,
                             need=(True, True, False), order=order, workspace=ws)
            ev[2].record()
            cg.conv_backward(plan, d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"], gx, gy, gw,
                             need=(False, False, True), order=order, workspace=ws)
            ev[3].record()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(max(a.steps, a.warmup))]
    for k in range(a.warmup):
        step(evs[k])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(a.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    evs = evs[:a.steps]
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    sparse, dense = uvw_conv_flops(plan, N, E)
    # fixed counting convention of the backward: dx/dY pass = G (dense) + dx and dY contractions
    # (2 x sparse); dW pass = T again (sparse) + the dW contraction (dense)
    phases = [("cgtp_conv_uvw", ms, sparse + dense)]
    config = {"workload": spec.name, "N": N, "E": E, "in_irreps": spec.in_irreps, "out_irreps": spec.out_irreps,
              "sh_lmax": spec.lmax_sh, "paths": plan.num_paths, "d_out": plan.d_out,
              "step": "conv_forward (uvw: shared weights, MFMA mixing per 16-receiver tile)",
              "receiver_schedule": "natural" if a.natural_order else "heavy-first", "fwd_ms": ms}
    if backward:
        xy_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        w_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
        phases += [("dx/dY pass (cgtp_conv_uvw_bwd_g + cgtp_conv_uvw_bwd_xy)", xy_ms, dense + 2 * sparse),
                   ("dW pass (cgtp_conv_uvw_bwd_w + cgtp_reduce_chunks)", w_ms, sparse + dense)]
        config.update({"step": "conv_forward + conv_backward_ws (grad_x, grad_y, grad_w; uvw)",
                       "bwd_xy_ms": xy_ms, "bwd_w_ms": w_ms, "bwd_ms": xy_ms + w_ms,
                       "workspace_bytes": int(ws.numel())})
    dom = max(phases, key=lambda p: p[1])
    tflops = dom[2] / (dom[1] * 1e-3) / 1e12
    peak = 157.3 if a.dtype == "f32" else 78.6
    roof = {"bound": "alu", "kernel": dom[0], "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
            "frac": tflops / peak, "traffic": None, "flops_per_launch": dom[2], "avg_launch_ms": dom[1]}
    if dom[0] == "cgtp_conv_uvw":
        roof.update({"traffic": measured_traffic(plan, spec, a.dtype, "cgtp_conv_uvw"),
                     "flops_per_launch": {"sparse_valu": sparse, "mixing_mfma": dense},
                     "hbm_algorithmic_bytes_per_launch": (N + 1) * 4 + E * 4 + es * (
                         N * plan.d_x + E * plan.d_sh + plan.weight_numel + N * plan.d_out)})
    if backward:
        roof["phases"] = [{"kernel": p[0], "avg_ms": p[1], "flops": p[2],
                           "tflops": p[2] / (p[1] * 1e-3) / 1e12} for p in phases]
    line = {
        "metric": METRIC, "value": E / (wall / a.steps), "unit": "edges/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": wall * 1e3 / a.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": a.dtype, "data": "synthetic", "config": config, "roofline": roof,
        "cpu_baseline": None,
    }
    if not a.no_cpu:
        line["cpu_baseline"] = cpu_baseline_uvw_conv(None, spec, a.seed, host_graph, backward=backward)
    print(json.dumps(line), flush=True)


def bench_conv_uvw_double_backward(a, spec, plan, d, y, order, device):
    """uvw convolution double backward: one step = cgtp_conv_double_backward_ws with all four results
    (G and G' on MFMA, the unit-weight sender pass twice, the dW pass twice and its reduction, the
    forward three times), workspace preallocated."""
    import torch
    from clebsch_gordan_tensor_cgtp_amd import binding as cg
    from clebsch_gordan_tensor_cgtp_amd import synth
    N, E = d["row_ptr"].shape[0] - 1, d["col"].shape[0]
    npdt = np.float32 if a.dtype == "f32" else np.float64
    up = synth.upstream_streams(a.seed)
    dev = lambda t: torch.from_numpy(np.ascontiguousarray(t)).to(device)
    gg = (dev(synth.normal(up["gg_x"], (N, plan.d_x), dtype=npdt)),
          dev(synth.normal(up["gg_y"], (E, plan.d_sh), dtype=npdt)),
          dev(synth.normal(up["gg_w"], (plan.weight_numel,), 1.0 / np.sqrt(32.0), dtype=npdt)))
    plan.conv_uvw_backward_source(0)  # JIT outside the timed region
    tr = cg.graph_transpose(d["row_ptr"], d["col"])
    ws = torch.empty(cg.conv_double_backward_workspace_size(plan, N, E), dtype=torch.uint8, device=device)
    outs = (torch.empty_like(d["x"]), torch.empty_like(y), torch.empty_like(d["w"]),
            torch.empty((N, plan.d_out), dtype=plan.torch_dtype, device=device))

    def step():
        cg.conv_double_backward(plan, d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"], *gg, order=order,
                                outs=outs, workspace=ws)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(a.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / a.steps
    ms = e0.elapsed_time(e1) / a.steps
    sparse, dense = uvw_conv_flops(plan, N, E)
    # fixed counting convention: d/dg = three forwards; d/dx, d/dy = G and G' (dense) + two
    # sender passes (2 x sparse each); d/dW = two dW passes (sparse + dense each)
    flops = 3 * (sparse + dense) + 2 * (dense + 2 * sparse) + 2 * (sparse + dense)
    peak = 157.3 if a.dtype == "f32" else 78.6
    tflops = flops / (ms * 1e-3) / 1e12
    line = {
        "metric": METRIC, "value": E / wall, "unit": "edges/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": wall * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": a.dtype, "data": "synthetic",
        "config": {"workload": spec.name, "N": N, "E": E, "in_irreps": spec.in_irreps, "out_irreps": spec.out_irreps,
                   "sh_lmax": spec.lmax_sh, "paths": plan.num_paths,
                   "step": "conv_double_backward_ws (uvw: grad_x, grad_y, grad_w, grad_grad_out)",
                   "receiver_schedule": "natural" if a.natural_order else "heavy-first", "dbl_ms": ms,
                   "workspace_bytes": int(ws.numel())},
        "roofline": {"bound": "alu", "kernel": "cgtp_conv_double_backward_ws (uvw, all launches of one call)",
                     "achieved": tflops, "peak": peak, "unit": "TFLOP/s", "frac": tflops / peak, "traffic": None,
                     "flops_per_launch": flops, "avg_launch_ms": ms},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_radial(spec, seed, host_graph, R, max_seconds=30.0, backward=False):
    """The oracle (W = rho @ Theta for the slice's edges, then the explicit uvu loops) on a
    contiguous receiver slice with ~5% of the edges (with ``backward`` also dx, dY, drho and dTheta
    of that sub-graph); random values.  Rate = slice edges/s."""
    from oracle import irreps as oirreps
    from oracle import loops
    row_ptr, col = (np.asarray(a, dtype=np.int64) for a in host_graph)
    N, E = len(row_ptr) - 1, len(col)
    out_ir = oirreps.per_path_out_irreps(spec.in_irreps, spec.lmax_sh, spec.lmax_out)
    prob = oirreps.build_problem(spec.in_irreps, oirreps.sh_irreps(spec.lmax_sh), out_ir, "uvu")
    tab = loops.Tables(prob)
    threads = loops.default_threads()
    rng = np.random.default_rng(seed + 95)
    target = max(2_000, E // 20)
    start = int(rng.integers(0, max(1, N // 2)))
    stop = min(max(int(np.searchsorted(row_ptr, row_ptr[start] + target)), start + 1), N)
    e0, e1 = int(row_ptr[start]), int(row_ptr[stop])
    sub_ptr = row_ptr[start:stop + 1] - e0
    uniq, inv = np.unique(col[e0:e1], return_inverse=True)
    x = rng.standard_normal((len(uniq), prob.d_in))
    y = rng.standard_normal((e1 - e0, prob.d_sh))
    rho = rng.standard_normal((e1 - e0, R))
    theta = rng.standard_normal((R, prob.weight_numel))
    rows = np.arange(stop - start)
    g = rng.standard_normal((stop - start, prob.d_out))
    t0 = time.perf_counter()
    reps = 0
    while True:
        loops.conv_forward_radial_rows(tab, sub_ptr, inv, x, y, rho, theta, rows, threads)
        if backward:
            loops.conv_backward_radial_rows(tab, sub_ptr, inv, x, y, rho, theta, g, rows, np.arange(len(uniq)), threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= 10.0 or el >= max_seconds:
            break
    what = "forward and backward (dx, dY, drho, dTheta)" if backward else "forward"
    return {"value": (e1 - e0) * reps / el, "unit": "edges/s", "cores": threads, "kind": "oracle",
            "sample": f"receivers [{start},{stop}) = {e1 - e0} of {E} edges, R = {R}: W = rho @ Theta for those "
                      f"edges, then the fp64 explicit loops, {what}; mean of {reps} rep(s)"}


def radial_flops(plan, E, R):
    """Counting convention of the radial passes: per edge the uvu contraction
    sum_p mul (2 nnz_p + 2 (2l3+1)) plus 2R flops per weight to rebuild W_e (forward); the
    backward counts 3x the contraction plus 3 x 2R per weight (W_e rebuilt, drho, dTheta)."""
    contr = 0
    for p in range(plan.num_paths):
        info = plan.path(p)
        contr += info["mul_in"] * (2 * info["nnz"] + 2 * (2 * info["l3"] + 1))
    radial = 2 * R * plan.weight_numel
    return E * (contr + radial), E * (3 * contr + 3 * radial)


def bench_radial(a, spec, plan, d, host_graph, device):
    import torch
    from clebsch_gordan_tensor_cgtp_amd import binding as cg
    from clebsch_gordan_tensor_cgtp_amd import synth
    R = a.radial
    N, E = d["row_ptr"].shape[0] - 1, d["col"].shape[0]
    es = 4 if a.dtype == "f32" else 8
    npdt = np.float32 if a.dtype == "f32" else np.float64
    up = synth.upstream_streams(a.seed)
    rho = synth.normal(up["gg_y"], (E, R), dtype=npdt, device=device)
    theta = synth.normal(up["gg_w"], (R, plan.weight_numel), 1.0 / np.sqrt(R * E / N), dtype=npdt)
    rho = torch.from_numpy(rho).to(device) if isinstance(rho, np.ndarray) else rho
    theta = torch.from_numpy(theta).to(device)
    y = cg.spherical_harmonics(spec.lmax_sh, d["vec"])
    order = cg.graph_order(d["row_ptr"]) if not a.natural_order else None
    out = torch.empty((N, plan.d_out), dtype=plan.torch_dtype, device=device)
    plan.radial_source(R)  # JIT outside the timed region

    def timed(fn):
        for _ in range(a.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(a.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / a.steps, (time.perf_counter() - t0) / a.steps

    fwd = lambda: cg.conv_forward_radial(plan, d["row_ptr"], d["col"], d["x"], y, rho, theta, out=out, order=order)
    ms, wall = timed(fwd)
    ms_w, _ = timed(lambda: cg.conv_forward(plan, d["row_ptr"], d["col"], d["x"], y, d["w"], out=out, order=order))
    alg = (N + 1) * 4 + E * 4 + es * (N * plan.d_x + E * plan.d_sh + E * R + R * plan.weight_numel + N * plan.d_out)
    config = {"workload": spec.name, "N": N, "E": E, "in_irreps": spec.in_irreps, "sh_lmax": spec.lmax_sh,
              "paths": plan.num_paths, "d_out": plan.d_out, "radial_features": R,
              "step": "conv_forward_radial (W_e = rho_e Theta rebuilt in registers, never stored)",
              "receiver_schedule": "natural" if a.natural_order else "heavy-first", "fwd_ms": ms,
              "materialised_weights_fwd_ms": ms_w}
    dom = ("cgtp_conv_fwd_radial", ms, alg)
    if a.backward:
        tr = cg.graph_transpose(d["row_ptr"], d["col"])
        ws = torch.empty(cg.conv_backward_radial_workspace_size(plan, N, E, R), dtype=torch.uint8, device=device)
        outs = (torch.empty_like(d["x"]), torch.empty_like(y), torch.empty_like(rho), torch.empty_like(theta))
        bwd = lambda: cg.conv_backward_radial(plan, d["row_ptr"], d["col"], tr, d["x"], y, rho, theta, d["g"],
                                              outs=outs, workspace=ws)
        bms, _ = timed(bwd)

        def step():
            fwd()
            bwd()
        _, wall = timed(step)
        gw = (torch.empty_like(d["x"]), torch.empty_like(y), torch.empty_like(d["w"]))
        bms_w, _ = timed(lambda: cg.conv_backward(plan, d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"], *gw))
        # reads x, Y, rho, Theta, g and the transpose once; writes dx, dY, drho once (the dTheta
        # partials are chunk-sized, not edge-sized)
        alg_b = (N + 1) * 4 + 2 * E * 4 + es * (2 * N * plan.d_x + 2 * E * plan.d_sh + 2 * E * R
                                               + 2 * R * plan.weight_numel + N * plan.d_out)
        config.update({"step": "conv_forward_radial + conv_backward_radial (dx, dY, drho, dTheta; W_e and dW_e "
                               "never stored)", "bwd_ms": bms, "materialised_weights_bwd_ms": bms_w,
                       "bwd_launches": plan.radial_source(R).count("void rbw_g")})
        if bms >= ms:
            dom = ("cgtp_conv_bwd_radial", bms, alg_b)
    # Rebuilding W (and consuming dW) costs R FMAs per weight and edge, against 4 or 8 bytes of W
    # saved: the radial passes are bound by VALU issue, not by HBM.  Fixed counting convention:
    # forward = the uvu contraction + 2R per weight; backward = 3x the contraction + 3 x 2R per
    # weight (W rebuilt, drho, dTheta).
    f_fwd, f_bwd = radial_flops(plan, E, R)
    flops = f_bwd if dom[0] == "cgtp_conv_bwd_radial" else f_fwd
    tflops = flops / (dom[1] * 1e-3) / 1e12
    peak = 157.3 if a.dtype == "f32" else 78.6
    line = {
        "metric": METRIC, "value": E / wall, "unit": "edges/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": wall * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": a.dtype, "data": "synthetic", "config": config,
        "roofline": {"bound": "alu", "kernel": dom[0], "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": tflops / peak, "traffic": None, "flops_per_launch": flops, "avg_launch_ms": dom[1],
                     "hbm_algorithmic_bytes_per_launch": dom[2],
                     "hbm_achieved_gbs": dom[2] / (dom[1] * 1e-3) / 1e9},
        "cpu_baseline": None,
    }
    if not a.no_cpu:
        line["cpu_baseline"] = cpu_baseline_radial(spec, a.seed, host_graph, R, backward=a.backward)
    print(json.dumps(line), flush=True)


def cpu_baseline_radial_uvw(spec, seed, host_graph, R, max_seconds=30.0, backward=False):
    """The oracle (oracle.ref: W_e = rho_e Theta formed per edge, then each edge's fully connected
    product, summed per receiver; with ``backward`` also dx, dY, drho and dTheta) on a contiguous
    receiver slice of about 2,000 edges (the formed W_e take E x weight_numel values); random
    values.  Rate = slice edges/s."""
    from oracle import irreps as oirreps
    from oracle import ref
    row_ptr, col = (np.asarray(a, dtype=np.int64) for a in host_graph)
    N, E = len(row_ptr) - 1, len(col)
    prob = oirreps.build_problem(spec.in_irreps, oirreps.sh_irreps(spec.lmax_sh), spec.out_irreps, "uvw")
    rng = np.random.default_rng(seed + 96)
    start = int(rng.integers(0, max(1, N // 2)))
    stop = min(max(int(np.searchsorted(row_ptr, row_ptr[start] + 2_000)), start + 1), N)
    e0, e1 = int(row_ptr[start]), int(row_ptr[stop])
    sub_ptr = row_ptr[start:stop + 1] - e0
    uniq, inv = np.unique(col[e0:e1], return_inverse=True)
    x = rng.standard_normal((len(uniq), prob.d_in))
    y = rng.standard_normal((e1 - e0, prob.d_sh))
    rho = rng.standard_normal((e1 - e0, R))
    theta = rng.standard_normal((R, prob.weight_numel))
    g = rng.standard_normal((stop - start, prob.d_out))
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):  # numpy's BLAS on one thread, so that `cores` is what ran
        t0 = time.perf_counter()
        reps = 0
        while True:
            ref.conv_forward_radial(prob, sub_ptr, inv, x, y, rho, theta)
            if backward:
                ref.conv_backward_radial(prob, sub_ptr, inv, x, y, rho, theta, g)
            reps += 1
            el = time.perf_counter() - t0
            if el >= 10.0 or el >= max_seconds:
                break
    what = "forward and backward (dx, dY, drho, dTheta)" if backward else "forward"
    return {"value": (e1 - e0) * reps / el, "unit": "edges/s", "cores": 1, "kind": "oracle",
            "sample": f"receivers [{start},{stop}) = {e1 - e0} of {E} edges, R = {R}: W_e = rho_e Theta formed "
                      f"for those edges, then the fp64 numpy definition, {what}; mean of {reps} rep(s)"}


def bench_radial_uvw(a, spec, plan, d, host_graph, device):
    """uvw convolution with per-edge weights W_e = rho_e Theta: one step = conv_forward_radial (with
    --backward: + conv_backward_radial for dx, dY, drho, dTheta).  Each radial channel r runs the
    shared-weight uvw kernels on rho[:, r] * Y with Theta's row r; W_e is never formed."""
    import torch
    from clebsch_gordan_tensor_cgtp_amd import binding as cg
    from clebsch_gordan_tensor_cgtp_amd import synth
    R = a.radial
    N, E = d["row_ptr"].shape[0] - 1, d["col"].shape[0]
    npdt = np.float32 if a.dtype == "f32" else np.float64
    up = synth.upstream_streams(a.seed)
    rho = torch.from_numpy(synth.normal(up["gg_y"], (E, R), dtype=npdt)).to(device)
    theta = torch.from_numpy(synth.normal(up["gg_w"], (R, plan.weight_numel), 1.0 / np.sqrt(R * E / N),
                                          dtype=npdt)).to(device)
    y = cg.spherical_harmonics(spec.lmax_sh, d["vec"])
    order = cg.graph_order(d["row_ptr"]) if not a.natural_order else None
    out = torch.empty((N, plan.d_out), dtype=plan.torch_dtype, device=device)
    plan.radial_source(R)  # JIT outside the timed region
    tr = cg.graph_transpose(d["row_ptr"], d["col"])
    ws = torch.empty(max(1, cg.conv_backward_radial_workspace_size(plan, N, E, R)), dtype=torch.uint8, device=device)
    outs = (torch.empty_like(d["x"]), torch.empty_like(y), torch.empty_like(rho), torch.empty_like(theta))
    fwd = lambda: cg.conv_forward_radial(plan, d["row_ptr"], d["col"], d["x"], y, rho, theta, out=out, order=order)
    bwd = lambda: cg.conv_backward_radial(plan, d["row_ptr"], d["col"], tr, d["x"], y, rho, theta, d["g"],
                                          outs=outs, workspace=ws)

    def step(ev):
        ev[0].record()
        fwd()
        ev[1].record()
        if a.backward:
            bwd()
        ev[2].record()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(max(a.steps, a.warmup))]
    for k in range(a.warmup):
        step(evs[k])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(a.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / a.steps
    evs = evs[:a.steps]
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    sparse, dense = uvw_conv_flops(plan, N, E)
    # counting convention: R times the shared-weight uvw passes (forward sparse + dense; backward
    # dx/dY (dense + 2 sparse) and dTheta (sparse + dense)); the SH scaling and the fold are E d_sh
    # multiplies per channel, not counted
    phases = [("conv_forward_radial (R x cgtp_conv_uvw_rad)", ms, R * (sparse + dense))]
    config = {"workload": spec.name, "N": N, "E": E, "in_irreps": spec.in_irreps, "out_irreps": spec.out_irreps,
              "sh_lmax": spec.lmax_sh, "paths": plan.num_paths, "d_out": plan.d_out, "radial_features": R,
              "step": "conv_forward_radial (uvw; W_e = rho_e Theta never formed)",
              "receiver_schedule": "natural" if a.natural_order else "heavy-first", "fwd_ms": ms,
              "formed_weights_bytes_avoided": E * plan.weight_numel * (4 if a.dtype == "f32" else 8)}
    if a.backward:
        bms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        phases.append(("conv_backward_radial (per channel: scale, G, sender pass, fold, dW pass)", bms,
                       R * (3 * sparse + 2 * dense)))
        config.update({"step": "conv_forward_radial + conv_backward_radial (uvw; dx, dY, drho, dTheta)",
                       "bwd_ms": bms, "workspace_bytes": int(ws.numel())})
    dom = max(phases, key=lambda p: p[1])
    tflops = dom[2] / (dom[1] * 1e-3) / 1e12
    peak = 157.3 if a.dtype == "f32" else 78.6
    line = {
        "metric": METRIC, "value": E / wall, "unit": "edges/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": wall * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": a.dtype, "data": "synthetic", "config": config,
        "roofline": {"bound": "alu", "kernel": dom[0], "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": tflops / peak, "traffic": None, "flops_per_launch": dom[2], "avg_launch_ms": dom[1],
                     "phases": [{"kernel": p[0], "avg_ms": p[1], "flops": p[2]} for p in phases]},
        "cpu_baseline": None,
    }
    if not a.no_cpu:
        line["cpu_baseline"] = cpu_baseline_radial_uvw(spec, a.seed, host_graph, R, backward=a.backward)
    print(json.dumps(line), flush=True)


def spread(evs):
    """Median, min and max over the timed steps of the forward and backward launch times."""
    f = [e[0].elapsed_time(e[1]) for e in evs]
    b = [e[1].elapsed_time(e[2]) for e in evs]
    return {"fwd": [float(np.median(f)), float(np.min(f)), float(np.max(f))],
            "bwd": [float(np.median(b)), float(np.min(b)), float(np.max(b))], "order": "median, min, max"}


def cold_cache_times(a, step, device):
    """The same steps, each after writing a 1 GiB buffer (more than the 4 MB L2 of every XCD and
    the 256 MB last-level cache) outside its timed region: the forward and backward launch times
    with nothing of the step's inputs left in the caches.  Reported beside the warm figures; the
    headline value is the warm K-step wall time."""
    import torch
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=device)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    for k in range(a.steps):
        scratch.fill_(float(k))
        step(evs[k])
    torch.cuda.synchronize()
    del scratch
    return {"fwd_ms": float(np.median([e[0].elapsed_time(e[1]) for e in evs])),
            "bwd_ms": float(np.median([e[1].elapsed_time(e[2]) for e in evs])),
            "flush": "1 GiB fill before each step, outside its events", "statistic": "median"}


def split_kernel(base, split):
    """Name of the receiver-owned kernel that gives each receiver row `split` waves."""
    return base if split == 1 else f"{base}_split{split}"


def kernel_digest(source, kernel):
    """SHA-1 of the generated code one kernel runs: the module's shared preamble plus that
    kernel's own section (the generator marks sections with '// @@section NAME' lines); a
    `_splitN` entry point also runs the code of its base kernel's section."""
    import hashlib
    import re
    parts, name = {}, None
    for line in source.splitlines(keepends=True):
        if line.startswith("// @@section "):
            name = line[len("// @@section "):].strip()
        parts[name] = parts.get(name, "") + line
    if "common" not in parts or kernel not in parts:
        return None
    m = re.fullmatch(r"(.+)_split\d+", kernel)
    base = parts.get(m.group(1), "") if m else ""
    return hashlib.sha1((parts["common"] + base + parts[kernel]).encode()).hexdigest()


def measured_traffic(plan, spec, dtype, kernel):
    """HBM-side bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE record, scaled
    by the copy-kernel calibration; None unless the record was taken on exactly this kernel's code.
    A tuple of kernels (one call made of several kernels) gives the sum, or None if any is missing."""
    import glob
    if isinstance(kernel, tuple):
        parts = [measured_traffic(plan, spec, dtype, k) for k in kernel]
        return None if any(p is None for p in parts) else sum(parts)
    digest = kernel_digest(plan.source, kernel)
    for path in glob.glob(os.path.join(ROOT, "profiles", "*_hbm_counters.json")):
        rec = json.load(open(path))
        k = rec.get("kernels", {}).get(kernel)
        if digest is None or k is None or k.get("code_sha1") != digest or rec.get("dtype") != dtype:
            continue
        cal = rec["calibration"]
        kib = (k["FETCH_SIZE_kib_per_dispatch"] * cal["fetch_factor"]
               + k["WRITE_SIZE_kib_per_dispatch"] * cal["write_factor"]) * k["dispatches_per_call"]
        return kib * 1024
    return None


def make_inputs(spec, dtype, seed, device):
    import torch
    from clebsch_gordan_tensor_cgtp_amd import binding as cg
    from clebsch_gordan_tensor_cgtp_amd import synth
    st = synth.streams(seed)
    row_ptr, col = synth.conv_graph(spec, seed)
    N, E = len(row_ptr) - 1, len(col)
    plan = cg.plan_for(spec, dtype)
    npdt = np.float32 if dtype == "f32" else np.float64
    fan_in = E / N

    def dev(a):
        if isinstance(a, np.ndarray):
            return torch.from_numpy(a).to(device)
        return a

    d = {
        "row_ptr": dev(row_ptr), "col": dev(col),
        "x": dev(synth.normal(st["x"], (N, plan.d_x), dtype=npdt, device=device)),
        "vec": dev(synth.normal(st["vec"], (E, 3), dtype=npdt, device=device)),
        "w": dev(synth.normal(st["w"], (E, plan.weight_numel), 1.0 / np.sqrt(fan_in), dtype=npdt, device=device))
        if spec.mode == "uvu" else dev(synth.normal(st["w"], (plan.weight_numel,), 1.0 / np.sqrt(32.0), dtype=npdt)),
        "g": dev(synth.normal(st["sample"], (N, plan.d_out), dtype=npdt, device=device)),
    }
    return plan, d, (row_ptr, col)


def cpu_baseline(spec, seed, host_graph, max_seconds=30.0):
    """The oracle's explicit loops (fp64, OpenMP) on the host cores, on a bounded sample of
    the same graph: forward and edge gradients of a contiguous receiver slice holding ~5% of
    the edges, and grad_x of a contiguous sender range with about as many edges.  Values are
    random (timing only); the rate is edges of the slice per second of the three passes."""
    from oracle import irreps as oirreps
    from oracle import loops
    row_ptr, col = (np.asarray(a, dtype=np.int64) for a in host_graph)
    N, E = len(row_ptr) - 1, len(col)
    out_ir = oirreps.per_path_out_irreps(spec.in_irreps, spec.lmax_sh, spec.lmax_out)
    prob = oirreps.build_problem(spec.in_irreps, oirreps.sh_irreps(spec.lmax_sh), out_ir, "uvu")
    tab = loops.Tables(prob)
    threads = loops.default_threads()
    rng = np.random.default_rng(seed + 99)
    target = max(2_000, E // 20)
    start = int(rng.integers(0, max(1, N // 2)))
    stop = min(max(int(np.searchsorted(row_ptr, row_ptr[start] + target)), start + 1), N)
    e0, e1 = int(row_ptr[start]), int(row_ptr[stop])
    n_e = e1 - e0
    sub_ptr = row_ptr[start:stop + 1] - e0
    uniq, inv = np.unique(col[e0:e1], return_inverse=True)
    x_c = rng.standard_normal((len(uniq), prob.d_in))
    y_s = rng.standard_normal((n_e, prob.d_sh))
    w_s = rng.standard_normal((n_e, prob.weight_numel))
    g_s = rng.standard_normal((stop - start, prob.d_out))
    # senders [s0, s1) with about n_e outgoing edges, and their edges in sender order
    order = np.argsort(col, kind="stable")
    t_ptr = np.concatenate([[0], np.cumsum(np.bincount(col, minlength=N))])
    s0 = int(rng.integers(0, max(1, N // 2)))
    s1 = min(max(int(np.searchsorted(t_ptr, t_ptr[s0] + n_e)), s0 + 1), N)
    t_edges = order[t_ptr[s0]:t_ptr[s1]]
    dst = np.searchsorted(row_ptr, t_edges, side="right") - 1
    guniq, ginv = np.unique(dst, return_inverse=True)
    sptr = t_ptr[s0:s1 + 1] - t_ptr[s0]
    g_c = rng.standard_normal((len(guniq), prob.d_out))
    y_t = rng.standard_normal((len(t_edges), prob.d_sh))
    w_t = rng.standard_normal((len(t_edges), prob.weight_numel))
    t0 = time.perf_counter()
    reps = 0
    while True:
        loops.uvu_forward(tab, sub_ptr, inv, x_c, y_s, w_s, threads)
        loops.uvu_backward_edges(tab, sub_ptr, inv, x_c, y_s, w_s, g_s, threads)
        loops.uvu_backward_x(tab, sptr, ginv, y_t, w_t, g_c, threads)
        reps += 1
        el = time.perf_counter() - t0
        if el > 10.0 or el * (reps + 1) / reps > max_seconds:
            break
    sec = (time.perf_counter() - t0) / reps
    return {"value": n_e / sec, "unit": "edges/s", "cores": threads, "kind": "oracle",
            "sample": f"receivers [{start},{stop}) = {n_e} of {E} edges: forward + grad_y/grad_w; "
                      f"grad_x of senders [{s0},{s1}) = {len(t_edges)} edges; fp64 explicit loops, "
                      f"mean of {reps} rep(s)"}


def tp_flops(plan_paths, mul, mode):
    """Counting convention: uvw per row sum_p [2 mul nnz_p + 2 mul_in mul_out (2l3+1)] (+ nnz_p);
    uvu per row sum_p [mul (2 nnz_p + 2 (2l3+1)) + nnz_p]."""
    f = 0
    for p in plan_paths:
        n3 = 2 * p["l3"] + 1
        if mode == "uvw":
            f += 2 * p["mul_in"] * p["nnz"] + 2 * p["mul_in"] * p["mul_out"] * n3 + p["nnz"]
        else:
            f += p["mul_in"] * (2 * p["nnz"] + 2 * n3) + p["nnz"]
    return f


def cpu_baseline_tp(spec, plan_paths, seed, max_seconds=30.0):
    """The oracle's explicit loops (fp64, OpenMP) on a bounded sample of rows of the same batch
    (random values, timing only): the forward, and with ``plan_paths == "backward"`` also the
    backward (uvu: per-row dY, dW and dx; uvw: dx, dY and the shared dW over the sample).
    Rate = rows per second."""
    from oracle import irreps as oirreps
    from oracle import loops
    out_ir = spec.out_irreps if spec.mode == "uvw" else oirreps.per_path_out_irreps(spec.in_irreps, spec.lmax_sh,
                                                                                     spec.lmax_sh)
    prob = oirreps.build_problem(spec.in_irreps, oirreps.sh_irreps(spec.lmax_sh), out_ir, spec.mode)
    tab = loops.Tables(prob)
    threads = loops.default_threads()
    rng = np.random.default_rng(seed + 96)
    n = max(1, min(spec.batch, 20_000 if spec.mode == "uvu" else 500))
    x = rng.standard_normal((n, prob.d_in))
    y = rng.standard_normal((n, prob.d_sh))
    w = rng.standard_normal(prob.weight_numel if spec.mode == "uvw" else (n, prob.weight_numel))
    g = rng.standard_normal((n, prob.d_out))
    ident = np.arange(n + 1)
    t0 = time.perf_counter()
    reps = 0
    while True:
        if spec.mode == "uvw":
            loops.uvw_forward(tab, x, y, w, threads)
            if plan_paths == "backward":
                loops.uvw_backward(tab, x, y, w, g, np.arange(n), np.arange(n), threads)
        else:
            loops.uvu_forward(tab, ident, np.arange(n), x, y, w, threads)
            if plan_paths == "backward":
                loops.uvu_backward_edges(tab, ident, np.arange(n), x, y, w, g, threads)
                loops.uvu_backward_x(tab, ident, np.arange(n), y, w, g, threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= 10.0 or el >= max_seconds:
            break
    what = f"{spec.mode} forward + backward" if plan_paths == "backward" else f"{spec.mode} forward"
    return {"value": n * reps / el, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {spec.batch} rows, {what}; fp64 explicit loops, mean of {reps} rep(s)"}


def bench_tp(a, spec, device):
    """Batched tensor product workloads: one step = one cgtp_tp_forward over the batch (with
    --backward: cgtp_tp_forward + cgtp_tp_backward)."""
    import torch
    from clebsch_gordan_tensor_cgtp_amd import binding as cg
    from clebsch_gordan_tensor_cgtp_amd import synth
    plan = cg.plan_for(spec, a.dtype)
    st = synth.streams(a.seed)
    npdt = np.float32 if a.dtype == "f32" else np.float64
    es = 4 if a.dtype == "f32" else 8
    B = spec.batch
    backward = a.backward
    x = torch.from_numpy(synth.normal(st["x"], (B, plan.d_x), dtype=npdt)).to(device)
    vec = torch.from_numpy(synth.normal(st["vec"], (B, 3), dtype=npdt)).to(device)
    wshape = (plan.weight_numel,) if spec.mode == "uvw" else (B, plan.weight_numel)
    w = torch.from_numpy(synth.normal(st["w"], wshape, 0.25, dtype=npdt)).to(device)
    g = torch.from_numpy(synth.normal(st["sample"], (B, plan.d_out), dtype=npdt)).to(device) if backward else None
    y = cg.spherical_harmonics(spec.lmax_sh, vec)
    out = torch.empty((B, plan.d_out), dtype=plan.torch_dtype, device=device)
    grads = (torch.empty_like(x), torch.empty_like(y), torch.empty_like(w)) if backward else None
    ws = None
    if backward and spec.mode == "uvw":
        # JIT outside the timed region: plans with a multiplicity above 16 run the uvw convolution
        # backward on the identity graph, the others the batched backward's own module
        if plan.wide_uvw:
            plan.conv_uvw_backward_source(0)
        else:
            plan.uvw_backward_source()
        ws = torch.empty(-(-cg.tp_backward_workspace_size(plan, B) // es), dtype=plan.torch_dtype, device=device)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        cg.tp_forward(plan, x, y, w, out=out)
        if ev is not None:
            ev[1].record()
        if backward:
            cg.tp_backward(plan, x, y, w, g, *grads, workspace=ws)
        if ev is not None:
            ev[2].record()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    t0 = time.perf_counter()
    for k in range(a.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) if backward else 0.0
    # the same steps captured once in a HIP graph and replayed (the library allocates and
    # synchronises nothing, so its launches can be captured): what a launch-bound caller gets
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(a.steps):
            step()
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    graph.replay()
    g1.record()
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / a.steps
    del graph
    paths = [plan.path(p) for p in range(plan.num_paths)]
    config = {"workload": spec.name, "B": B, "in_irreps": spec.in_irreps, "mode": spec.mode,
              "paths": plan.num_paths, "nnz": plan.nnz_total, "fwd_ms": fwd_ms,
              "step": "tp_forward + tp_backward" if backward else "tp_forward",
              "graph_replay_ms_per_step": graph_ms, "graph_rows_per_s": B / (graph_ms * 1e-3)}
    if spec.mode == "uvw":
        flops = tp_flops(paths, None, spec.mode) * B
        peak = 157.3 if a.dtype == "f32" else 78.6
        # fixed counting convention: the backward (dx, dY, dW) counts 3x the forward's flops
        dom = ("cgtp_tp_uvw_bwd", bwd_ms, 3 * flops) if backward and bwd_ms >= fwd_ms else ("cgtp_tp_uvw", fwd_ms, flops)
        achieved = dom[2] / (dom[1] * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom[0], "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": None, "flops_per_launch": dom[2], "avg_launch_ms": dom[1]}
        if backward:
            config["bwd_ms"] = bwd_ms
    else:
        # uvu is HBM-bound: every row reads x, y, W once and writes out once (backward: reads
        # x, y, W, grad_out, writes grad_x, grad_y, grad_w)
        fwd_b = B * es * (plan.d_x + plan.d_sh + plan.weight_numel + plan.d_out)
        bwd_b = B * es * (2 * plan.d_x + 2 * plan.d_sh + 2 * plan.weight_numel + plan.d_out)
        dom = ("cgtp_tp_bwd", bwd_ms, bwd_b) if backward and bwd_ms >= fwd_ms else ("cgtp_tp_fwd", fwd_ms, fwd_b)
        achieved = dom[2] / (dom[1] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom[0], "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(plan, spec, a.dtype, dom[0]),
                "algorithmic_bytes_per_launch": dom[2], "avg_launch_ms": dom[1]}
        if backward:
            config["bwd_ms"] = bwd_ms
    line = {"metric": "rows/sec batched CGTP forward and % of FP32 roofline", "value": B / (wall / a.steps),
            "unit": "rows/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
            "ms_per_step": wall * 1e3 / a.steps, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": a.dtype, "data": "synthetic", "config": config, "roofline": roof,
            "cpu_baseline": None}
    if not a.no_cpu:
        line["cpu_baseline"] = cpu_baseline_tp(spec, "backward" if backward else None, a.seed)
    print(json.dumps(line), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if a.copy_probe:
        copy_probe()
        return
    import torch
    from clebsch_gordan_tensor_cgtp_amd import binding as cg
    from clebsch_gordan_tensor_cgtp_amd import synth
    device = "cuda:0"
    torch.cuda.set_device(0)
    spec = {**synth.WORKLOADS, **synth.EXTRA_WORKLOADS}[a.workload]
    if not hasattr(spec, "n_edges"):
        return bench_tp(a, spec, device)
    if a.nodes or a.edges:
        if a.nodes <= 0 or a.edges < 0:
            print(json.dumps({"error": "--nodes needs a positive value and --edges a non-negative one"}))
            sys.exit(2)
        spec = synth.scaled(spec, a.nodes, a.edges)
    plan, d, host_graph = make_inputs(spec, a.dtype, a.seed, device)
    if spec.mode == "uvw":
        if a.radial:
            return bench_radial_uvw(a, spec, plan, d, host_graph, device)
        return bench_conv_uvw(a, spec, plan, d, host_graph, device)
    if a.radial:
        return bench_radial(a, spec, plan, d, host_graph, device)
    if a.double_backward:
        return bench_double_backward(a, spec, plan, d, host_graph, device)
    N, E = d["row_ptr"].shape[0] - 1, d["col"].shape[0]
    es = 4 if a.dtype == "f32" else 8
    y = cg.spherical_harmonics(spec.lmax_sh, d["vec"])
    tr = cg.graph_transpose(d["row_ptr"], d["col"])
    order = cg.graph_order(d["row_ptr"]) if not a.natural_order else None
    out = torch.empty((N, plan.d_out), dtype=plan.torch_dtype, device=device)
    gx = torch.empty_like(d["x"])
    gy = torch.empty_like(y)
    gw = torch.empty_like(d["w"])

    receiver = a.backward_schedule == "receiver"
    ws = None
    if receiver:
        full, least = cg.conv_backward_receiver_workspace_size(plan, N, E)
        ws = torch.empty(max(least, min(full, int(a.receiver_workspace_gib * 2**30))), dtype=torch.uint8,
                         device=device)
        row_bytes = plan.d_x * es
        ranges = -(-E // (ws.numel() // row_bytes)) if E else 0

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        cg.conv_forward(plan, d["row_ptr"], d["col"], d["x"], y, d["w"], out=out, order=order)
        if ev is not None:
            ev[1].record()
        if receiver:
            cg.conv_backward_receiver(plan, d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"], gx, gy, gw,
                                      workspace=ws)
        else:
            cg.conv_backward(plan, d["row_ptr"], d["col"], tr, d["x"], y, d["w"], d["g"], gx, gy, gw)
        if ev is not None:
            ev[2].record()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(a.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    bwd_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms_per_step = wall * 1e3 / a.steps
    cold = cold_cache_times(a, step, device)
    fwd_b, bwd_b = algorithmic_bytes(plan, N, E, es)
    fwd_k = split_kernel("cgtp_conv_fwd", plan.row_split(N, E))
    # the receiver-order backward is one call of several launches (cgtp_conv_rbw per path group and
    # edge range, cgtp_conv_rbw_dx per range); its time and bytes are those of the whole call
    bwd_k = ("cgtp_conv_rbw", "cgtp_conv_rbw_dx") if receiver else "cgtp_conv_bwd"
    dom = (bwd_k, bwd_ms, bwd_b) if bwd_ms >= fwd_ms else (fwd_k, fwd_ms, fwd_b)
    achieved = dom[2] / (dom[1] * 1e-3) / 1e9
    traffic = measured_traffic(plan, spec, a.dtype, dom[0])
    line = {
        "metric": METRIC,
        "value": E / (ms_per_step * 1e-3),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": a.dtype,
        "data": "synthetic",
        "config": {"workload": spec.name, "N": N, "E": E, "in_irreps": spec.in_irreps,
                   "sh_lmax": spec.lmax_sh, "paths": plan.num_paths, "d_out": plan.d_out,
                   "step": "conv_forward + conv_backward (grad_x, grad_y, grad_w)",
                   "receiver_schedule": "natural" if a.natural_order else "heavy-first",
                   "backward_schedule": (f"receiver order, {ws.numel()} B workspace, {ranges} edge range(s), "
                                         f"{plan.info.fwd_tasks} task(s)") if receiver else "sender order",
                   "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
                   "fwd_edges_per_s": E / (fwd_ms * 1e-3), "bwd_edges_per_s": E / (bwd_ms * 1e-3),
                   "spread_ms": spread(evs), "cold_cache": cold},
        "roofline": {"bound": "hbm", "kernel": "+".join(dom[0]) if isinstance(dom[0], tuple) else dom[0],
                     "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": dom[2], "avg_launch_ms": dom[1],
                     "algorithmic_bytes_per_edge": dom[2] / E if E else None,
                     "other": {"kernel": fwd_k if dom[0] == bwd_k else "+".join(bwd_k) if receiver else bwd_k,
                               "achieved": (fwd_b / (fwd_ms * 1e-3) if dom[0] == bwd_k
                                            else bwd_b / (bwd_ms * 1e-3)) / 1e9}},
        "cpu_baseline": None,
    }
    if not a.no_cpu:
        line["cpu_baseline"] = cpu_baseline(spec, a.seed, host_graph)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
