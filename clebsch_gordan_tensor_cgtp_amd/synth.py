"""Seeded synthetic inputs: graphs, features, edge vectors, weights, gradients.

This module draws random numbers and builds index arrays only; it holds none
of the tensor product's arithmetic (no CG coefficients, no spherical
harmonics).  It is the one piece shared by the HIP path's callers and the
CPU checks.

Recipe (the pages name no dataset; these stand in for the molecular graphs
NequIP/MACE run on, sciencestack.ai page Figures 4-5, and for the
edge-scaling regimes of the Sobek page):

* seeds: ``np.random.SeedSequence(seed)`` spawns six children in the order
  graph, x, vec, w, sample, upstream; each drives its own PCG64
  ``default_rng`` (``upstream`` spawns three more, for the double backward's
  upstream gradients of dx, dY and dW, all ~ N(0, 1)).  Draws are float64 and
  cast to the run's dtype afterwards.
* uniform graph: E receivers drawn uniformly from [0, N) (so the in-degree is
  Binomial(E, 1/N) ~ Poisson(E/N) with an exact total), E senders drawn
  uniformly with replacement (self-loops and duplicates allowed), a stable
  sort by receiver gives the receiver CSR.
* power-law graph: raw degree min(zipf(a), cap) per node, scaled by a water
  level so that sum(min(level*raw, cap)) = E, floored, the remainder handed
  out by largest fractional part with ties to the lower node index; senders
  drawn uniformly in CSR order.
* edge vectors ~ N(0, I3) and weights ~ N(0, 1)/sqrt(fan_in) are drawn after
  the sort, in CSR order; x ~ N(0, 1); the output gradient ~ N(0, 1) comes
  from the ``sample`` child.
* tensors above ``HOST_LIMIT`` elements (the per-edge weights of the largest
  graphs, tens of GB) are drawn on the GPU by torch's seeded generator, in
  float64, then cast; the seed is the first word of the child's state.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np

HOST_LIMIT = 400_000_000
STREAMS = ("graph", "x", "vec", "w", "sample", "upstream")


def streams(seed: int = 0):
    children = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {name: child for name, child in zip(STREAMS, children)}


def upstream_streams(seed: int = 0):
    """Three independent children (for the upstream gradients of dx, dY and dW in the
    double backward); adding them left the first five streams unchanged."""
    gx, gy, gw = streams(seed)["upstream"].spawn(3)
    return {"gg_x": gx, "gg_y": gy, "gg_w": gw}


def rng(child: np.random.SeedSequence) -> np.random.Generator:
    return np.random.default_rng(child)


# ---------------------------------------------------------------------------- graphs

def uniform_graph(n_nodes: int, n_edges: int, gen: np.random.Generator):
    """Receiver CSR (row_ptr[N+1], col[E], int32) with uniformly drawn receivers and senders."""
    recv = gen.integers(0, n_nodes, n_edges, dtype=np.int64)
    send = gen.integers(0, n_nodes, n_edges, dtype=np.int64)
    order = np.argsort(recv, kind="stable")
    deg = np.bincount(recv, minlength=n_nodes)
    row_ptr = np.zeros(n_nodes + 1, dtype=np.int64)
    np.cumsum(deg, out=row_ptr[1:])
    return row_ptr.astype(np.int32), send[order].astype(np.int32)


def powerlaw_degrees(n_nodes: int, n_edges: int, a: float, cap: int, gen: np.random.Generator):
    """In-degrees with a Zipf(a) shape, capped, summing exactly to n_edges."""
    if n_edges > n_nodes * cap:
        raise ValueError("cap too small for the edge count")
    raw = np.minimum(gen.zipf(a, n_nodes), cap).astype(np.float64)
    lo, hi = 0.0, float(cap)  # water level: sum(min(level*raw, cap)) is monotone in level
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.minimum(mid * raw, cap).sum() < n_edges:
            lo = mid
        else:
            hi = mid
    target = np.minimum(hi * raw, cap)
    deg = np.floor(target).astype(np.int64)
    rem = int(n_edges - deg.sum())
    frac = target - deg
    # largest fractional part first, ties -> lower index; never exceed cap
    order = np.lexsort((np.arange(n_nodes), -frac))
    order = order[deg[order] < cap]
    deg[order[:rem]] += 1
    assert deg.sum() == n_edges and deg.max() <= cap
    return deg


def powerlaw_graph(n_nodes: int, n_edges: int, a: float, cap: int, gen: np.random.Generator):
    deg = powerlaw_degrees(n_nodes, n_edges, a, cap, gen)
    row_ptr = np.zeros(n_nodes + 1, dtype=np.int64)
    np.cumsum(deg, out=row_ptr[1:])
    col = gen.integers(0, n_nodes, n_edges, dtype=np.int64)
    return row_ptr.astype(np.int32), col.astype(np.int32)


# ---------------------------------------------------------------------------- dense draws

def normal(child: np.random.SeedSequence, shape, scale: float = 1.0, dtype=np.float64,
           device: Optional[str] = None):
    """N(0, scale^2) draws.  Host numpy below HOST_LIMIT elements, else torch on ``device``."""
    numel = int(np.prod(shape))
    if numel <= HOST_LIMIT or device is None:
        a = rng(child).standard_normal(shape)
        if scale != 1.0:
            a *= scale
        return a.astype(dtype, copy=False)
    import torch
    tdtype = {np.float32: torch.float32, np.float64: torch.float64}[np.dtype(dtype).type]
    g = torch.Generator(device=device)
    g.manual_seed(int(child.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1)))
    out = torch.empty(shape, dtype=tdtype, device=device)
    chunk = 1 << 27
    flat = out.view(-1)
    for s in range(0, numel, chunk):
        n = min(chunk, numel - s)
        t = torch.randn(n, generator=g, dtype=torch.float64, device=device)
        if scale != 1.0:
            t.mul_(scale)
        flat[s:s + n].copy_(t)
        del t
    return out


# ---------------------------------------------------------------------------- workloads

@dataclass(frozen=True)
class ConvSpec:
    name: str
    n_nodes: int
    n_edges: int
    in_irreps: str
    lmax_sh: int
    lmax_out: int
    graph: str = "uniform"      # or "powerlaw"
    zipf_a: float = 2.0
    cap: int = 2000
    mode: str = "uvu"           # "uvw": shared [P][mul_in][mul_out] weights, outputs ``out_irreps``
    out_irreps: Optional[str] = None


@dataclass(frozen=True)
class TPSpec:
    name: str
    batch: int
    in_irreps: str
    lmax_sh: int
    mode: str                   # "uvu" or "uvw"
    out_irreps: Optional[str] = None


def _ladder(mul: int, lmax: int) -> str:
    return "+".join(f"{mul}x{l}{'e' if l % 2 == 0 else 'o'}" for l in range(lmax + 1))


# The five workloads: a small batched product, a NequIP-like convolution, a
# MACE-like convolution, a high-L dense-mixing product and a large power-law
# streaming convolution.
TP_SMALL = TPSpec("tp-uvu-B1024-4x(0e,1o)-sh2", 1024, "4x0e+4x1o", 2, "uvu")
CONV_NEQUIP = ConvSpec("conv-N5000-E200k-32x(0e,1o,2e)-sh2", 5000, 200_000, _ladder(32, 2), 2, 2)
CONV_MACE = ConvSpec("conv-N20000-E1M-128x(0e,1o,2e,3o)-sh3", 20_000, 1_000_000, _ladder(128, 3), 3, 3)
TP_HIGHL = TPSpec("tp-uvw-B50000-16x(0..7)-sh7", 50_000, _ladder(16, 7), 7, "uvw", _ladder(16, 7))
CONV_STREAM = ConvSpec("conv-N200k-E10M-powerlaw-64x(0e,1o,2e)-sh2", 200_000, 10_000_000,
                       _ladder(64, 2), 2, 2, graph="powerlaw", zipf_a=2.0, cap=2000)

WORKLOADS = {"c1": TP_SMALL, "c2": CONV_NEQUIP, "c3": CONV_MACE, "c4": TP_HIGHL, "c5": CONV_STREAM}

# The NequIP-like graph and inputs with fully connected multiplicity mixing (uvw, shared
# weights) into every reachable output irrep at 32 channels (Sobek page, Abstract: the fully
# connected operator family).
CONV_NEQUIP_UVW = ConvSpec("conv-uvw-N5000-E200k-32x(0e,1o,2e)-sh2", 5000, 200_000, _ladder(32, 2), 2, 2,
                           mode="uvw", out_irreps="32x0e+32x1o+32x2e+32x1e+32x2o")
# A batched uvu product over as many rows as the streaming graph has nodes, with the NequIP-like
# irreps (HBM-bound, unlike the 1,024-row batch that is launch-bound).
TP_BIG = TPSpec("tp-uvu-B200k-32x(0e,1o,2e)-sh2", 200_000, _ladder(32, 2), 2, "uvu")
# A batched uvw product with multiplicities above 16 (32 channels in and out): its backward runs
# through the uvw convolution's kernels on the identity graph.
TP_WIDE_UVW = TPSpec("tp-uvw-B50000-32x(0e,1o,2e)-sh2", 50_000, _ladder(32, 2), 2, "uvw",
                     "32x0e+32x1o+32x2e+32x1e+32x2o")
EXTRA_WORKLOADS = {"c2uvw": CONV_NEQUIP_UVW, "c1big": TP_BIG, "c4wide": TP_WIDE_UVW}


def conv_graph(spec: ConvSpec, seed: int = 0):
    st = streams(seed)
    g = rng(st["graph"])
    if spec.graph == "uniform":
        return uniform_graph(spec.n_nodes, spec.n_edges, g)
    return powerlaw_graph(spec.n_nodes, spec.n_edges, spec.zipf_a, spec.cap, g)


def scaled(spec: ConvSpec, n_nodes: int, n_edges: int, in_irreps: Optional[str] = None) -> ConvSpec:
    """Same recipe at another size (parity cases the oracle finishes in seconds)."""
    return ConvSpec(spec.name + f"@N{n_nodes}E{n_edges}", n_nodes, n_edges,
                    in_irreps or spec.in_irreps, spec.lmax_sh, spec.lmax_out, spec.graph,
                    spec.zipf_a, min(spec.cap, max(1, n_edges)))
