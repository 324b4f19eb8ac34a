"""The seeded input generators: deterministic, valid CSR, the stated degree laws."""
import numpy as np

from clebsch_gordan_tensor_cgtp_amd import synth


def test_streams_are_deterministic_and_distinct():
    a, b = synth.streams(0), synth.streams(0)
    for k in synth.STREAMS:
        assert np.array_equal(synth.rng(a[k]).integers(0, 1 << 30, 8), synth.rng(b[k]).integers(0, 1 << 30, 8))
    draws = {k: synth.rng(a[k]).integers(0, 1 << 30, 4).tolist() for k in synth.STREAMS}
    assert len({tuple(v) for v in draws.values()}) == len(synth.STREAMS)


def test_uniform_graph_csr():
    rp, col = synth.uniform_graph(500, 20_000, np.random.default_rng(1))
    assert rp.dtype == np.int32 and col.dtype == np.int32
    assert rp[0] == 0 and rp[-1] == 20_000 and np.all(np.diff(rp) >= 0)
    assert col.min() >= 0 and col.max() < 500
    deg = np.diff(rp)
    assert abs(deg.mean() - 40) < 1e-9 and 30 < deg.var() < 50   # ~Poisson(40)


def test_uniform_graph_is_stable_sort_by_receiver():
    g = np.random.default_rng(2)
    rp, col = synth.uniform_graph(50, 400, g)
    g = np.random.default_rng(2)
    recv = g.integers(0, 50, 400)
    send = g.integers(0, 50, 400)
    assert np.array_equal(col, send[np.argsort(recv, kind="stable")])


def test_powerlaw_degrees_full_size():
    deg = synth.powerlaw_degrees(200_000, 10_000_000, 2.0, 2000, synth.rng(synth.streams(0)["graph"]))
    assert deg.sum() == 10_000_000 and deg.max() == 2000
    assert deg.min() >= 1
    n_cap = int((deg == 2000).sum())
    assert 300 < n_cap < 2000
    # heavy tail: a small fraction of receivers holds a large share of the edges
    top = np.sort(deg)[::-1]
    assert top[: n_cap].sum() / deg.sum() > 0.05


def test_powerlaw_graph_exact_draw():
    """The 10M-edge graph is pinned exactly (min 12, max 2,000, 749 capped receivers, median 13,
    99th percentile 743, and a digest of the degree array), so a change to the draw order or to
    the water-filling rounding is noticed.  (Another derivation of the same rule, with its own raw
    Zipf draws, counts 737 capped receivers: the count depends on the draws, not only on the
    rule.)"""
    import hashlib
    deg = synth.powerlaw_degrees(200_000, 10_000_000, 2.0, 2000, synth.rng(synth.streams(0)["graph"]))
    assert (int(deg.min()), int(deg.max()), int((deg == 2000).sum())) == (12, 2000, 749)
    assert (int(np.median(deg)), int(np.percentile(deg, 99))) == (13, 743)
    assert hashlib.sha1(deg.astype(np.int64).tobytes()).hexdigest() == "9f75f124259f964bb63e0f3b48d08395638aee6f"


def test_chunked_normal_equals_one_shot():
    child = synth.streams(0)["w"]
    one = synth.rng(child).standard_normal(3_000_000)
    g = synth.rng(child)
    parts = [g.standard_normal(1_000_000) for _ in range(3)]
    assert np.array_equal(one, np.concatenate(parts))


def test_workload_table():
    assert set(synth.WORKLOADS) == {"c1", "c2", "c3", "c4", "c5"}
    c2 = synth.WORKLOADS["c2"]
    assert (c2.n_nodes, c2.n_edges, c2.in_irreps) == (5000, 200_000, "32x0e+32x1o+32x2e")
    assert synth.WORKLOADS["c4"].in_irreps == "+".join(f"16x{l}{'eo'[l % 2]}" for l in range(8))
