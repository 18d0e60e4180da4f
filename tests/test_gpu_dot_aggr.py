"""GPU parity of gnn_dot_aggr (the dot-aggr reordering micro-benchmark)
against the fp64 oracle.

y_i = sum over row i's sources j of <x_i, x_j>.  Bar: 1e-5 of the oracle with
the error scaled by sum |x_i,d x_j,d| (an fp32 sum, like the SpMM bar); rows
without sources must give exactly 0.  Every mapping (feature- and
neighbour-parallel) and load width (4-byte, 16-byte) is checked on R-MAT
graphs with hub rows of several 64-edge rounds, rows split into plan chunks,
empty rows and a node count that does not fill the last workgroup; then at
the benchmark's size (R-MAT 1,000,000 nodes / 16,000,000 edges, D = 128) on
sampled rows, in the original and both reordered numberings.
"""
import numpy as np
import pytest
import torch

import gen
import graph_neural_network_amd as gnn
import oracle
from gpu_util import dev, dev_csr, host, scaled_err

pytestmark = pytest.mark.gpu
TOL = 1e-5
VARIANTS = [(m, l) for m in ("feature", "neighbor") for l in ("scalar", "vec16")]


@pytest.fixture(scope="module")
def small():
    # 3001 nodes: the last workgroup holds one node; rows up to several hundred edges
    rp, ci = gen.rmat(0x5EED0100, 3001, 45_000)
    d = np.diff(rp)
    assert d.max() > 200 and (d == 0).any()
    return rp, ci


def check(rp, ci, Xh, y, rows=None):
    ref, mag = oracle.dot_aggr(rp, ci, Xh, rows=rows)
    got = y if rows is None else y[rows]
    err = scaled_err(got, ref, mag)
    assert err <= TOL, f"scaled error {err}"
    return err


@pytest.mark.parametrize("map_,load", VARIANTS)
@pytest.mark.parametrize("D", [1, 3, 4, 17, 32, 64, 100, 128, 260, 512, 1024])
def test_dot_aggr_small(small, map_, load, D):
    if load == "vec16" and D % 4:
        pytest.skip("16-byte loads need D % 4 == 0")
    rp, ci = small
    Xh = gen.gauss_f32(0xFEA70100 + D, (rp.size - 1, D))
    csr = dev_csr(rp, ci)
    y = gnn.gnn_dot_aggr(csr, dev(Xh), map_, load)
    check(rp, ci, Xh, host(y))


@pytest.mark.parametrize("map_,load", VARIANTS)
def test_dot_aggr_split_rows_and_strides(small, map_, load):
    """Rows cut into 64-edge chunks (partials added in chunk order), no split
    at all, and a padded row stride."""
    rp, ci = small
    n, D = rp.size - 1, 96
    full = gen.gauss_f32(0xFEA70200, (n, D + 12))
    Xh = np.ascontiguousarray(full[:, :D])
    csr = dev_csr(rp, ci)
    Xd = dev(full)[:, :D]
    assert Xd.stride(0) == D + 12
    for opts in (dict(heavy_quantile=0.5, chunk_edges=64), dict(heavy_quantile=-1.0)):
        plan = gnn.gnn_plan_create(csr, **opts)
        st = gnn.gnn_plan_stats(plan)
        if opts.get("chunk_edges"):
            assert st["heavy_rows"] > 0
        y = gnn.gnn_dot_aggr(csr, Xd, map_, load, plan=plan)
        check(rp, ci, Xh, host(y))


@pytest.mark.parametrize("map_,load", VARIANTS)
def test_dot_aggr_closed_forms(map_, load):
    """All-ones features give D * deg exactly; a graph without edges gives 0;
    single self-loop rows give |x_i|^2."""
    rp, ci = gen.rmat(0x5EED0101, 1000, 9000)
    D = 64
    csr = dev_csr(rp, ci)
    y = host(gnn.gnn_dot_aggr(csr, torch.ones((1000, D), device="cuda"), map_, load))
    assert np.array_equal(y, (D * np.diff(rp)).astype(np.float32))
    empty = dev_csr(np.zeros(501, np.int32), np.zeros(0, np.int32))
    y0 = host(gnn.gnn_dot_aggr(empty, torch.randn((500, D), device="cuda"), map_, load))
    assert np.all(y0 == 0.0)
    n = 257
    rpl, cil = np.arange(n + 1, dtype=np.int32), np.arange(n, dtype=np.int32)
    Xh = gen.gauss_f32(0xFEA70300, (n, D))
    y1 = host(gnn.gnn_dot_aggr(dev_csr(rpl, cil), dev(Xh), map_, load))
    check(rpl, cil, Xh, y1)


def test_dot_aggr_mappings_agree(small):
    """Same sums from every mapping and load width (different rounding order only)."""
    rp, ci = small
    D = 128
    Xh = gen.gauss_f32(0xFEA70400, (rp.size - 1, D))
    csr = dev_csr(rp, ci)
    Xd = dev(Xh)
    ys = [host(gnn.gnn_dot_aggr(csr, Xd, m, l)) for m, l in VARIANTS]
    _, mag = oracle.dot_aggr(rp, ci, Xh)
    for y in ys[1:]:
        assert scaled_err(y, ys[0], mag) <= 2 * TOL


@pytest.fixture(scope="module")
def big():
    w = gen.reduce_rmat(with_x=False)
    D = 128
    Xh = gen.gauss_f32(0xFEA70500, (w.n, D))
    csr = gnn.Csr(torch.from_numpy(w.row_ptr).cuda(), torch.from_numpy(w.col_idx).cuda())
    return w, Xh, csr


def sample_rows(rp, k, seed):
    d = np.diff(rp)
    rng = np.random.default_rng(seed)
    return np.unique(np.r_[rng.integers(0, rp.size - 1, k), np.argsort(-d, kind="stable")[:16]]).astype(np.int32)


@pytest.mark.slow
def test_dot_aggr_rmat1m_all_orders(big):
    """The benchmark's graph and plan (chunks of 256 edges) at D = 128: sampled
    rows of every variant in the original, degree-sorted and RCM numberings."""
    w, Xh, csr = big
    rows = sample_rows(w.row_ptr, 3000, 12)
    ref, mag = oracle.dot_aggr(w.row_ptr, w.col_idx, Xh, rows=rows)
    Xd = torch.from_numpy(Xh).cuda()
    graphs = {"original": (csr, Xd, np.arange(w.n, dtype=np.int32))}
    for kind in ("degree", "rcm"):
        perm, rp2, ci2 = gnn.gnn_reorder(csr, kind)
        P = host(perm)
        inv = np.empty_like(P)
        inv[P] = np.arange(P.size, dtype=np.int32)
        graphs[kind] = (gnn.Csr(rp2, ci2), gnn.gnn_permute_rows(perm, Xd), inv)
    for kind, (c, X, inv) in graphs.items():
        plan = gnn.gnn_plan_create(c, chunk_edges=256)
        for m, l in VARIANTS:
            y = gnn.gnn_dot_aggr(c, X, m, l, plan=plan)
            got = host(y[torch.from_numpy(inv[rows]).long().cuda()])
            err = scaled_err(got, ref, mag)
            assert err <= TOL, (kind, m, l, err)
