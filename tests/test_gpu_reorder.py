"""GPU parity of gnn_reorder (degree sort, RCM), the relabelled CSR and
gnn_permute_rows against the oracle: permutations and CSR arrays are integer
results and must be bit-equal."""
import os

import numpy as np
import pytest
import torch

import gen
import graph_neural_network_amd as gnn
import oracle
from gpu_util import dev, dev_bf16, dev_csr, host, scaled_err

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def graphs():
    out = {}
    lines = [l.split("#")[0].split() for l in open(os.path.join(GOLDEN, "rcm_hand.txt"))]
    lines = [l for l in lines if l]
    n = int([l for l in lines if l[0] == "n"][0][1])
    arcs = np.array([int(t) for t in [l for l in lines if l[0] == "arcs"][0][1:]]).reshape(-1, 2)
    out["golden"] = gen.from_edges(n, arcs[:, 0], arcs[:, 1])
    rng = np.random.default_rng(4)
    lab = rng.permutation(500)
    out["path"] = gen.from_edges(500, np.r_[lab[:-1], lab[1:]], np.r_[lab[1:], lab[:-1]])
    k = 30
    lab = rng.permutation(k * k)
    s, d = [], []
    for r in range(k):
        for c in range(k):
            if c + 1 < k:
                s.append(lab[r * k + c]); d.append(lab[r * k + c + 1])
            if r + 1 < k:
                s.append(lab[r * k + c]); d.append(lab[(r + 1) * k + c])
    out["grid"] = gen.from_edges(k * k, np.r_[s, d], np.r_[d, s])
    out["rmat"] = gen.rmat(0x5EED0400, 20000, 160000)
    out["rmat_loops"] = gen.rmat(0x5EED0401, 7001, 50000, self_loops=True)
    out["cluster"] = gen.cluster(0x5EED0402, 64 * 50, 64, 0.5, 0.01, self_loops=True)
    out["empty"] = gen.from_edges(37, [], [])
    out["components"] = components(rng)
    return out


def components(rng):
    """Disjoint pieces under shuffled labels: a 5001-vertex star (the largest
    component, its centre's row past 4096 entries), three hubs with 100, 2000
    and 4500 neighbours among 4600 vertices (rows in each sort tier), a
    3000-vertex path, a small R-MAT graph, cliques of 5-12 and isolated
    vertices; every edge in both directions."""
    pieces, n = [], 0

    def add(k, s, d):
        nonlocal n
        pieces.append((np.asarray(s, np.int64) + n, np.asarray(d, np.int64) + n))
        n += k

    add(5001, np.zeros(5000), np.arange(1, 5001))
    hub_s, hub_d = [], []
    for h, deg in enumerate((100, 2000, 4500)):
        nb = 3 + rng.choice(4597, size=deg, replace=False)
        hub_s.append(np.full(deg, h)); hub_d.append(nb)
    add(4600, np.concatenate(hub_s + [[0, 1]]), np.concatenate(hub_d + [[1, 2]]))
    add(3000, np.arange(2999), np.arange(1, 3000))
    rrp, rci = gen.rmat(0x5EED0403, 1500, 6000)
    add(1500, np.repeat(np.arange(1500), np.diff(rrp)), rci)
    for size in rng.integers(5, 13, size=40):
        i, j = np.triu_indices(int(size), 1)
        add(int(size), i, j)
    add(200, [], [])
    s = np.concatenate([p[0] for p in pieces])
    d = np.concatenate([p[1] for p in pieces])
    lab = rng.permutation(n)
    return gen.from_edges(n, np.r_[lab[s], lab[d]], np.r_[lab[d], lab[s]])


GRAPHS = graphs()


@pytest.mark.parametrize("name", sorted(GRAPHS))
@pytest.mark.parametrize("kind", ["degree", "rcm"])
def test_reorder_matches_oracle(name, kind):
    rp, ci = GRAPHS[name]
    csr = dev_csr(rp, ci)
    perm, rp2, ci2 = gnn.gnn_reorder(csr, kind)
    perm = host(perm)
    ref = oracle.degree_sort(rp) if kind == "degree" else oracle.rcm(rp, ci)
    assert np.array_equal(perm, ref)
    orp, oci = oracle.permute_csr(rp, ci, ref)
    assert np.array_equal(host(rp2), orp)
    assert np.array_equal(host(ci2), oci)


def test_rcm_bandwidth_on_relabelled_path_and_grid():
    for name, bound in (("path", 1), ("grid", 59)):
        rp, ci = GRAPHS[name]
        perm = host(gnn.gnn_reorder(dev_csr(rp, ci), "rcm", apply=False))
        inv = np.empty_like(perm)
        inv[perm] = np.arange(perm.size)
        rows = np.repeat(np.arange(rp.size - 1), np.diff(rp))
        assert np.abs(inv[rows] - inv[ci]).max() <= bound


@pytest.mark.parametrize("n", [7, 20001])
@pytest.mark.parametrize("F", [33, 64, 100, 128, 256])
def test_permute_rows_widths(n, F):
    """Rows that are whole 16-byte units take the 16-byte copy, 132 B rows
    the element copy; row counts that do not fill the last workgroup."""
    rng = np.random.default_rng(F * 1000 + n)
    P = rng.permutation(n).astype(np.int32)
    X = gen.gauss_f32(F + n, (n, F))
    Xp = gnn.gnn_permute_rows(dev(P), dev(X))
    assert np.array_equal(host(Xp), X[P])


def test_permute_rows_and_reordered_spmm():
    rp, ci = GRAPHS["rmat"]
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    X = gen.gauss_f32(3, (n, 128))
    Xb = gen.gauss_bf16(4, (n, 256))
    for kind in ("degree", "rcm"):
        perm, rp2, ci2 = gnn.gnn_reorder(csr, kind)
        P = host(perm)
        Xp = gnn.gnn_permute_rows(perm, dev(X))
        assert np.array_equal(host(Xp), X[P])
        Xbp = gnn.gnn_permute_rows(perm, dev_bf16(Xb))
        assert np.array_equal(host(Xbp.view(torch.int16)).view(np.uint16), Xb[P])
        # (P A P^T)(P X) = P (A X)
        csr2 = gnn.Csr(rp2, ci2)
        Y = host(gnn.gnn_spmm(csr, dev(X), "both"))
        Y2 = host(gnn.gnn_spmm(csr2, Xp, "both"))
        ref, mag = oracle.spmm(rp, ci, X, "both")
        assert scaled_err(Y2, ref[P], mag[P]) <= 1e-5
        assert scaled_err(Y, ref, mag) <= 1e-5
        # max is order-independent: values bit-exact after un-permuting; the
        # source index holds that value (which of several equal sources wins
        # depends on the numbering, so it is checked for validity only)
        Ym, am = gnn.gnn_reduce(csr, dev(X), "max", arg=True)
        Ym2, am2 = gnn.gnn_reduce(csr2, Xp, "max", arg=True)
        assert np.array_equal(host(Ym2), host(Ym)[P])
        a2 = host(am2)
        ok = a2 >= 0
        f = np.broadcast_to(np.arange(128), a2.shape)
        assert np.array_equal(host(Xp)[a2[ok], f[ok]], host(Ym2)[ok])
        assert np.array_equal(ok, (np.diff(host(rp2)) > 0)[:, None].repeat(128, 1))


def test_reorder_rmat1m_full():
    w = gen.reduce_rmat(with_x=False)
    csr = dev_csr(w.row_ptr, w.col_idx)
    for kind in ("degree", "rcm"):
        perm, rp2, ci2 = gnn.gnn_reorder(csr, kind)
        ref = oracle.degree_sort(w.row_ptr) if kind == "degree" else oracle.rcm(w.row_ptr, w.col_idx)
        assert np.array_equal(host(perm), ref)
        orp, oci = oracle.permute_csr(w.row_ptr, w.col_idx, ref)
        assert np.array_equal(host(rp2), orp) and np.array_equal(host(ci2), oci)
