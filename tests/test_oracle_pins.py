"""Pins for the CPU oracle: every oracle function is checked against
something other than itself — a dense brute force written as matrix algebra,
closed forms, invariants, hand-worked examples under tests/golden/, or a
library routine that reaches the same plain definition.

Definitions: Fomina et al., "On efficient scaling of GNNs via IO-aware layer
implementations" (three operator families; reduction, fused attention and
block-sparse appendices), and the textbook RCM named in Tang et al., "A
High-Throughput Solver for Marginalized Graph Kernels on GPU".
"""
import math
import os

import numpy as np
import pytest

import gen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# helpers (test-side, independent of oracle.c)
# ----------------------------------------------------------------------------

def random_graph(rng, n, p, loops=False, sym=False):
    A = rng.random((n, n)) < p          # A[i, j]: edge j -> i
    if sym:
        A = A | A.T
    np.fill_diagonal(A, loops)
    dst, src = np.nonzero(A)
    rp, ci = gen.from_edges(n, src, dst)
    return A, rp, ci


def dense_from_csr(rp, ci, n_cols):
    n = rp.size - 1
    A = np.zeros((n, n_cols), bool)
    for i in range(n):
        A[i, ci[rp[i]:rp[i + 1]]] = True
    return A


def bf16(rng, shape, std=1.0):
    return gen.f32_to_bf16((rng.standard_normal(shape) * std).astype(np.float32))


def dec(b):
    return gen.bf16_to_f32(b).astype(np.float64)


def load_pairs(path):
    out = {}
    with open(path) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            out.setdefault(key, []).append(vals)
    return out


# ----------------------------------------------------------------------------
# generator sanity (inputs only)
# ----------------------------------------------------------------------------

def test_gen_csr_shape_and_determinism():
    rp, ci = gen.rmat(7, 5000, 40000)
    rp2, ci2 = gen.rmat(7, 5000, 40000)
    assert np.array_equal(rp, rp2) and np.array_equal(ci, ci2)
    assert rp[-1] == 40000 and rp.size == 5001
    rows = np.repeat(np.arange(5000), np.diff(rp))
    key = rows.astype(np.int64) * (1 << 32) + ci
    assert np.all(np.diff(key) > 0), "rows sorted, no duplicates"
    assert np.all(rows != ci), "no self loops"
    rp, ci = gen.rmat(7, 5000, 40000, self_loops=True)
    rows = np.repeat(np.arange(5000), np.diff(rp))
    assert (rows == ci).sum() == 5000 and rp[-1] == 45000


def test_gen_er_symmetric():
    rp, ci = gen.er_undirected(1, 300, 1000)
    A = dense_from_csr(rp, ci, 300)
    assert np.array_equal(A, A.T) and A.diagonal().all()
    assert A.sum() == 2 * 1000 + 300


def test_gen_cluster_structure():
    rp, ci = gen.cluster(3, 64 * 20, 64, 0.5, 0.01)
    n = 64 * 20
    rows = np.repeat(np.arange(n), np.diff(rp))
    intra = (rows // 64 == ci // 64) & (rows != ci)
    inter = rows // 64 != ci // 64
    assert (rows == ci).sum() == n
    assert inter.sum() == round(0.01 * intra.sum())
    assert abs(intra.sum() / (20 * 64 * 63) - 0.5) < 0.03


def test_gen_gauss_moments():
    x = gen.gauss_f32(5, 200000)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    b = gen.gauss_bf16(5, 1000)
    assert np.array_equal(b, gen.f32_to_bf16(gen.gauss_f32(5, 1000)))


# ----------------------------------------------------------------------------
# SpMM: dense brute force, identity, complete graph, eigenvector, permutation
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("norm", ["none", "left", "right", "both"])
@pytest.mark.parametrize("weighted", [False, True])
def test_spmm_dense_bruteforce(rng, norm, weighted):
    n, F = 48, 5
    A, rp, ci = random_graph(rng, n, 0.15, loops=True)
    X = rng.standard_normal((n, F)).astype(np.float32)
    ev = rng.standard_normal(ci.size).astype(np.float32) if weighted else None
    W = np.zeros((n, n))
    for i in range(n):
        for e in range(rp[i], rp[i + 1]):
            W[i, ci[e]] = float(ev[e]) if weighted else 1.0
    din = A.sum(1).astype(np.float64)
    dout = A.sum(0).astype(np.float64)
    with np.errstate(divide="ignore"):
        if norm == "left":
            W = np.diag(np.where(din > 0, 1 / din, 0)) @ W
        elif norm == "right":
            W = W @ np.diag(np.where(dout > 0, 1 / dout, 0))
        elif norm == "both":
            W = np.diag(np.where(din > 0, din ** -0.5, 0)) @ W @ np.diag(np.where(dout > 0, dout ** -0.5, 0))
    ref = W @ X.astype(np.float64)
    Y, Ya = oracle.spmm(rp, ci, X, norm, edge_val=ev)
    np.testing.assert_allclose(Y, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(Ya, np.abs(W) @ np.abs(X.astype(np.float64)), rtol=0, atol=1e-12)


def test_spmm_rows_subset_and_bf16(rng):
    n, F = 40, 7
    A, rp, ci = random_graph(rng, n, 0.2)
    Xb = bf16(rng, (n, F))
    full = oracle.spmm(rp, ci, Xb, "none", x_is_bf16=True, want_abs=False)
    np.testing.assert_allclose(full, A.astype(np.float64) @ dec(Xb), atol=1e-12, rtol=0)
    rows = np.array([5, 0, 39, 5], np.int32)
    sub = oracle.spmm(rp, ci, Xb, "none", x_is_bf16=True, rows=rows, want_abs=False)
    assert np.array_equal(sub, full[rows])


@pytest.mark.parametrize("norm", ["none", "left", "right", "both"])
def test_spmm_identity(rng, norm):
    n, F = 33, 4
    rp, ci = gen.from_edges(n, np.arange(n), np.arange(n))
    X = rng.standard_normal((n, F)).astype(np.float32)
    Y, _ = oracle.spmm(rp, ci, X, norm)
    assert np.array_equal(Y, X.astype(np.float64))


def test_spmm_complete_graph_closed_forms(rng):
    n, F = 200, 3
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    rp, ci = gen.from_edges(n, j.ravel(), i.ravel())
    X = rng.standard_normal((n, F)).astype(np.float32)
    Y, _ = oracle.spmm(rp, ci, X, "both")
    np.testing.assert_allclose(Y, np.broadcast_to(X.astype(np.float64).mean(0), (n, F)),
                               atol=1e-13, rtol=0)
    ones = np.ones((n, 1), np.float32)
    assert np.array_equal(oracle.spmm(rp, ci, ones, "none")[0][:, 0], np.full(n, float(n)))
    np.testing.assert_allclose(oracle.spmm(rp, ci, ones, "left")[0][:, 0], 1.0, atol=1e-14)


def test_spmm_sqrt_degree_eigenvector():
    # GCN normalisation on a symmetric graph: A_hat sqrt(d) = sqrt(d), since
    # sum_j (d_i d_j)^-1/2 sqrt(d_j) = deg(i) / sqrt(d_i) = sqrt(d_i).
    rp, ci = gen.er_undirected(0x5EED0001, 2000, 8000, self_loops=True)
    d = np.diff(rp).astype(np.float64)
    X = np.sqrt(d).astype(np.float32)[:, None]
    Y, _ = oracle.spmm(rp, ci, X, "both")
    np.testing.assert_allclose(Y[:, 0], X[:, 0].astype(np.float64), rtol=1e-6)


def test_spmm_permutation_equivariance(rng):
    n, F = 300, 6
    rp, ci = gen.rmat(11, n, 3000)
    X = rng.standard_normal((n, F)).astype(np.float32)
    pi = rng.permutation(n)        # new id of old vertex v is pi[v]
    rows = np.repeat(np.arange(n), np.diff(rp))
    rp2, ci2 = gen.from_edges(n, pi[ci], pi[rows])
    X2 = np.empty_like(X)
    X2[pi] = X
    for norm in ("none", "both"):
        Y, _ = oracle.spmm(rp, ci, X, norm)
        Y2, _ = oracle.spmm(rp2, ci2, X2, norm)
        np.testing.assert_allclose(Y2[pi], Y, atol=1e-12, rtol=0)


def test_degrees_against_bincount():
    rp, ci = gen.rmat(3, 1000, 9000)
    din, dout = oracle.degrees(rp, ci)
    assert np.array_equal(din, np.diff(rp))
    assert np.array_equal(dout, np.bincount(ci, minlength=1000))


# ----------------------------------------------------------------------------
# Reductions
# ----------------------------------------------------------------------------

def test_reduce_dense_bruteforce(rng):
    n, F = 50, 6
    A, rp, ci = random_graph(rng, n, 0.2)
    X = rng.standard_normal((n, F)).astype(np.float32)
    Xd = X.astype(np.float64)
    deg = A.sum(1)
    s, _, sa = oracle.reduce(rp, ci, X, "sum")
    np.testing.assert_allclose(s, A @ Xd, atol=1e-12, rtol=0)
    np.testing.assert_allclose(sa, A @ np.abs(Xd), atol=1e-12, rtol=0)
    m, _, _ = oracle.reduce(rp, ci, X, "mean")
    ref = np.where(deg[:, None] > 0, (A @ Xd) / np.maximum(deg, 1)[:, None], 0.0)
    np.testing.assert_allclose(m, ref, atol=1e-12, rtol=0)
    for op, fn in (("max", np.max), ("min", np.min)):
        y, arg, _ = oracle.reduce(rp, ci, X, op)
        for i in range(n):
            nb = np.nonzero(A[i])[0]
            if nb.size == 0:
                assert np.all(y[i] == 0) and np.all(arg[i] == -1)
                continue
            best = fn(X[nb], axis=0)
            assert np.array_equal(y[i], best.astype(np.float64))
            # smallest source holding the extreme value (Gaussian: no ties)
            first = np.array([nb[np.nonzero(X[nb, f] == best[f])[0][0]] for f in range(F)])
            assert np.array_equal(arg[i], first)


def test_reduce_ties_golden():
    g = load_pairs(os.path.join(GOLDEN, "reduce_ties.txt"))
    n, F = 4, 3
    X = np.zeros((n, F), np.float32)
    for v in g["x"]:
        X[int(v[0])] = [float(t) for t in v[1:]]
    src, dst = [], []
    for v in g["row"]:
        for s in v[1:]:
            src.append(int(s))
            dst.append(int(v[0]))
    rp, ci = gen.from_edges(n, src, dst)
    for op in ("max", "min"):
        y, arg, _ = oracle.reduce(rp, ci, X, op)
        for v in g[op]:
            i = int(v[0])
            exp_val = np.array([float(t) for t in v[1::2]], np.float32)
            exp_arg = np.array([int(t) for t in v[2::2]])
            got = y[i].astype(np.float32)
            assert np.array_equal(got.view(np.uint32), exp_val.view(np.uint32)), (op, i, got)
            assert np.array_equal(arg[i], exp_arg), (op, i, arg[i])


def test_reduce_identity_and_membership(rng):
    n, F = 64, 5
    rp, ci = gen.from_edges(n, np.arange(n), np.arange(n))
    X = rng.standard_normal((n, F)).astype(np.float32)
    for op in ("sum", "mean", "max", "min"):
        y, arg, _ = oracle.reduce(rp, ci, X, op)
        assert np.array_equal(y, X.astype(np.float64))
        if op in ("max", "min"):
            assert np.array_equal(arg, np.repeat(np.arange(n)[:, None], F, 1))
    rp, ci = gen.rmat(9, 400, 4000)
    X = rng.standard_normal((400, F)).astype(np.float32)
    y, arg, _ = oracle.reduce(rp, ci, X, "max")
    nz = arg >= 0
    f_idx = np.broadcast_to(np.arange(F), arg.shape)
    assert np.array_equal(X[arg[nz], f_idx[nz]], y[nz].astype(np.float32))


def test_reduce_permutation_equivariance(rng):
    n, F = 500, 4
    rp, ci = gen.rmat(13, n, 6000)
    X = rng.standard_normal((n, F)).astype(np.float32)
    pi = rng.permutation(n)
    rows = np.repeat(np.arange(n), np.diff(rp))
    rp2, ci2 = gen.from_edges(n, pi[ci], pi[rows])
    X2 = np.empty_like(X)
    X2[pi] = X
    for op in ("max", "min"):
        y, a, _ = oracle.reduce(rp, ci, X, op)
        y2, a2, _ = oracle.reduce(rp2, ci2, X2, op)
        assert np.array_equal(y2[pi], y)
        a_map = np.where(a >= 0, pi[np.maximum(a, 0)], -1)
        assert np.array_equal(a2[pi], a_map)


# ----------------------------------------------------------------------------
# Attention (GATv2 and Graph Transformer)
# ----------------------------------------------------------------------------

def dense_softmax_aggregate(E, mask, V):
    """E [n, n] logits, mask [n, n], V [n, D] -> (out [n, D], lse [n])."""
    Em = np.where(mask, E, -np.inf)
    m = Em.max(1, keepdims=True)
    P = np.where(mask, np.exp(Em - np.where(np.isfinite(m), m, 0)), 0.0)
    s = P.sum(1, keepdims=True)
    out = np.where(s > 0, P @ V / np.where(s > 0, s, 1), 0.0)
    lse = np.where(s[:, 0] > 0, m[:, 0] + np.log(np.where(s[:, 0] > 0, s[:, 0], 1)), -np.inf)
    return out, lse


def test_gatv2_dense_bruteforce(rng):
    n, H, D = 40, 3, 8
    A, rp, ci = random_graph(rng, n, 0.2, loops=True)
    xl, xr = bf16(rng, (n, H, D)), bf16(rng, (n, H, D))
    att = rng.standard_normal((H, D)).astype(np.float32)
    out, lse, va = oracle.gatv2(rp, ci, xl, xr, att, 0.2)
    L, R = dec(xl), dec(xr)
    for h in range(H):
        Z = L[:, None, h, :] + R[None, :, h, :]                  # [i, j, d]
        act = np.where(Z > 0, Z, np.float64(np.float32(0.2)) * Z)
        E = act @ att[h].astype(np.float64)
        o, ls = dense_softmax_aggregate(E, A, R[:, h, :])
        np.testing.assert_allclose(out[:, h], o, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse[:, h], ls, atol=1e-12, rtol=0)


def test_gt_dense_bruteforce(rng):
    n, H, D = 40, 2, 16
    A, rp, ci = random_graph(rng, n, 0.25, loops=True)
    q, k, v = bf16(rng, (n, H, D)), bf16(rng, (n, H, D)), bf16(rng, (n, H, D))
    out, lse, va = oracle.gt(rp, ci, q, k, v)
    Q, K, V = dec(q), dec(k), dec(v)
    for h in range(H):
        E = (Q[:, h] @ K[:, h].T) / math.sqrt(D)                  # E[i, j] = q_i . k_j
        o, ls = dense_softmax_aggregate(E, A, V[:, h])
        np.testing.assert_allclose(out[:, h], o, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse[:, h], ls, atol=1e-12, rtol=0)
        np.testing.assert_allclose(va[:, h], dense_softmax_aggregate(E, A, np.abs(V[:, h]))[0],
                                   atol=1e-12, rtol=0)


def test_attention_two_edge_logistic_closed_form():
    # Row 0 <- {1, 2}: with two logits the softmax weight of the first is the
    # logistic function of their difference, 1 / (1 + exp(e2 - e1)).
    # GT, D = 1, scale 1: e_0j = q_0 k_j.
    rp, ci = gen.from_edges(3, [1, 2], [0, 0])
    f = lambda a: gen.f32_to_bf16(np.array(a, np.float32))
    q = f([[[1.5]], [[0.0]], [[0.0]]])
    k = f([[[0.0]], [[2.0]], [[-0.5]]])
    v = f([[[4.0]], [[1.0]], [[-3.0]]])
    out, lse, _ = oracle.gt(rp, ci, q, k, v, scale=1.0)
    e1, e2 = 1.5 * 2.0, 1.5 * -0.5
    w1 = 1.0 / (1.0 + math.exp(e2 - e1))
    assert abs(out[0, 0, 0] - (w1 * 1.0 + (1 - w1) * -3.0)) < 1e-14
    assert abs(lse[0, 0] - (e1 + math.log1p(math.exp(e2 - e1)))) < 1e-14
    # GATv2, D = 2: l_0 + r_j has one negative component, so the slope applies.
    xl = f([[[1.0, -2.0]], [[0.0, 0.0]], [[0.0, 0.0]]])
    xr = f([[[0.0, 0.0]], [[0.5, 1.0]], [[-3.0, 4.0]]])
    att = np.array([[2.0, -1.0]], np.float32)
    out, lse, _ = oracle.gatv2(rp, ci, xl, xr, att, 0.25)
    # z1 = (1.5, -1) -> act (1.5, -0.25) -> e1 = 3.25 ; z2 = (-2, 2) -> act (-0.5, 2) -> e2 = -3
    e1, e2 = 3.25, -3.0
    w1 = 1.0 / (1.0 + math.exp(e2 - e1))
    np.testing.assert_allclose(out[0, 0], w1 * np.array([0.5, 1.0]) + (1 - w1) * np.array([-3.0, 4.0]),
                               atol=1e-14, rtol=0)


def test_attention_invariants(rng):
    n, H, D = 300, 4, 8
    rp, ci = gen.rmat(21, n, 3000, self_loops=True)
    q, k, v = bf16(rng, (n, H, D)), bf16(rng, (n, H, D)), bf16(rng, (n, H, D))
    ones = gen.f32_to_bf16(np.ones((n, H, D), np.float32))
    out, _, _ = oracle.gt(rp, ci, q, k, ones)
    np.testing.assert_allclose(out, 1.0, atol=1e-13)
    # K = 0: uniform weights -> per-head mean of the neighbours' values,
    # i.e. the LEFT-normalised SpMM of V (a cross-operator identity).
    zeros = np.zeros((n, H, D), np.uint16)
    out, lse, _ = oracle.gt(rp, ci, q, zeros, v)
    ref = oracle.spmm(rp, ci, v.reshape(n, H * D), "left", x_is_bf16=True, want_abs=False)
    np.testing.assert_allclose(out.reshape(n, H * D), ref, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse, np.log(np.diff(rp))[:, None].repeat(H, 1), atol=1e-13)
    # GATv2 with a = 0: same mean of r_j
    att0 = np.zeros((H, D), np.float32)
    out, _, _ = oracle.gatv2(rp, ci, q, v, att0, 0.2)
    np.testing.assert_allclose(out.reshape(n, H * D), ref, atol=1e-13, rtol=0)
    # r_j constant: out = that constant whatever the weights
    c = gen.f32_to_bf16(np.full((n, H, D), 0.375, np.float32))
    att = rng.standard_normal((H, D)).astype(np.float32)
    out, _, _ = oracle.gatv2(rp, ci, q, c, att, 0.2)
    np.testing.assert_allclose(out, 0.375, atol=1e-14)
    # large logits: max subtraction keeps it finite
    big = gen.f32_to_bf16(dec(q).astype(np.float32) * 100)
    out, lse, _ = oracle.gt(rp, ci, big, big, v)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_project_dense_and_closed_forms(rng):
    # Y = X W^T (W output-major, one row per output feature), as a matrix product
    n, fi, fo = 37, 64, 48
    X, W = bf16(rng, (n, fi)), bf16(rng, (fo, fi), std=fi ** -0.5)
    Y, Ya = oracle.project(X, W)
    np.testing.assert_allclose(Y, dec(X) @ dec(W).T, atol=1e-12, rtol=0)
    np.testing.assert_allclose(Ya, np.abs(dec(X)) @ np.abs(dec(W)).T, atol=1e-12, rtol=0)
    # identity weights give the input back exactly
    I = gen.f32_to_bf16(np.eye(fi, dtype=np.float32))
    Y, _ = oracle.project(X, I)
    assert np.array_equal(Y, dec(X))
    # a selector row picks one input feature, scaled: row o = 2 e_{(3o) mod fi}
    S = np.zeros((fo, fi), np.float32)
    S[np.arange(fo), (3 * np.arange(fo)) % fi] = 2.0
    Y, _ = oracle.project(X, gen.f32_to_bf16(S))
    assert np.array_equal(Y, 2.0 * dec(X)[:, (3 * np.arange(fo)) % fi])
    # one input row of ones: each output is the sum of its weight row
    ones = gen.f32_to_bf16(np.ones((1, fi), np.float32))
    Y, _ = oracle.project(ones, W)
    np.testing.assert_allclose(Y[0], dec(W).sum(1), atol=1e-13, rtol=0)


def test_gatv2_f64_agrees_with_bf16_form(rng):
    # float64 inputs that are bf16 values give exactly the bf16 oracle's result
    n, H, D = 60, 2, 16
    rp, ci = gen.rmat(41, n, 500, self_loops=True)
    xl, xr = bf16(rng, (n, H, D)), bf16(rng, (n, H, D))
    att = rng.standard_normal((H, D)).astype(np.float32)
    a = oracle.gatv2(rp, ci, xl, xr, att, 0.2)
    b = oracle.gatv2_f64(rp, ci, dec(xl), dec(xr), att, 0.2)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_gatv2_layer_dense_bruteforce(rng):
    # the layer from node features: l = W_l h_i, r = W_r h_j, then the
    # masked softmax of a^T LeakyReLU(l_i + r_j) over each row's sources
    n, fi, H, D = 36, 32, 2, 8
    A, rp, ci = random_graph(rng, n, 0.25, loops=True)
    X = bf16(rng, (n, fi))
    Wl, Wr = bf16(rng, (H * D, fi), std=fi ** -0.5), bf16(rng, (H * D, fi), std=fi ** -0.5)
    att = (rng.standard_normal((H, D)) / math.sqrt(D)).astype(np.float32)
    out, lse, va = oracle.gatv2_layer(rp, ci, X, Wl, Wr, att, H, D, 0.2)
    L = (dec(X) @ dec(Wl).T).reshape(n, H, D)
    R = (dec(X) @ dec(Wr).T).reshape(n, H, D)
    for h in range(H):
        Z = L[:, None, h, :] + R[None, :, h, :]
        act = np.where(Z > 0, Z, np.float64(np.float32(0.2)) * Z)
        E = act @ att[h].astype(np.float64)
        o, ls = dense_softmax_aggregate(E, A, R[:, h, :])
        np.testing.assert_allclose(out[:, h], o, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse[:, h], ls, atol=1e-12, rtol=0)
        np.testing.assert_allclose(va[:, h], dense_softmax_aggregate(E, A, np.abs(R[:, h, :]))[0],
                                   atol=1e-12, rtol=0)


def test_attention_single_edge_and_empty():
    # row 0 <- {2}; row 1 empty; row 2 <- {0}
    rp, ci = gen.from_edges(3, [2, 0], [0, 2])
    rng = np.random.default_rng(1)
    q, k, v = bf16(rng, (3, 2, 4)), bf16(rng, (3, 2, 4)), bf16(rng, (3, 2, 4))
    out, lse, _ = oracle.gt(rp, ci, q, k, v, scale=0.5)
    assert np.array_equal(out[0], dec(v)[2])
    e = (dec(q)[0] * dec(k)[2]).sum(-1) * 0.5
    np.testing.assert_allclose(lse[0], e, atol=1e-15, rtol=0)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


def test_attention_permutation_equivariance(rng):
    n, H, D = 200, 2, 8
    rp, ci = gen.rmat(31, n, 1500, self_loops=True)
    q, k, v = bf16(rng, (n, H, D)), bf16(rng, (n, H, D)), bf16(rng, (n, H, D))
    pi = rng.permutation(n)
    rows = np.repeat(np.arange(n), np.diff(rp))
    rp2, ci2 = gen.from_edges(n, pi[ci], pi[rows])
    perm = lambda a: (lambda b: (b.__setitem__(pi, a), b)[1])(np.empty_like(a))
    o1, l1, _ = oracle.gt(rp, ci, q, k, v)
    o2, l2, _ = oracle.gt(rp2, ci2, perm(q), perm(k), perm(v))
    np.testing.assert_allclose(o2[pi], o1, atol=1e-13, rtol=0)
    np.testing.assert_allclose(l2[pi], l1, atol=1e-13, rtol=0)
    att = rng.standard_normal((H, D)).astype(np.float32)
    o1, l1, _ = oracle.gatv2(rp, ci, q, k, att)
    o2, l2, _ = oracle.gatv2(rp2, ci2, perm(q), perm(k), att)
    np.testing.assert_allclose(o2[pi], o1, atol=1e-13, rtol=0)


# ----------------------------------------------------------------------------
# Reordering
# ----------------------------------------------------------------------------

def test_degree_sort_matches_stable_argsort():
    rp, ci = gen.rmat(4, 5000, 30000)
    perm = oracle.degree_sort(rp)
    assert np.array_equal(perm, np.argsort(-np.diff(rp), kind="stable"))


def test_rcm_golden():
    g = load_pairs(os.path.join(GOLDEN, "rcm_hand.txt"))
    n = int(g["n"][0][0])
    arcs = np.array([int(t) for t in g["arcs"][0]]).reshape(-1, 2)
    rp, ci = gen.from_edges(n, arcs[:, 0], arcs[:, 1])
    perm = oracle.rcm(rp, ci)
    assert perm.tolist() == [int(t) for t in g["perm"][0]]


def _bandwidth(rp, ci, perm):
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    rows = np.repeat(np.arange(rp.size - 1), np.diff(rp))
    return int(np.abs(inv[rows] - inv[ci]).max()) if ci.size else 0


def test_rcm_relabelled_path_and_grid(rng):
    n = 500
    lab = rng.permutation(n)
    s, d = lab[:-1], lab[1:]
    rp, ci = gen.from_edges(n, np.r_[s, d], np.r_[d, s])
    perm = oracle.rcm(rp, ci)
    assert np.array_equal(np.sort(perm), np.arange(n))
    assert _bandwidth(rp, ci, perm) == 1
    assert _bandwidth(rp, ci, np.arange(n)) > 50          # the random labelling is far from banded
    k = 30
    lab = rng.permutation(k * k)
    src, dst = [], []
    for r in range(k):
        for c in range(k):
            if c + 1 < k:
                src.append(lab[r * k + c]); dst.append(lab[r * k + c + 1])
            if r + 1 < k:
                src.append(lab[r * k + c]); dst.append(lab[(r + 1) * k + c])
    src, dst = np.array(src), np.array(dst)
    rp, ci = gen.from_edges(k * k, np.r_[src, dst], np.r_[dst, src])
    perm = oracle.rcm(rp, ci)
    assert np.array_equal(np.sort(perm), np.arange(k * k))
    assert _bandwidth(rp, ci, perm) <= 2 * k - 1
    assert _bandwidth(rp, ci, np.arange(k * k)) > 10 * k


def test_permute_csr_matches_relabelled_edges(rng):
    n = 700
    rp, ci = gen.rmat(5, n, 5000)
    perm = rng.permutation(n).astype(np.int32)     # perm[new] = old
    inv = np.empty(n, np.int64)
    inv[perm] = np.arange(n)
    rows = np.repeat(np.arange(n), np.diff(rp))
    rp_ref, ci_ref = gen.from_edges(n, inv[ci], inv[rows])
    rp2, ci2 = oracle.permute_csr(rp, ci, perm)
    assert np.array_equal(rp2, rp_ref) and np.array_equal(ci2, ci_ref)


# ----------------------------------------------------------------------------
# WSB layout
# ----------------------------------------------------------------------------

def test_wsb_golden():
    g = load_pairs(os.path.join(GOLDEN, "wsb_hand.txt"))
    n = int(g["n"][0][0])
    src, dst = [], []
    for v in g["row"]:
        for s in v[1:]:
            src.append(int(s)); dst.append(int(v[0]))
    rp, ci = gen.from_edges(n, src, dst)
    wp, tc, tb = oracle.wsb_build(rp, ci)
    assert wp.tolist() == [int(t) for t in g["win_ptr"][0]]
    assert tc.shape[0] == len(g["block"])
    for b, v in enumerate(g["block"]):
        bar = v.index("|")
        cols = [int(t) for t in v[:bar]]
        bits = [int(t) for t in v[bar + 1:]]
        assert tc[b].tolist() == cols
        w = [0, 0]
        for t in bits:
            w[t // 64] |= 1 << (t % 64)
        assert [int(tb[b, 0]), int(tb[b, 1])] == w


def test_wsb_bijection(rng):
    rp, ci = gen.cluster(8, 64 * 10, 64, 0.5, 0.01, self_loops=True)
    n = rp.size - 1
    wp, tc, tb = oracle.wsb_build(rp, ci)
    got = set()
    for w in range(wp.size - 1):
        cols_seen = tc[wp[w]:wp[w + 1]].ravel()
        ncols = len(set(ci[rp[16 * w]:rp[min(16 * w + 16, n)]].tolist()))
        assert np.all(np.diff(cols_seen[:ncols]) > 0)               # sorted distinct
        assert np.all(cols_seen[ncols:] == 0)                         # pads are column 0
        for b in range(wp[w], wp[w + 1]):
            for t in range(128):
                if (int(tb[b, t // 64]) >> (t % 64)) & 1:
                    r, c = divmod(t, 8)
                    assert (b - wp[w]) * 8 + c < ncols                # no bit on a pad
                    got.add((16 * w + r, int(tc[b, c])))
    rows = np.repeat(np.arange(n), np.diff(rp))
    assert got == set(zip(rows.tolist(), ci.tolist()))


# ----------------------------------------------------------------------------
# backward passes: adjoint identities against the (pinned) forward oracle,
# automatic differentiation of dense fp64 formulations, closed forms
# ----------------------------------------------------------------------------

def _dot(a, b):
    return float(np.sum(np.asarray(a, np.float64) * np.asarray(b, np.float64)))


@pytest.mark.parametrize("norm", ["none", "left", "right", "both"])
@pytest.mark.parametrize("weighted", [False, True])
def test_spmm_backward_adjoint(rng, norm, weighted):
    """<A_norm X, dY> = <X, A_norm^T dY> for random X, dY: a dropped weight,
    a transposed index or a wrong degree breaks the identity."""
    n, nc, F = 70, 90, 5
    src = rng.integers(0, nc, 600)
    dst = rng.integers(0, n, 600)
    keep = np.unique(dst.astype(np.int64) * nc + src)        # sorted by (row, column), no duplicates
    rp = np.zeros(n + 1, np.int32)
    np.cumsum(np.bincount(keep // nc, minlength=n), out=rp[1:])
    ci = (keep % nc).astype(np.int32)
    ev = rng.standard_normal(ci.size).astype(np.float32) if weighted else None
    X = rng.standard_normal((nc, F)).astype(np.float32)
    dY = rng.standard_normal((n, F)).astype(np.float32)
    Y, _ = oracle.spmm(rp, ci, X, norm, edge_val=ev, n_cols=nc)
    dX, dXa = oracle.spmm_backward(rp, ci, dY, norm, edge_val=ev, n_cols=nc)
    lhs, rhs = _dot(Y, dY), _dot(X, dX)
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)), (lhs, rhs)
    assert np.all(dXa >= np.abs(dX) - 1e-12)
    # a column that no row uses gets no gradient
    used = np.zeros(nc, bool)
    used[ci] = True
    assert np.all(dX[~used] == 0)


@pytest.mark.parametrize("norm", ["none", "both"])
def test_spmm_backward_column_selection(rng, norm):
    """Selected columns reproduce the full result's rows exactly (same terms in
    the same order), in the order given; repeated or out-of-range columns fail."""
    rp, ci = gen.rmat(24, 800, 12000)
    dY = rng.standard_normal((800, 7)).astype(np.float32)
    full, fa = oracle.spmm_backward(rp, ci, dY, norm)
    deg_out = np.bincount(ci, minlength=800)
    cols = np.r_[rng.permutation(800)[:60], np.argsort(-deg_out)[:5], np.nonzero(deg_out == 0)[0][:3]]
    cols = np.array(list(dict.fromkeys(cols.tolist())), np.int32)
    part, pa = oracle.spmm_backward(rp, ci, dY, norm, cols=cols)
    assert np.array_equal(part, full[cols]) and np.array_equal(pa, fa[cols])
    for bad in ([3, 3], [800], [-1]):
        with pytest.raises(RuntimeError):
            oracle.spmm_backward(rp, ci, dY, norm, cols=np.array(bad, np.int32))


@pytest.mark.parametrize("op", ["sum", "mean", "max", "min"])
def test_reduce_backward_adjoint(rng, op):
    """For fixed selected sources the reductions are linear in X, so
    <reduce(X), dY> = <X, dX> holds exactly for every op; max / min route each
    gradient element to the source the forward selected."""
    n, p = 60, 0.1
    A, rp, ci = random_graph(rng, n, p)
    F = 4
    X = rng.standard_normal((n, F)).astype(np.float32)
    dY = rng.standard_normal((n, F)).astype(np.float32)
    Y, arg, _ = oracle.reduce(rp, ci, X, op)
    dX, _ = oracle.reduce_backward(rp, ci, dY, op, arg=arg if op in ("max", "min") else None)
    lhs, rhs = _dot(Y, dY), _dot(X, dX)
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)), (lhs, rhs)


def test_reduce_max_backward_autograd(rng):
    """Dense masked maximum differentiated by torch (distinct values, so the
    maximum is unique): the gradient reaches exactly the selected source."""
    torch = pytest.importorskip("torch")
    n, F = 30, 3
    A, rp, ci = random_graph(rng, n, 0.2)
    X = rng.permutation(n * F).reshape(n, F).astype(np.float32) / 7.0
    dY = rng.standard_normal((n, F)).astype(np.float32)
    for op in ("max", "min"):
        Y, arg, _ = oracle.reduce(rp, ci, X, op)
        dX, _ = oracle.reduce_backward(rp, ci, dY, op, arg=arg)
        Xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
        mask = torch.tensor(A)
        fill = -math.inf if op == "max" else math.inf
        M = torch.where(mask[:, :, None], Xt[None, :, :], torch.tensor(fill, dtype=torch.float64))
        red = M.amax(dim=1) if op == "max" else M.amin(dim=1)
        has = mask.any(dim=1)[:, None]
        red = torch.where(has, red, torch.zeros_like(red))
        (red * torch.tensor(dY, dtype=torch.float64)).sum().backward()
        np.testing.assert_allclose(dX, Xt.grad.numpy(), atol=1e-12, rtol=0)


def _dense_attention_grads(torch, A, E_fn, V, dO):
    """Autograd of sum(dO * out) with out_i = sum_j softmax_j(E_ij) V_j over the
    entries of A (rows without entries give 0)."""
    E = E_fn()
    mask = torch.tensor(A)
    Em = torch.where(mask, E, torch.tensor(-math.inf, dtype=torch.float64))
    has = mask.any(dim=1, keepdim=True)
    P = torch.softmax(torch.where(has, Em, torch.zeros_like(Em)), dim=1)
    P = torch.where(mask, P, torch.zeros_like(P))
    out = P @ V
    (out * dO).sum().backward()


def test_gt_backward_autograd(rng):
    torch = pytest.importorskip("torch")
    n, H, D = 36, 2, 8
    A, rp, ci = random_graph(rng, n, 0.25, loops=True)
    A[5, :] = False                                   # one row without entries
    rp, ci = gen.from_edges(n, *np.nonzero(A)[::-1])
    q, k, v = bf16(rng, (n, H, D)), bf16(rng, (n, H, D)), bf16(rng, (n, H, D))
    dO = rng.standard_normal((n, H, D)).astype(np.float32)
    dq, dk, dv, mq, mk, mv = oracle.gt_backward(rp, ci, q, k, v, dO)
    for g, m in ((dq, mq), (dk, mk), (dv, mv)):      # error scales bound the values
        assert np.all(m >= np.abs(g) * (1 - 1e-12))
    for h in range(H):
        Q, K, V = (torch.tensor(dec(x)[:, h], requires_grad=True) for x in (q, k, v))
        _dense_attention_grads(torch, A, lambda: (Q @ K.T) / math.sqrt(D), V,
                               torch.tensor(dO[:, h], dtype=torch.float64))
        np.testing.assert_allclose(dq[:, h], Q.grad.numpy(), atol=1e-11, rtol=0)
        np.testing.assert_allclose(dk[:, h], K.grad.numpy(), atol=1e-11, rtol=0)
        np.testing.assert_allclose(dv[:, h], V.grad.numpy(), atol=1e-11, rtol=0)


def test_gatv2_backward_autograd(rng):
    torch = pytest.importorskip("torch")
    n, H, D = 32, 2, 6
    A, rp, ci = random_graph(rng, n, 0.25, loops=True)
    xl, xr = bf16(rng, (n, H, D)), bf16(rng, (n, H, D))
    xl[0, 0, :3] = gen.f32_to_bf16(-gen.bf16_to_f32(xr[0, 0, :3]))   # z = 0 exactly on a self loop
    att = rng.standard_normal((H, D)).astype(np.float32)
    dO = rng.standard_normal((n, H, D)).astype(np.float32)
    dl, dr, da, ml, mr, ma = oracle.gatv2_backward(rp, ci, xl, xr, att, dO, 0.2)
    for g, m in ((dl, ml), (dr, mr), (da, ma)):
        assert np.all(m >= np.abs(g) * (1 - 1e-12))
    slope = float(np.float32(0.2))
    for h in range(H):
        Lt, Rt = (torch.tensor(dec(x)[:, h], requires_grad=True) for x in (xl, xr))
        at = torch.tensor(att[h], dtype=torch.float64, requires_grad=True)

        def E():
            Z = Lt[:, None, :] + Rt[None, :, :]
            return torch.nn.functional.leaky_relu(Z, slope) @ at
        _dense_attention_grads(torch, A, E, Rt, torch.tensor(dO[:, h], dtype=torch.float64))
        np.testing.assert_allclose(dl[:, h], Lt.grad.numpy(), atol=1e-11, rtol=0)
        np.testing.assert_allclose(dr[:, h], Rt.grad.numpy(), atol=1e-11, rtol=0)
        np.testing.assert_allclose(da[h], at.grad.numpy(), atol=1e-11, rtol=0)


def test_attention_backward_closed_forms(rng):
    """Single-entry rows: alpha = 1, so only the value path carries gradient
    (dq = dk = 0, dv_j = sum of dO over the rows j feeds).  Uniform weights
    (K = 0, or a = 0): the value gradient is the mean-SpMM backward of dO."""
    n, H, D = 50, 2, 4
    src = rng.integers(0, n, n)
    rp, ci = gen.from_edges(n, src, np.arange(n))
    q, k, v = bf16(rng, (n, H, D)), bf16(rng, (n, H, D)), bf16(rng, (n, H, D))
    dO = rng.standard_normal((n, H, D)).astype(np.float32)
    dq, dk, dv, *_ = oracle.gt_backward(rp, ci, q, k, v, dO)
    assert np.all(dq == 0) and np.all(dk == 0)
    expect = np.zeros((n, H, D))
    np.add.at(expect, src, dO.astype(np.float64))
    np.testing.assert_allclose(dv, expect, atol=1e-12, rtol=0)

    A, rp, ci = random_graph(rng, n, 0.15, loops=True)
    zero = np.zeros((n, H, D), np.uint16)
    ref, _ = oracle.spmm_backward(rp, ci, dO.reshape(n, H * D), "left")
    _, _, dv, *_ = oracle.gt_backward(rp, ci, q, zero, v, dO)
    np.testing.assert_allclose(dv.reshape(n, H * D), ref, atol=1e-12, rtol=0)
    _, dr, _, *_ = oracle.gatv2_backward(rp, ci, q, v, np.zeros((H, D), np.float32), dO, 0.2)
    np.testing.assert_allclose(dr.reshape(n, H * D), ref, atol=1e-12, rtol=0)


# ----------------------------------------------------------------------------
# dot-aggr (reordering micro-benchmark): dense brute force, closed forms,
# one-hot class counts, permutation equivariance
# ----------------------------------------------------------------------------

def test_dot_aggr_dense_brute_force(rng):
    """y = row sums of A o (X X^T): the Gram matrix masked by the adjacency."""
    for n, D, p in ((1, 3, 1.0), (17, 5, 0.3), (40, 33, 0.15), (64, 1, 0.5)):
        A, rp, ci = random_graph(rng, n, p, loops=True)
        X = rng.standard_normal((n, D)).astype(np.float32)
        Xd = X.astype(np.float64)
        G = Xd @ Xd.T
        want = (A * G).sum(axis=1)
        want_abs = (A * (np.abs(Xd) @ np.abs(Xd).T)).sum(axis=1)
        y, a = oracle.dot_aggr(rp, ci, X)
        np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(a, want_abs, rtol=1e-12, atol=0)


def test_dot_aggr_ones_and_one_hot(rng):
    n, D = 500, 7
    rp, ci = gen.rmat(21, n, 6000)
    deg = np.diff(rp)
    y, a = oracle.dot_aggr(rp, ci, np.ones((n, D), np.float32))
    assert np.array_equal(y, (D * deg).astype(np.float64))
    assert np.array_equal(a, y)
    # one-hot class rows: <x_i, x_j> = [c(i) == c(j)], so y_i counts same-class sources
    c = rng.integers(0, 4, n)
    X = np.zeros((n, 4), np.float32)
    X[np.arange(n), c] = 1.0
    y, _ = oracle.dot_aggr(rp, ci, X)
    rows = np.repeat(np.arange(n), deg)
    want = np.bincount(rows, weights=(c[rows] == c[ci]).astype(np.float64), minlength=n)
    assert np.array_equal(y, want)


def test_dot_aggr_single_feature_and_empty_rows(rng):
    """D = 1: y_i = x_i * (sum of the sources' x); rows without sources give 0."""
    n = 300
    rp, ci = gen.rmat(22, n, 900)          # R-MAT at this density leaves empty rows
    deg = np.diff(rp)
    assert (deg == 0).any()
    X = rng.standard_normal((n, 1)).astype(np.float32)
    y, _ = oracle.dot_aggr(rp, ci, X)
    x = X[:, 0].astype(np.float64)
    want = np.array([x[i] * x[ci[rp[i]:rp[i + 1]]].sum() for i in range(n)])
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-15)
    assert np.all(y[deg == 0] == 0.0)


def test_dot_aggr_permutation_equivariance_and_rows(rng):
    n, D = 400, 12
    rp, ci = gen.rmat(23, n, 5000)
    X = rng.standard_normal((n, D)).astype(np.float32)
    pi = rng.permutation(n)
    rows = np.repeat(np.arange(n), np.diff(rp))
    rp2, ci2 = gen.from_edges(n, pi[ci], pi[rows])
    X2 = np.empty_like(X)
    X2[pi] = X
    y, a = oracle.dot_aggr(rp, ci, X)
    y2, a2 = oracle.dot_aggr(rp2, ci2, X2)
    np.testing.assert_allclose(y2[pi], y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a2[pi], a, rtol=1e-12, atol=0)
    sel = np.sort(rng.choice(n, 50, replace=False)).astype(np.int32)
    ys, _ = oracle.dot_aggr(rp, ci, X, rows=sel)
    assert np.array_equal(ys, y[sel])
