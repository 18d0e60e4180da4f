"""GPU tests of the out-degree count (deg_out[j] = entries with column j),
bit-exact against the oracle's degrees.

The count is observed through the SpMM backward with dY = 1 (F = 1, no
normalisation): dX[j] = sum over the entries of row j of the transposed CSR
= deg_out(j), exact in fp32 below 2^24.  The transpose's row pointers are
the scan of deg_out, so a wrong count also misplaces the transposed rows.

Cases cover the bucketed count (about 1024 column buckets; hub-heavy
buckets split over several workgroups when the ids are not relabelled;
16384-column buckets past 2^24 columns), the atomic kernel (small graphs,
more than 2^26 columns), a col_idx that is not 16-byte aligned, and both
the plan's eager count and a transient plan's count on first use.
"""
import numpy as np
import pytest
import torch

import gen
import graph_neural_network_amd as gnn
import oracle
from gpu_util import host, scaled_err

pytestmark = pytest.mark.gpu


def out_degrees_via_backward(rp, ci, n_cols, plan=False, misalign=False):
    n = rp.size - 1
    row_ptr = torch.from_numpy(rp).cuda()
    if misalign:
        buf = torch.empty(ci.size + 1, dtype=torch.int32, device="cuda")
        buf[1:] = torch.from_numpy(ci).cuda()
        col = buf[1:]
        assert col.data_ptr() % 16 != 0
    else:
        col = torch.from_numpy(ci).cuda()
    csr = gnn.Csr(row_ptr, col, n_cols=n_cols)
    pl = gnn.gnn_plan_create(csr) if plan else None
    dY = torch.ones((n, 1), dtype=torch.float32, device="cuda")
    dX = gnn.gnn_spmm_backward(csr, dY, "none", plan=pl)
    return host(dX)[:, 0]


def check(rp, ci, n_cols, **kw):
    _, ref = oracle.degrees(rp, ci, n_cols)
    got = out_degrees_via_backward(rp, ci, n_cols, **kw)
    assert got.shape == ref.shape
    bad = np.flatnonzero(got != ref.astype(np.float32))
    assert bad.size == 0, (bad[:8], got[bad[:8]], ref[bad[:8]])


def random_rect(seed, n_rows, n_cols, per_row):
    rp = (np.arange(n_rows + 1, dtype=np.int64) * per_row).astype(np.int32)
    ci = (gen.uniform_u64(seed, n_rows * per_row) % np.uint64(n_cols)).astype(np.int32)
    return rp, ci


@pytest.mark.parametrize("plan", [False, True])
def test_rmat_1m_16m(plan):
    w = gen.reduce_rmat(with_x=False)
    print("rmat 1M/16M plan", plan, flush=True)
    check(w.row_ptr, w.col_idx, w.n, plan=plan)


def test_rmat_hub_buckets_split():
    # without relabelling the hubs sit at the smallest ids: the first buckets
    # are many times the average length and are counted by several parts
    rp, ci = gen.rmat(0x5EED0D01, 1 << 20, 12_000_000, relabel=False)
    print("rmat unrelabelled, max bucket share",
          np.bincount(ci >> 10).max() / ci.size, flush=True)
    check(rp, ci, rp.size - 1)


def test_uniform_and_misaligned():
    rp, ci = gen.rmat(0x5EED0D02, 300_000, 3_000_000, 0.25, 0.25, 0.25)
    check(rp, ci, rp.size - 1)
    check(rp, ci, rp.size - 1, misalign=True)


@pytest.mark.parametrize("n_rows,nnz_per_row", [(2000, 9), (1, 1), (40_000, 7)])
def test_small_graphs_atomic_path(n_rows, nnz_per_row):
    rp, ci = random_rect(0x5EED0D03 + n_rows, n_rows, n_rows + 5, nnz_per_row)
    check(rp, ci, n_rows + 5)


def test_wide_buckets_past_2_24_columns():
    # 50,000,000 columns: 16384-column buckets (3052 of them), LDS histogram of 64 KB
    rp, ci = random_rect(0x5EED0D04, 100_000, 50_000_000, 20)
    check(rp, ci, 50_000_000)
    check(rp, ci, 50_000_000, plan=True)


def test_atomic_fallback_past_2_26_columns():
    rp, ci = random_rect(0x5EED0D05, 50_000, 70_000_000, 10)
    check(rp, ci, 70_000_000)


def test_forward_right_norm_uses_transient_count():
    # a plan-less SpMM with the right normalisation counts the degrees on
    # first use: Y = A D_out^-1 X with X = 1 gives sum_j 1 / deg_out(j)
    rp, ci = gen.rmat(0x5EED0D06, 200_000, 2_000_000, self_loops=True)
    n = rp.size - 1
    csr = gnn.Csr(torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda())
    X = torch.ones((n, 1), dtype=torch.float32, device="cuda")
    Y = gnn.gnn_spmm(csr, X, "right")
    ref, mag = oracle.spmm(rp, ci, np.ones((n, 1), np.float32), "right")
    assert scaled_err(host(Y), ref, mag) <= 1e-5
