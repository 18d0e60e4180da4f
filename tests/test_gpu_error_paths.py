"""GPU tests of the error paths: allocation failures injected from the host
at every allocation of a call, and the plan's structure check.

GNN_FAIL_ALLOC=k:tag fails the k-th device allocation after the variable
took that value, before any HIP call; kernels already enqueued by the failing
call run to completion normally.  For k = 1, 2, ... until the call succeeds,
each attempt must return OUT_OF_MEMORY, and the library must stay usable: the
same plan is reused after a failed backward (its transpose is built on the
retry), and the final results match the oracle.

gnn_plan_verify re-samples 64 entries of row_ptr and of col_idx and compares
them with the samples taken when the plan was built: a graph rebuilt in place
under a plan is refused with PLAN_MISMATCH (also by every planned call when
GNN_DEBUG_VALIDATE=1), and restoring the arrays makes the plan valid again.
"""
import os

import numpy as np
import pytest
import torch

import gen
import graph_neural_network_amd as gnn
import oracle
from gpu_util import dev, dev_bf16, dev_csr, host, scaled_err
from test_gpu_backward import TOL_ATT, bwd_err

pytestmark = pytest.mark.gpu
OOM = 3
MISMATCH = 6


def sweep(tag, call, limit=120):
    """Run call() with the k-th allocation failing for k = 1, 2, ... until it
    succeeds; returns (failures, result)."""
    for k in range(1, limit):
        os.environ["GNN_FAIL_ALLOC"] = f"{k}:{tag}"
        try:
            res = call()
        except gnn.GnnError as e:
            assert e.status == OOM, (tag, k, str(e))
            assert "GNN_FAIL_ALLOC" in str(e)
            continue
        finally:
            del os.environ["GNN_FAIL_ALLOC"]
        return k - 1, res
    raise AssertionError(f"{tag}: still failing after {limit} allocations")


@pytest.fixture(scope="module")
def cluster():
    return gen.cluster(0x5EED0400, 64 * 10, 64, 0.5, 0.01, self_loops=True)


def test_plan_creation_every_allocation(cluster):
    rp, ci = cluster
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    X = gen.gauss_f32(0xFEA70400, (n, 64))
    print("plan create sweep", flush=True)
    fails, plan = sweep("plan", lambda: gnn.gnn_plan_create(csr, build_wsb=True, heavy_quantile=0.5,
                                                            chunk_edges=16))
    assert fails >= 8, fails  # degrees, fingerprint, bins, items, WSB layout, temporaries
    Y = gnn.gnn_spmm(csr, dev(X), "both", plan=plan)
    ref, mag = oracle.spmm(rp, ci, X, "both")
    assert scaled_err(host(Y), ref, mag) <= 1e-5
    H, D = 2, 64
    q, k, v = (gen.gauss_bf16(0x4400 + i, (n, H, D)) for i in range(3))
    out, lse = gnn.gnn_gt_fused(csr, dev_bf16(q), dev_bf16(k), dev_bf16(v), mode="block16", plan=plan)
    ro, rl, va = oracle.gt(rp, ci, q, k, v)
    assert scaled_err(host(out), ro, va) <= 2e-2


def test_transient_plans_and_workspace(cluster):
    rp, ci = cluster
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    X = gen.gauss_f32(0xFEA70401, (n, 32))
    fails, out = sweep("multi", lambda: gnn.gnn_reduce_multi(csr, dev(X)))
    assert fails >= 3
    for op in ("sum", "max"):
        ref, arg, mag = oracle.reduce(rp, ci, X, op)
        if op == "sum":
            assert scaled_err(host(out[op]), ref, mag) <= 1e-5
        else:
            assert np.array_equal(host(out[op]), ref.astype(np.float32))
            assert np.array_equal(host(out["argmax"]), arg)


def test_backward_retry_on_the_same_plan(cluster):
    rp, ci = cluster
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    plan = gnn.gnn_plan_create(csr, heavy_quantile=0.5, chunk_edges=16)
    H, D = 2, 32
    q, k, v = (gen.gauss_bf16(0x4500 + i, (n, H, D)) for i in range(3))
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    out, lse = gnn.gnn_gt_fused(csr, dq, dk, dv, plan=plan)
    dO = gen.gauss_f32(0xFEA70402, (n, H, D))
    fails, grads = sweep("gtbwd", lambda: gnn.gnn_gt_backward(csr, dq, dk, dv, out, lse, dev(dO), plan=plan))
    assert fails >= 3  # the transpose, its plan, the statistics buffer, the workspace
    ref = oracle.gt_backward(rp, ci, q, k, v, dO)
    for g, r, m in zip(grads, ref[:3], ref[3:]):
        assert bwd_err(host(g), r, m) <= TOL_ATT


def test_reorder_every_allocation():
    rp, ci = gen.rmat(0x5EED0401, 3000, 30000)
    csr = dev_csr(rp, ci)
    fails, (perm, rp2, ci2) = sweep("rcm", lambda: gnn.gnn_reorder(csr, "rcm"))
    assert fails >= 1
    assert np.array_equal(host(perm), oracle.rcm(rp, ci))


def test_plan_verify_detects_graph_rebuilt_in_place():
    rp, ci = gen.rmat(0x5EED0402, 5000, 60000, self_loops=True)
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    plan = gnn.gnn_plan_create(csr)
    gnn.gnn_plan_verify(plan)
    # another graph of the same size written into the same arrays
    rp_b, ci_b = gen.rmat(0x5EED0403, 5000, 60000, self_loops=True)
    assert rp_b.size == rp.size and ci_b.size == ci.size
    keep_rp, keep_ci = csr.row_ptr.clone(), csr.col_idx.clone()
    csr.row_ptr.copy_(torch.from_numpy(rp_b))
    csr.col_idx.copy_(torch.from_numpy(ci_b))
    with pytest.raises(gnn.GnnError) as e:
        gnn.gnn_plan_verify(plan)
    assert e.value.status == MISMATCH
    X = dev(gen.gauss_f32(0xFEA70403, (n, 16)))
    os.environ["GNN_DEBUG_VALIDATE"] = "1"
    try:
        with pytest.raises(gnn.GnnError) as e:
            gnn.gnn_spmm(csr, X, plan=plan)
        assert e.value.status == MISMATCH
    finally:
        del os.environ["GNN_DEBUG_VALIDATE"]
    # restoring the arrays makes the plan valid again
    csr.row_ptr.copy_(keep_rp)
    csr.col_idx.copy_(keep_ci)
    gnn.gnn_plan_verify(plan)
    Y = gnn.gnn_spmm(csr, X, plan=plan)
    ref, mag = oracle.spmm(rp, ci, host(X), "none")
    assert scaled_err(host(Y), ref, mag) <= 1e-5


def test_planless_calls_do_not_wait_for_the_gpu():
    """A call without a plan builds its transient plan in stream order: it
    returns while earlier work on the stream is still running (a 4-GiB copy,
    about a millisecond), and its result is right once the stream drains."""
    rp, ci = gen.rmat(0x5EED0404, 20000, 300000, self_loops=True)
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    X = gen.gauss_f32(0xFEA70404, (n, 64))
    Xd = dev(X)
    big = torch.empty(1 << 30, dtype=torch.float32, device="cuda")
    big2 = torch.empty_like(big)
    H, D = 4, 32
    xl, xr = gen.gauss_bf16(0x4600, (n, H, D)), gen.gauss_bf16(0x4601, (n, H, D))
    att = gen.gauss_f32(0x4602, (H, D), std=D ** -0.5)
    dl, dr, da = dev_bf16(xl), dev_bf16(xr), dev(att)
    # outputs allocated up front: a new torch allocation may wait for the GPU
    Y0 = torch.empty((n, 64), device="cuda")
    outs = {k: torch.empty((n, 64), device="cuda") for k in ("sum", "mean", "max", "min")}
    outs.update({k: torch.empty((n, 64), dtype=torch.int32, device="cuda") for k in ("argmax", "argmin")})
    o0, l0 = torch.empty((n, H, D), device="cuda"), torch.empty((n, H), device="cuda")
    dX0 = torch.empty((n, 64), device="cuda")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    busy = []
    for call in (lambda: gnn.gnn_spmm(csr, Xd, "both", Y=Y0),
                 lambda: gnn.gnn_reduce_multi(csr, Xd, out=outs),
                 lambda: gnn.gnn_gatv2_fused(csr, dl, dr, da, 0.2, out=o0, lse=l0),
                 lambda: gnn.gnn_spmm_backward(csr, Xd, "both", dX=dX0)):
        gnn.gnn_copy_bytes(big, big2)
        call()
        busy.append(not stream.query())
        torch.cuda.synchronize()
    assert all(busy), busy
    Y = gnn.gnn_spmm(csr, Xd, "both")
    ref, mag = oracle.spmm(rp, ci, X, "both")
    assert scaled_err(host(Y), ref, mag) <= 1e-5
    out, lse = gnn.gnn_gatv2_fused(csr, dl, dr, da, 0.2)
    ro, rl, va = oracle.gatv2(rp, ci, xl, xr, att, 0.2)
    assert scaled_err(host(out), ro, va) <= 1e-4
    dX = gnn.gnn_spmm_backward(csr, Xd, "both")
    rb, mb = oracle.spmm_backward(rp, ci, X, "both")
    assert bwd_err(host(dX), rb, mb) <= 1e-5
