"""GPU tests of gnn_plan_autotune_attention: the measured choice of the fused
attention layers' plan knobs (split threshold, chunk size, one-slot bound)
and, for the Graph Transformer, of CSR against block-sparse attention with
its tile threshold (the IO-aware GNN layers paper: appendix D.1 autotuning
parameters; appendix D.3 and section 5, the choice by local density).

On a locally dense cluster graph the block-sparse kernel must win, on a
power-law graph the CSR kernel; whatever wins, the plan built from the
returned options and called in the returned mode must match the oracle
(1e-4 for the fp32-exact CSR path, 2e-2 for BLOCK16, which rounds the
softmax weights to bf16).
"""
import numpy as np
import pytest

import gen
import graph_neural_network_amd as gnn
import oracle
from gpu_util import dev, dev_bf16, dev_csr, host, scaled_err

pytestmark = pytest.mark.gpu


def run_best(csr, res, call):
    o = res["opts"]
    plan = gnn.gnn_plan_create(csr, heavy_quantile=o["heavy_quantile"], chunk_edges=o["chunk_edges"],
                               att_slot_max=o["att_slot_max"], build_wsb=o["build_wsb"],
                               wsb_min_nnz=o["wsb_min_nnz"])
    return call(plan, res["mode"])


@pytest.mark.parametrize("graph,want", [("cluster", "block16"), ("rmat", "csr")])
def test_gt_autotune_picks_by_density(graph, want):
    if graph == "cluster":
        rp, ci = gen.cluster(0x5EED0500, 64 * 2000, 64, 0.5, 0.01, self_loops=True)
    else:
        rp, ci = gen.rmat(0x5EED0501, 100000, 1500000, self_loops=True)
    n = rp.size - 1
    H, D = 4, 64
    q, k, v = (gen.gauss_bf16(0x4700 + i, (n, H, D)) for i in range(3))
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    csr = dev_csr(rp, ci)
    res = gnn.gnn_plan_autotune_attention(csr, "gt", dq, dk, dv, reps=3)
    print(graph, res, flush=True)
    assert res["mode"] == want, res
    assert res["best_ms"] <= res["default_ms"] * 1.05, res
    out, lse = run_best(csr, res, lambda plan, mode: gnn.gnn_gt_fused(csr, dq, dk, dv, mode=mode, plan=plan))
    rows = np.unique(np.r_[np.random.default_rng(1).integers(0, n, 2000),
                           np.argsort(-np.diff(rp), kind="stable")[:16]]).astype(np.int32)
    ro, rl, va = oracle.gt(rp, ci, q, k, v, rows=rows)
    err = scaled_err(host(out)[rows], ro, va)
    assert err <= (2e-2 if res["mode"] == "block16" else 1e-4), err


def test_gatv2_autotune():
    rp, ci = gen.rmat(0x5EED0502, 100000, 1500000, self_loops=True)
    n = rp.size - 1
    H, D = 4, 32
    xl, xr = gen.gauss_bf16(0x4800, (n, H, D)), gen.gauss_bf16(0x4801, (n, H, D))
    att = gen.gauss_f32(0x4802, (H, D), std=D ** -0.5)
    dl, dr, da = dev_bf16(xl), dev_bf16(xr), dev(att)
    csr = dev_csr(rp, ci)
    res = gnn.gnn_plan_autotune_attention(csr, "gatv2", dl, dr, att=da, reps=3)
    print(res, flush=True)
    assert res["mode"] == "csr" and not res["opts"]["build_wsb"]
    assert res["opts"]["att_slot_max"] in (32, 128, 512) and res["opts"]["chunk_edges"] in (256, 1024)
    assert res["best_ms"] <= res["default_ms"] * 1.05, res
    out, lse = run_best(csr, res, lambda plan, mode: gnn.gnn_gatv2_fused(csr, dl, dr, da, 0.2, plan=plan))
    rows = np.unique(np.r_[np.random.default_rng(2).integers(0, n, 2000),
                           np.argsort(-np.diff(rp), kind="stable")[:16]]).astype(np.int32)
    ro, rl, va = oracle.gatv2(rp, ci, xl, xr, att, 0.2, rows=rows)
    assert scaled_err(host(out)[rows], ro, va) <= 1e-4


@pytest.mark.parametrize("slot_max", [1, 16, 4096])
def test_att_slot_max_extremes(slot_max):
    """The one-slot bound at its extremes: every row an item (1), or every
    unsplit row one slot (4096); both attention layers and the GT backward."""
    rp, ci = gen.rmat(0x5EED0503, 8000, 100000, self_loops=True)
    n = rp.size - 1
    H, D = 2, 32
    csr = dev_csr(rp, ci)
    # the one-slot bound never goes below the plan's light bound, so the
    # smallest case lowers that too
    plan = gnn.gnn_plan_create(csr, att_slot_max=slot_max, light_max_deg=1 if slot_max == 1 else 0,
                               heavy_quantile=0.99, chunk_edges=256)
    q, k, v = (gen.gauss_bf16(0x4900 + i, (n, H, D)) for i in range(3))
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    out, lse = gnn.gnn_gt_fused(csr, dq, dk, dv, plan=plan)
    ro, rl, va = oracle.gt(rp, ci, q, k, v)
    assert scaled_err(host(out), ro, va) <= 1e-4
    att = gen.gauss_f32(0x4903, (H, D), std=D ** -0.5)
    o2, _ = gnn.gnn_gatv2_fused(csr, dq, dk, dev(att), 0.2, plan=plan)
    r2, _, v2 = oracle.gatv2(rp, ci, q, k, att, 0.2)
    assert scaled_err(host(o2), r2, v2) <= 1e-4
    dO = gen.gauss_f32(0x4904, (n, H, D))
    grads = gnn.gnn_gt_backward(csr, dq, dk, dv, out, lse, dev(dO), plan=plan)
    from test_gpu_backward import TOL_ATT, bwd_err
    ref = oracle.gt_backward(rp, ci, q, k, v, dO)
    for g, r, m in zip(grads, ref[:3], ref[3:]):
        assert bwd_err(host(g), r, m) <= TOL_ATT
