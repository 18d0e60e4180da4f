"""GPU parity of the fused attention kernels (GATv2, Graph Transformer CSR)
against the fp64 oracle.

Bar (bf16 inputs, fp32 accumulation): max |out - ref| / (sum_j alpha_ij |v_j|)
<= 2e-2, and |lse - ref| <= 2e-2 * max(1, |ref|) (absolute for logsumexp
values of order one; relative where |lse| is so large that the fp32 spacing
alone exceeds 2e-2).  The CSR kernels compute in fp32 with exp2,
so the tests also hold them to a tighter 1e-4 to catch subtle mistakes that
the loose bar would hide.  Special cases: constant values, uniform weights
(K = 0) against gnn_spmm, single-edge rows, empty rows, very large logits.
"""
import numpy as np
import pytest
import torch

import gen
import graph_neural_network_amd as gnn
import oracle
from gpu_util import dev, dev_bf16, dev_csr, host, scaled_err

pytestmark = pytest.mark.gpu
TOL = 2e-2
TIGHT = 1e-4
SMALL_PLAN = dict(light_max_deg=4, chunk_edges=40, heavy_quantile=0.9)


def check(out, lse, ref_out, ref_lse, vabs, tol=TIGHT, rows=None):
    if rows is not None:
        out, lse = out[rows], lse[rows]
    err = scaled_err(out, ref_out, vabs)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(lse), fin), "lse finiteness differs"
    lerr = (float((np.abs(lse[fin] - ref_lse[fin]) / np.maximum(1.0, np.abs(ref_lse[fin]))).max())
            if fin.any() else 0.0)
    assert err <= min(tol, TOL), f"out scaled error {err}"
    assert lerr <= min(tol, TOL), f"lse error {lerr}"
    return err, lerr


@pytest.fixture(scope="module")
def rmat_loops():
    return gen.rmat(0x5EED0200, 20000, 240000, self_loops=True)


def bf16_inputs(n, H, D, seed, count):
    return [gen.gauss_bf16(seed + i, (n, H, D)) for i in range(count)]


# ---------------------------------------------------------------------------
# GATv2
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("H,D,dt", [(4, 32, "bf16"), (2, 64, "bf16"), (8, 16, "bf16"), (1, 8, "bf16"),
                                    (4, 32, "f32"), (2, 16, "f32"), (8, 64, "bf16")])
@pytest.mark.parametrize("planned", [False, True])
def test_gatv2_rmat(rmat_loops, H, D, dt, planned):
    rp, ci = rmat_loops
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    plan = gnn.gnn_plan_create(csr, **SMALL_PLAN) if planned else None
    xl, xr = bf16_inputs(n, H, D, 31, 2)
    att = gen.gauss_f32(33, (H, D), std=(1.0 / D) ** 0.5)
    if dt == "bf16":
        dl, dr = dev_bf16(xl), dev_bf16(xr)
    else:
        dl, dr = dev(gen.bf16_to_f32(xl)), dev(gen.bf16_to_f32(xr))
    out, lse = gnn.gnn_gatv2_fused(csr, dl, dr, dev(att), 0.2, plan=plan)
    ro, rl, va = oracle.gatv2(rp, ci, xl, xr, att, 0.2)
    check(host(out), host(lse), ro, rl, va)


def test_gatv2_special_cases(rmat_loops):
    rp, ci = rmat_loops
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    H, D = 4, 32
    xl, xr = bf16_inputs(n, H, D, 41, 2)
    # r constant: output is that constant
    c = gen.f32_to_bf16(np.full((n, H, D), -1.25, np.float32))
    att = gen.gauss_f32(43, (H, D))
    out, _ = gnn.gnn_gatv2_fused(csr, dev_bf16(xl), dev_bf16(c), dev(att))
    np.testing.assert_allclose(host(out), -1.25, rtol=1e-6)
    # a = 0: uniform weights, out = LEFT-normalised SpMM of r (cross-kernel identity)
    out, lse = gnn.gnn_gatv2_fused(csr, dev_bf16(xl), dev_bf16(xr), dev(np.zeros((H, D), np.float32)))
    sp = gnn.gnn_spmm(csr, dev_bf16(xr.reshape(n, H * D)), "left")
    assert scaled_err(host(out).reshape(n, -1), host(sp), 1.0 + np.abs(host(sp))) <= 1e-5
    np.testing.assert_allclose(host(lse), np.log(np.diff(rp))[:, None].repeat(H, 1), atol=1e-5)


# ---------------------------------------------------------------------------
# Graph Transformer, CSR mode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("H,D,dt", [(8, 64, "bf16"), (4, 32, "bf16"), (2, 128, "bf16"), (8, 128, "bf16"),
                                    (1, 16, "bf16"), (4, 64, "f32"), (2, 32, "f32"), (16, 32, "bf16")])
@pytest.mark.parametrize("planned", [False, True])
def test_gt_csr_rmat(rmat_loops, H, D, dt, planned):
    rp, ci = rmat_loops
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    plan = gnn.gnn_plan_create(csr, **SMALL_PLAN) if planned else None
    q, k, v = bf16_inputs(n, H, D, 51, 3)
    if dt == "bf16":
        dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    else:
        dq, dk, dv = (dev(gen.bf16_to_f32(a)) for a in (q, k, v))
    out, lse = gnn.gnn_gt_fused(csr, dq, dk, dv, plan=plan)
    ro, rl, va = oracle.gt(rp, ci, q, k, v)
    check(host(out), host(lse), ro, rl, va)


def test_gt_special_cases(rmat_loops):
    rp, ci = rmat_loops
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    H, D = 8, 64
    q, k, v = bf16_inputs(n, H, D, 61, 3)
    ones = gen.f32_to_bf16(np.ones((n, H, D), np.float32))
    out, _ = gnn.gnn_gt_fused(csr, dev_bf16(q), dev_bf16(k), dev_bf16(ones))
    np.testing.assert_allclose(host(out), 1.0, rtol=1e-6)
    # K = 0: uniform weights -> gnn_spmm(V, left), per head
    zeros = torch.zeros((n, H, D), dtype=torch.bfloat16, device="cuda")
    out, lse = gnn.gnn_gt_fused(csr, dev_bf16(q), zeros, dev_bf16(v))
    sp = host(gnn.gnn_spmm(csr, dev_bf16(v.reshape(n, H * D)), "left"))
    assert scaled_err(host(out).reshape(n, -1), sp, 1.0 + np.abs(sp)) <= 1e-5
    # logits scaled x 100: the max subtraction keeps everything finite
    big = gen.f32_to_bf16(gen.bf16_to_f32(q) * 100)
    out, lse = gnn.gnn_gt_fused(csr, dev_bf16(big), dev_bf16(big), dev_bf16(v))
    ro, rl, va = oracle.gt(rp, ci, big, big, v)
    assert np.isfinite(host(out)).all() and np.isfinite(host(lse)).all()
    check(host(out), host(lse), ro, rl, va, tol=TOL)


@pytest.mark.parametrize("opts", [dict(light_max_deg=150), dict(light_max_deg=1, chunk_edges=16),
                                  dict(heavy_quantile=-1.0)])
def test_attention_plan_thresholds(rmat_loops, opts):
    """One-slot rows come from the plan's length-sorted list: its bound
    follows the plan's light threshold when that is larger, stops below
    split rows when chunks are small, and covers everything below 128 edges
    when nothing is split."""
    rp, ci = rmat_loops
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    plan = gnn.gnn_plan_create(csr, **opts)
    H, D = 4, 32
    xl, xr = gen.gauss_bf16(41, (n, H, D)), gen.gauss_bf16(42, (n, H, D))
    att = gen.gauss_f32(43, (H, D), std=(1.0 / D) ** 0.5)
    out, lse = gnn.gnn_gatv2_fused(csr, dev_bf16(xl), dev_bf16(xr), dev(att), 0.2, plan=plan)
    ro, rl, va = oracle.gatv2(rp, ci, xl, xr, att, 0.2)
    check(host(out), host(lse), ro, rl, va)
    q, k, v = bf16_inputs(n, H, D, 44, 3)
    out, lse = gnn.gnn_gt_fused(csr, dev_bf16(q), dev_bf16(k), dev_bf16(v), plan=plan)
    ro, rl, va = oracle.gt(rp, ci, q, k, v)
    check(host(out), host(lse), ro, rl, va)


def test_attention_single_edge_and_empty_rows():
    # row 0 <- {2}; row 1 empty; rows 2.. <- {0, 1}; plus a hub row
    n = 3000
    src = [2] + [0, 1] * (n - 3) + list(range(n))
    dst = [0] + [i for i in range(3, n) for _ in (0, 1)] + [2] * n
    rp, ci = gen.from_edges(n, src, dst)
    csr = dev_csr(rp, ci)
    H, D = 8, 64
    q, k, v = bf16_inputs(n, H, D, 71, 3)
    for planned in (False, True):
        plan = gnn.gnn_plan_create(csr, **SMALL_PLAN) if planned else None
        out, lse = gnn.gnn_gt_fused(csr, dev_bf16(q), dev_bf16(k), dev_bf16(v), plan=plan)
        o, l = host(out), host(lse)
        assert np.array_equal(o[0], gen.bf16_to_f32(v)[2]), "single edge: out = v_j exactly"
        assert np.all(o[1] == 0) and np.all(np.isneginf(l[1])), "empty row"
        ro, rl, va = oracle.gt(rp, ci, q, k, v)
        check(o, l, ro, rl, va)
        out, lse = gnn.gnn_gatv2_fused(csr, dev_bf16(q), dev_bf16(k), dev(gen.gauss_f32(3, (H, D))),
                                       plan=plan)
        assert np.array_equal(host(out)[0], gen.bf16_to_f32(k)[2])
        assert np.all(np.isneginf(host(lse)[1]))


# ---------------------------------------------------------------------------
# Full-size workloads, sampled rows
# ---------------------------------------------------------------------------

def sample_rows(rp, k, seed):
    d = np.diff(rp)
    rng = np.random.default_rng(seed)
    return np.unique(np.r_[rng.integers(0, rp.size - 1, k), np.argsort(-d, kind="stable")[:32]]).astype(np.int32)


def test_gatv2_rmat200k_full():
    w = gen.gatv2_rmat()
    csr = dev_csr(w.row_ptr, w.col_idx)
    plan = gnn.gnn_plan_create(csr)
    xl, xr, att = w.arrays["xl"], w.arrays["xr"], w.arrays["att"]
    out, lse = gnn.gnn_gatv2_fused(csr, dev_bf16(xl), dev_bf16(xr), dev(att), 0.2, plan=plan)
    rows = sample_rows(w.row_ptr, 3000, 5)
    ro, rl, va = oracle.gatv2(w.row_ptr, w.col_idx, xl, xr, att, 0.2, rows=rows)
    check(host(out), host(lse), ro, rl, va, rows=rows)


def test_gt_cluster512k_full_csr():
    w = gen.gt_cluster()
    csr = dev_csr(w.row_ptr, w.col_idx)
    plan = gnn.gnn_plan_create(csr)
    q, k, v = w.arrays["q"], w.arrays["k"], w.arrays["v"]
    out, lse = gnn.gnn_gt_fused(csr, dev_bf16(q), dev_bf16(k), dev_bf16(v), plan=plan)
    rows = sample_rows(w.row_ptr, 3000, 6)
    ro, rl, va = oracle.gt(w.row_ptr, w.col_idx, q, k, v, rows=rows)
    check(host(out), host(lse), ro, rl, va, rows=rows)
