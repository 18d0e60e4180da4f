"""Calls without a plan split long rows too.

A call given no plan builds a transient one in stream order, with no host
read-back: no degree quantile, so every row of more than one chunk (1024
entries) is split into chunks, and the item, chunk and split-row counts stay
on the device (the launches are sized by host bounds and the surplus
workgroups exit).  The graph here has rows of exactly 1024 and 1025 entries,
rows of several chunks and a column hub (a long row of the transpose, which
the backward passes walk), over an R-MAT background.  Every operation that
walks the plan's items is checked against the fp64 oracle, and against the
same call with a plan built with the same split rule (degree threshold at
one chunk), which must agree bit for bit: the work items are the same.
"""
import numpy as np
import pytest
import torch

import gen
import graph_neural_network_amd as gnn
import oracle
from gpu_util import bits_equal_f32, dev, dev_bf16, dev_csr, host, scaled_err

pytestmark = pytest.mark.gpu
TOL = 1e-5
TOL_ATT = 1e-4
SAME_RULE = dict(heavy_quantile=0.5, light_max_deg=32, chunk_edges=1024)
HUB_ROWS = {10: 5000, 11: 1024, 12: 1025, 13: 2049, 14: 3000}
HUB_COL = 20


@pytest.fixture(scope="module")
def graph():
    n = 5000
    rp, ci = gen.rmat(0x5EED0901, n, 40_000, self_loops=True)
    rows = np.repeat(np.arange(n), np.diff(rp))
    keep = ~np.isin(rows, list(HUB_ROWS))
    rng = np.random.default_rng(0x901)
    src, dst = [ci[keep]], [rows[keep]]
    for r, d in HUB_ROWS.items():
        src.append(rng.choice(n, d, replace=False))
        dst.append(np.full(d, r))
    # a column hub: 3000 rows gain an entry in column HUB_COL
    src.append(np.full(3000, HUB_COL))
    dst.append(rng.choice(np.setdiff1d(np.arange(n), list(HUB_ROWS)), 3000, replace=False))
    rp, ci = gen.from_edges(n, np.concatenate(src), np.concatenate(dst))
    deg = np.diff(rp)
    for r, d in HUB_ROWS.items():
        assert deg[r] == d
    assert np.bincount(ci, minlength=n)[HUB_COL] > 2048
    return rp, ci


def _both(fn, csr):
    """The call without a plan, then with a plan of the same split rule."""
    got = fn(None)
    plan = gnn.gnn_plan_create(csr, **SAME_RULE)
    st = gnn.gnn_plan_stats(plan)
    assert st["heavy_rows"] >= 4 and st["heavy_threshold"] == 1024, st
    return got, fn(plan)


def _equal(a, b):
    a = a if isinstance(a, (tuple, list)) else (a,)
    b = b if isinstance(b, (tuple, list)) else (b,)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        if x is None:
            continue
        assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x,
                           y.view(torch.int32) if y.dtype == torch.float32 else y)


@pytest.mark.parametrize("norm,F,dt", [("both", 64, "f32"), ("right", 128, "bf16"), ("none", 40, "f32")])
def test_planless_spmm(graph, norm, F, dt):
    rp, ci = graph
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    if dt == "bf16":
        xb = gen.gauss_bf16(0xFEA70901, (n, F))
        X, Xh = dev_bf16(xb), xb
    else:
        Xh = gen.gauss_f32(0xFEA70901, (n, F))
        X = dev(Xh)
    Y, Yp = _both(lambda pl: gnn.gnn_spmm(csr, X, norm, plan=pl), csr)
    ref, mag = oracle.spmm(rp, ci, Xh, norm, x_is_bf16=dt == "bf16")
    assert scaled_err(host(Y), ref, mag) <= TOL
    _equal(Y, Yp)


@pytest.mark.parametrize("op", ["sum", "mean", "max", "min"])
def test_planless_reduce(graph, op):
    rp, ci = graph
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    Xh = gen.gauss_f32(0xFEA70902, (n, 64))
    X = dev(Xh)
    want_arg = op in ("max", "min")
    (Y, a), (Yp, ap) = _both(lambda pl: gnn.gnn_reduce(csr, X, op, arg=want_arg, plan=pl), csr)
    y, ra, mag = oracle.reduce(rp, ci, Xh, op)
    if want_arg:
        assert bits_equal_f32(host(Y), y)
        assert np.array_equal(host(a), ra)
    else:
        assert scaled_err(host(Y), y, mag) <= TOL
    _equal((Y, a), (Yp, ap))


def test_planless_reduce_multi(graph):
    rp, ci = graph
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    Xh = gen.gauss_f32(0xFEA70903, (n, 128))
    X = dev(Xh)
    out, outp = _both(lambda pl: gnn.gnn_reduce_multi(csr, X, plan=pl), csr)
    for op in ("sum", "mean", "max", "min"):
        y, ra, mag = oracle.reduce(rp, ci, Xh, op)
        if op in ("max", "min"):
            assert bits_equal_f32(host(out[op]), y), op
            assert np.array_equal(host(out["arg" + op]), ra), op
        else:
            assert scaled_err(host(out[op]), y, mag) <= TOL, op
    _equal([out[k] for k in sorted(out)], [outp[k] for k in sorted(out)])


def test_planless_attention_forward(graph):
    rp, ci = graph
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    H, D = 4, 32
    xl, xr = gen.gauss_bf16(0x4901, (n, H, D)), gen.gauss_bf16(0x4902, (n, H, D))
    att = gen.gauss_f32(0x4903, (H, D), std=D ** -0.5)
    (o, l), (op, lp) = _both(lambda pl: gnn.gnn_gatv2_fused(csr, dev_bf16(xl), dev_bf16(xr), dev(att), 0.2,
                                                             plan=pl), csr)
    ro, rl, va = oracle.gatv2(rp, ci, xl, xr, att, 0.2)
    assert scaled_err(host(o), ro, va) <= TOL_ATT
    _equal((o, l), (op, lp))
    H, D = 8, 64
    q, k, v = (gen.gauss_bf16(0x4904 + i, (n, H, D)) for i in range(3))
    (o, l), (op, lp) = _both(lambda pl: gnn.gnn_gt_fused(csr, dev_bf16(q), dev_bf16(k), dev_bf16(v), plan=pl),
                             csr)
    ro, rl, va = oracle.gt(rp, ci, q, k, v)
    assert scaled_err(host(o), ro, va) <= TOL_ATT
    _equal((o, l), (op, lp))


def _bwd_err(got, ref, mag):
    got, ref, mag = (np.asarray(a, np.float64) for a in (got, ref, mag))
    floor = 1e-6 * float(mag.max())
    return float((np.abs(got - ref) / (mag + floor + 1e-300)).max())


def test_planless_backward(graph):
    rp, ci = graph
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    dYh = gen.gauss_f32(0x4910, (n, 64))
    dX, dXp = _both(lambda pl: gnn.gnn_spmm_backward(csr, dev(dYh), "both", plan=pl), csr)
    ref, mag = oracle.spmm_backward(rp, ci, dYh, "both")
    assert _bwd_err(host(dX), ref, mag) <= TOL
    _equal(dX, dXp)
    H, D = 4, 32
    q, k, v = (gen.gauss_bf16(0x4911 + i, (n, H, D)) for i in range(3))
    dO = gen.gauss_f32(0x4914, (n, H, D))

    def gt(pl):
        out, lse = gnn.gnn_gt_fused(csr, dev_bf16(q), dev_bf16(k), dev_bf16(v), plan=pl)
        return gnn.gnn_gt_backward(csr, dev_bf16(q), dev_bf16(k), dev_bf16(v), out, lse, dev(dO), plan=pl)
    g, gp = _both(gt, csr)
    rq, rk, rv, mq, mk, mv = oracle.gt_backward(rp, ci, q, k, v, dO)
    for a, r, m in zip(g, (rq, rk, rv), (mq, mk, mv)):
        assert _bwd_err(host(a), r, m) <= TOL_ATT
    _equal(g, gp)
    att = gen.gauss_f32(0x4915, (H, D), std=0.2)

    def gat(pl):
        out, lse = gnn.gnn_gatv2_fused(csr, dev_bf16(q), dev_bf16(k), dev(att), 0.2, plan=pl)
        return gnn.gnn_gatv2_backward(csr, dev_bf16(q), dev_bf16(k), dev(att), out, lse, dev(dO), 0.2, plan=pl)
    g, gp = _both(gat, csr)
    rl, rr, ra, ml, mr, ma = oracle.gatv2_backward(rp, ci, q, k, att, dO, 0.2)
    for a, r, m in zip(g, (rl, rr, ra), (ml, mr, ma)):
        assert _bwd_err(host(a), r, m) <= TOL_ATT
    # datt adds per-workgroup shares, whose number follows the launch size
    _equal(g[:2], gp[:2])
    assert _bwd_err(host(g[2]), host(gp[2]), ma) <= 1e-6


def test_planless_dot_aggr(graph):
    rp, ci = graph
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    Xh = gen.gauss_f32(0x4920, (n, 64))
    y, yp = _both(lambda pl: gnn.gnn_dot_aggr(csr, dev(Xh), plan=pl), csr)
    ref, mag = oracle.dot_aggr(rp, ci, Xh)
    assert scaled_err(host(y), ref, mag) <= TOL
    _equal(y, yp)


def test_planless_single_split_row():
    """One row of 1025 entries and nothing else: two chunks, bounds at their tightest."""
    n = 1
    rp = np.array([0, 1025], np.int64)
    ci = np.zeros(1025, np.int64)
    csr = dev_csr(rp, ci)
    Xh = gen.gauss_f32(0x4930, (1, 32))
    out = gnn.gnn_reduce_multi(csr, dev(Xh))
    for op in ("sum", "max"):
        y, ra, mag = oracle.reduce(rp, ci, Xh, op)
        if op == "max":
            assert bits_equal_f32(host(out[op]), y) and np.array_equal(host(out["argmax"]), ra)
        else:
            assert scaled_err(host(out[op]), y, mag) <= TOL


def test_block_cache_reuse_across_streams(graph):
    """Temporaries released by a call without a plan are cached and taken
    again by the next call, on the same stream or another one (which first
    waits for the release); results stay exact, and giving the cache back to
    the runtime leaves later calls working."""
    rp, ci = graph
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    X = dev(gen.gauss_f32(0xFEA70905, (n, 96)))
    ref = gnn.gnn_reduce_multi(csr, X, plan=gnn.gnn_plan_create(csr, **SAME_RULE))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for k in range(6):
        st = (s1, s2)[k % 2]
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            outs.append(gnn.gnn_reduce_multi(csr, X, stream=st))
        if k == 3:
            gnn.gnn_release_cached_memory()
    torch.cuda.synchronize()
    for out in outs:
        _equal([out[k] for k in sorted(ref)], [ref[k] for k in sorted(ref)])


def test_block_cache_two_host_threads(graph):
    """Two host threads make calls without a plan on their own streams at the
    same time: the block cache hands a block to one call at a time, and every
    result stays exact."""
    import threading
    rp, ci = graph
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    X = dev(gen.gauss_f32(0xFEA70906, (n, 64)))
    ref = gnn.gnn_reduce_multi(csr, X, plan=gnn.gnn_plan_create(csr, **SAME_RULE))
    torch.cuda.synchronize()
    results, errors = {0: [], 1: []}, []

    def work(tid):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for _ in range(8):
                    results[tid].append(gnn.gnn_reduce_multi(csr, X, stream=st))
            st.synchronize()
        except Exception as e:  # reported below, on the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(t,)) for t in (0, 1)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    torch.cuda.synchronize()
    for tid in (0, 1):
        assert len(results[tid]) == 8
        for out in results[tid]:
            _equal([out[k] for k in sorted(ref)], [ref[k] for k in sorted(ref)])
