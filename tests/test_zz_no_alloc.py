"""The allocation-free gnn_reduce_multi_noalloc against gnn_reduce_multi.

Both run the same kernels; the allocation-free call keeps the split rows'
partial sums and packed (key, index) words in the library's fixed per-GPU
scratch array instead of the plan's workspace, so every output must be
bit-identical (sums are merged in chunk order, so they are deterministic).
Two calls in a row, the second on a smaller graph and width, check that the
array's leftover contents from the first call do not leak into the second.
A plan whose split rows would need more scratch than the array holds is
refused on the host before any launch.
"""
import numpy as np
import pytest
import torch

import gen
import graph_neural_network_amd as gnn
from gpu_util import dev, dev_bf16, dev_csr

pytestmark = pytest.mark.gpu

OPS = ("sum", "mean", "max", "min")
SPLIT = dict(heavy_quantile=0.9, light_max_deg=16, chunk_edges=64)


def _outs(n, F):
    o = {op: torch.empty((n, F), dtype=torch.float32, device="cuda") for op in OPS}
    o["argmax"] = torch.empty((n, F), dtype=torch.int32, device="cuda")
    o["argmin"] = torch.empty((n, F), dtype=torch.int32, device="cuda")
    return o


def _case(seed, n, m, F, dt):
    rp, ci = gen.rmat(0x5EED0100 + seed, n, m)
    csr = dev_csr(rp, ci)
    plan = gnn.gnn_plan_create(csr, **SPLIT)
    st = gnn.gnn_plan_stats(plan)
    assert st["heavy_rows"] > 0 and st["items"] > st["heavy_rows"], st
    if dt == "f32":
        X = dev(gen.gauss_f32(0xFEA70100 + seed, (n, F)))
    else:
        X = dev_bf16(gen.gauss_bf16(0xFEA70100 + seed, (n, F)))
    return csr, plan, X


def _same(a, b):
    for k in a:
        x, y = a[k], b[k]
        if x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), k


def test_noalloc_matches_reduce_multi_twice():
    print("noalloc: 20000-node R-MAT F=128 f32, then 3000-node F=40 bf16", flush=True)
    first = _case(1, 20_000, 400_000, 128, "f32")
    second = _case(2, 3_000, 60_000, 40, "bf16")
    for csr, plan, X in (first, second):
        n, F = csr.n_rows, X.shape[1]
        ref = gnn.gnn_reduce_multi(csr, X, plan=plan)
        out = gnn.gnn_reduce_multi_noalloc(csr, X, _outs(n, F), plan)
        torch.cuda.synchronize()
        _same(ref, out)
    # the larger case again, after the smaller one left its words in the array
    csr, plan, X = first
    ref = gnn.gnn_reduce_multi(csr, X, plan=plan)
    out = gnn.gnn_reduce_multi_noalloc(csr, X, _outs(csr.n_rows, X.shape[1]), plan)
    torch.cuda.synchronize()
    _same(ref, out)


def test_noalloc_subset_outputs_and_no_split_rows():
    csr, plan, X = _case(3, 5_000, 80_000, 64, "f32")
    out = gnn.gnn_reduce_multi_noalloc(csr, X, {"mean": torch.empty((5_000, 64), device="cuda"),
                                                "min": torch.empty((5_000, 64), device="cuda")},
                                       plan, ops=("mean", "min"), args=False)
    ref = gnn.gnn_reduce_multi(csr, X, ops=("mean", "min"), args=False, plan=plan)
    torch.cuda.synchronize()
    _same(ref, out)
    # a plan without split rows needs no scratch at all
    plain = gnn.gnn_plan_create(csr, heavy_quantile=-1.0)
    assert gnn.gnn_plan_stats(plain)["heavy_rows"] == 0
    out = gnn.gnn_reduce_multi_noalloc(csr, X, _outs(5_000, 64), plain)
    ref = gnn.gnn_reduce_multi(csr, X, plan=plain)
    torch.cuda.synchronize()
    _same(ref, out)


def test_noalloc_refuses_oversized_scratch_and_missing_plan():
    # about 1,000 split rows of 40-60 chunks at F = 1024: far beyond the array
    n = 2_000
    deg = 64 * (20 + np.arange(n) % 40)
    dst = np.repeat(np.arange(n), deg)
    src = np.random.default_rng(4).integers(0, n, dst.size)
    rp, ci = gen.from_edges(n, src, dst)
    csr = dev_csr(rp, ci)
    plan = gnn.gnn_plan_create(csr, heavy_quantile=0.5, chunk_edges=64)
    X = torch.zeros((n, 1024), dtype=torch.float32, device="cuda")
    with pytest.raises(gnn.GnnError) as e:
        gnn.gnn_reduce_multi_noalloc(csr, X, _outs(n, 1024), plan)
    assert e.value.status == 5 and "scratch" in str(e.value)
    with pytest.raises(ValueError):
        gnn.gnn_reduce_multi_noalloc(csr, X, _outs(n, 1024), None)
