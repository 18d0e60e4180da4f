"""CPU tests of the host-side pieces: the binding fails loudly without the
library, the benchmark keeps its contract on the command line, and every
benchmark workload names the sources its counter profiles are keyed to."""
import json
import os
import subprocess
import sys

import pytest

import graph_neural_network_amd as gnn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_missing_library_raises(tmp_path):
    saved = gnn._lib
    try:
        gnn._lib = None
        with pytest.raises(ImportError):
            gnn.load_library(str(tmp_path / "libgnn.so"))
    finally:
        gnn._lib = saved


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_bench_workloads_name_existing_sources():
    import bench
    assert set(bench.WORKLOADS) == set(bench.SOURCES)
    csrc = os.path.join(ROOT, "graph_neural_network_amd", "csrc")
    for wl, files in bench.SOURCES.items():
        for f in files:
            assert os.path.exists(os.path.join(csrc, f)), (wl, f)
        assert len(bench.kernel_source_hash(wl)) == 16


def test_committed_profiles_parse():
    prof = os.path.join(ROOT, "profiles")
    names = os.listdir(prof)
    import bench
    for wl in bench.SOURCES:
        d = json.load(open(os.path.join(prof, f"traffic_{wl}.json")))
        assert d["fetch_scale"] > 0 and d["write_scale"] > 0 and d["kernels"]
        assert any(n.endswith(f"_{wl}.md") for n in names), wl


def test_binding_checks_tensor_arguments():
    """The binding rejects wrongly shaped, typed, strided or placed tensors
    before any pointer reaches the library (CPU tensors: nothing runs)."""
    import torch
    import graph_neural_network_amd as gnn
    rp = torch.tensor([0, 1, 2], dtype=torch.int32)
    ci = torch.tensor([0, 1], dtype=torch.int32)
    csr = gnn.Csr(rp, ci)
    with pytest.raises(ValueError, match="X has shape"):
        gnn.gnn_spmm(csr, torch.zeros((1, 8)))                      # fewer rows than columns of A
    with pytest.raises(TypeError, match="dtype"):
        gnn.gnn_spmm(csr, torch.zeros((2, 8), dtype=torch.float64))
    with pytest.raises(ValueError, match="GPU"):
        gnn.gnn_spmm(csr, torch.zeros((2, 8)))
    with pytest.raises(ValueError, match="last dimension"):
        gnn.gnn_reduce(csr, torch.zeros((8, 2)).t())
    with pytest.raises(TypeError, match="arg has dtype"):
        gnn.gnn_reduce(csr, torch.zeros((2, 8)), "max", arg=torch.zeros((2, 8)))
    q = torch.zeros((2, 2, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k has shape"):
        gnn.gnn_gt_fused(csr, q, torch.zeros((2, 2, 16), dtype=torch.bfloat16), q)
    with pytest.raises(TypeError, match="v has dtype"):
        gnn.gnn_gt_fused(csr, q, q, q.float())
    with pytest.raises(ValueError, match="contiguous"):
        gnn.gnn_gt_fused(csr, torch.zeros((2, 32, 2), dtype=torch.bfloat16).transpose(1, 2), q, q)
    with pytest.raises(ValueError, match="att has shape"):
        gnn.gnn_gatv2_fused(csr, q, q, torch.zeros((2, 16)))
    with pytest.raises(ValueError, match="lse has shape"):
        gnn.gnn_gt_backward(csr, q, q, q, torch.zeros((2, 2, 32)), torch.zeros((2, 3)), torch.zeros((2, 2, 32)))
    with pytest.raises(TypeError, match="q has dtype"):
        gnn.gnn_gt_backward_block16(csr, q.float(), q, q, torch.zeros((2, 2, 32)), torch.zeros((2, 2)),
                                    torch.zeros((2, 2, 32)))
    with pytest.raises(TypeError, match="edge_val"):
        gnn.Csr(rp, ci, edge_val=torch.ones(3))
