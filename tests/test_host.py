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
