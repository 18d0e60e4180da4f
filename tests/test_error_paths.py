"""CPU tests of the library's allocation-failure paths.

GNN_FAIL_ALLOC=k (or k:tag; a new value restarts the count) makes the k-th
device allocation after the variable took its value fail with
GNN_ERR_OUT_OF_MEMORY before any HIP call.  Every entry
point that allocates (plan creation, and every call that builds a transient
plan or takes temporaries) must then return OUT_OF_MEMORY with a message,
without touching the GPU, so these run on a host without one; the pointers
below are never dereferenced.  Entry points that never allocate (projection,
row permutation, copy, the allocation-free reductions) are checked to be
unaffected by the hook on host validation.
"""
import ctypes
import os

import pytest

import graph_neural_network_amd as gnn

P = ctypes.c_void_p
OOM = 3
F = ctypes.c_float


def csr(n=64, nnz=256):
    return ctypes.byref(gnn._Csr(n, n, nnz, 0x1000, 0x2000, None))


CASES = {
    "gnn_plan_create": lambda: ("gnn_plan_create", csr(), ctypes.byref(gnn._PlanOpts()), None, ctypes.byref(P())),
    "gnn_plan_create wsb": lambda: ("gnn_plan_create", csr(), ctypes.byref(gnn._PlanOpts(0, 0, 0, 1, 0)), None,
                                    ctypes.byref(P())),
    "gnn_spmm": lambda: ("gnn_spmm", csr(), P(16), 0, 4, 4, P(16), 4, 3, None, None),
    "gnn_spmm_block16": lambda: ("gnn_spmm_block16", csr(), P(16), 0, 4, 4, P(16), 4, 0, None, None),
    "gnn_reduce": lambda: ("gnn_reduce", csr(), P(16), 0, 4, 4, 2, P(16), 4, P(16), None, None),
    "gnn_reduce_multi": lambda: ("gnn_reduce_multi", csr(), P(16), 0, 4, 4, P(16), P(16), P(16), P(16), P(16),
                                 P(16), 4, None, None),
    "gnn_gatv2_fused": lambda: ("gnn_gatv2_fused", csr(), P(16), P(16), 1, P(16), 4, 32, F(0.2), P(16), P(16),
                                None, None),
    "gnn_gt_fused csr": lambda: ("gnn_gt_fused", csr(), P(16), P(16), P(16), 1, 8, 64, F(0), 0, P(16), P(16),
                                 None, None),
    "gnn_gt_fused block16": lambda: ("gnn_gt_fused", csr(), P(16), P(16), P(16), 1, 8, 64, F(0), 1, P(16), P(16),
                                     None, None),
    "gnn_spmm_backward": lambda: ("gnn_spmm_backward", csr(), P(16), 4, 4, P(16), 4, 0, None, None),
    "gnn_reduce_backward": lambda: ("gnn_reduce_backward", csr(), 0, P(16), 4, 4, None, P(16), 4, None, None),
    "gnn_gatv2_backward": lambda: ("gnn_gatv2_backward", csr(), P(16), P(16), 1, P(16), 4, 32, F(0.2), P(16),
                                   P(16), P(16), P(16), P(16), P(16), None, None),
    "gnn_gt_backward": lambda: ("gnn_gt_backward", csr(), P(16), P(16), P(16), 1, 8, 64, F(0), P(16), P(16),
                                P(16), P(16), P(16), P(16), None, None),
    "gnn_gt_backward_block16": lambda: ("gnn_gt_backward_block16", csr(), P(16), P(16), P(16), 8, 64, 0.0,
                                        P(16), P(16), P(16), P(16), P(16), P(16), None, None),
    "gnn_dot_aggr": lambda: ("gnn_dot_aggr", csr(), P(16), 4, 4, 0, 1, P(16), None, None),
    "gnn_reorder": lambda: ("gnn_reorder", csr(), 1, P(16), P(16), P(16), None),
    "gnn_plan_autotune": lambda: ("gnn_plan_autotune", csr(), P(16), 0, 4, 4, 2, 3, ctypes.byref(gnn._PlanOpts()),
                                  ctypes.byref(F()), None, None),
    "gnn_plan_autotune_attention": lambda: ("gnn_plan_autotune_attention", csr(), 1, P(16), P(16), P(16), 1, None, 8,
                                            64, 3, ctypes.byref(gnn._PlanOpts()), ctypes.byref(ctypes.c_int()),
                                            ctypes.byref(F()), None, None),
}


@pytest.fixture
def fail_first_alloc(request):
    # a fresh value (the tag after the count) restarts the hook's count
    os.environ["GNN_FAIL_ALLOC"] = f"1:{request.node.name}"
    yield
    del os.environ["GNN_FAIL_ALLOC"]


@pytest.mark.parametrize("name", sorted(CASES))
def test_first_allocation_failure_returns_oom(name, fail_first_alloc):
    lib = gnn.load_library()
    fn, *args = CASES[name]()
    rc = getattr(lib, fn)(*args)
    msg = lib.gnn_last_error().decode()
    assert rc == OOM, (name, rc, msg)
    assert "GNN_FAIL_ALLOC" in msg


def test_hook_counts_from_when_the_value_is_set():
    """k = 2: the first allocation of the first call passes (and then, with no
    GPU here, that call fails otherwise); the second allocation fails, the
    third passes again; a new value restarts the count."""
    lib = gnn.load_library()
    fn, *args = CASES["gnn_plan_create"]()
    os.environ["GNN_FAIL_ALLOC"] = "2:count"
    try:
        first = getattr(lib, fn)(*args)          # allocation 1 passes to HIP
        assert first != OOM or "GNN_FAIL_ALLOC" not in lib.gnn_last_error().decode()
        second = getattr(lib, fn)(*args)         # allocation 2 is the injected failure
        assert second == OOM and "GNN_FAIL_ALLOC" in lib.gnn_last_error().decode()
        third = getattr(lib, fn)(*args)          # allocation 3: past the count
        assert "GNN_FAIL_ALLOC" not in lib.gnn_last_error().decode() or third != OOM
        os.environ["GNN_FAIL_ALLOC"] = "1:count"  # a new value restarts the count
        assert getattr(lib, fn)(*args) == OOM
    finally:
        del os.environ["GNN_FAIL_ALLOC"]


def test_non_allocating_calls_ignore_the_hook(fail_first_alloc):
    lib = gnn.load_library()
    # host validation still decides; nothing here would allocate
    assert lib.gnn_copy_bytes(None, None, 0, None) == 0
    assert lib.gnn_permute_rows(P(8), 0, P(8), 0, 4, 4, P(8), 4, None) == 0
    W = (P * 1)(P(16))
    Y = (P * 1)(P(16))
    assert lib.gnn_project(P(16), 0, 32, 32, 1, W, 16, Y, None) == 0
    rc = lib.gnn_reduce_multi_noalloc(csr(), P(16), 0, 4, 4, P(16), None, None, None, None, None, 4, None, None)
    assert rc == 1  # no plan: INVALID_VALUE, not OUT_OF_MEMORY
