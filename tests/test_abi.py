"""CPU tests of the C ABI: the library loads, exports every symbol that
include/gnn.h declares, and rejects invalid arguments on the host before any
launch (no GPU is touched: every call here fails validation)."""
import ctypes
import os
import re

import pytest

import graph_neural_network_amd as gnn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "gnn.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gnn_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = gnn.load_library()
    names = header_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(gnn.EXPORTS)


def test_status_strings():
    lib = gnn.load_library()
    for code, name in gnn.STATUS.items():
        assert lib.gnn_status_string(code).decode() == name


def fake_csr(n_rows=4, n_cols=4, nnz=4, rp=0x1000, ci=0x2000):
    return gnn._Csr(n_rows, n_cols, nnz, rp, ci, None)


def call(fn, *args):
    lib = gnn.load_library()
    rc = getattr(lib, fn)(*args)
    return rc, lib.gnn_last_error().decode()


P = ctypes.c_void_p
INV, UNS, OVF = 1, 2, 5


@pytest.mark.parametrize("case", [
    ("null csr", lambda: call("gnn_spmm", None, P(8), 0, 4, 4, P(8), 4, 0, None, None), INV),
    ("F=0", lambda: call("gnn_spmm", ctypes.byref(fake_csr()), P(8), 0, 0, 4, P(8), 4, 0, None, None), INV),
    ("ldx<F", lambda: call("gnn_spmm", ctypes.byref(fake_csr()), P(8), 0, 8, 4, P(8), 8, 0, None, None), INV),
    ("bad dtype", lambda: call("gnn_spmm", ctypes.byref(fake_csr()), P(8), 7, 4, 4, P(8), 4, 0, None, None), INV),
    ("bad norm", lambda: call("gnn_spmm", ctypes.byref(fake_csr()), P(8), 0, 4, 4, P(8), 4, 9, None, None), INV),
    ("null Y", lambda: call("gnn_spmm", ctypes.byref(fake_csr()), P(8), 0, 4, 4, None, 4, 0, None, None), INV),
    ("nnz>=2^31", lambda: call("gnn_spmm", ctypes.byref(fake_csr(nnz=2**31)), P(8), 0, 4, 4, P(8), 4, 0, None, None), OVF),
    ("negative rows", lambda: call("gnn_reduce", ctypes.byref(fake_csr(n_rows=-1)), P(8), 0, 4, 4, 0, P(8), 4, None, None, None), INV),
    ("arg with sum", lambda: call("gnn_reduce", ctypes.byref(fake_csr()), P(8), 0, 4, 4, 0, P(8), 4, P(8), None, None), INV),
    ("bad op", lambda: call("gnn_reduce", ctypes.byref(fake_csr()), P(8), 0, 4, 4, 11, P(8), 4, None, None, None), INV),
    ("multi no output", lambda: call("gnn_reduce_multi", ctypes.byref(fake_csr()), P(16), 0, 4, 4, None, None, None, None, None, None, 4, None, None), INV),
    ("multi arg without value", lambda: call("gnn_reduce_multi", ctypes.byref(fake_csr()), P(16), 0, 4, 4, P(16), None, None, P(16), None, None, 4, None, None), INV),
    ("multi ldy<F", lambda: call("gnn_reduce_multi", ctypes.byref(fake_csr()), P(16), 0, 8, 8, P(16), None, None, None, None, None, 4, None, None), INV),
    ("noalloc null plan", lambda: call("gnn_reduce_multi_noalloc", ctypes.byref(fake_csr()), P(16), 0, 4, 4, P(16), None, None, None, None, None, 4, None, None), INV),
    ("noalloc no output", lambda: call("gnn_reduce_multi_noalloc", ctypes.byref(fake_csr()), P(16), 0, 4, 4, None, None, None, None, None, None, 4, None, None), INV),
    ("noalloc null csr", lambda: call("gnn_reduce_multi_noalloc", None, P(16), 0, 4, 4, P(16), None, None, None, None, None, 4, None, None), INV),
    ("gatv2 H=0", lambda: call("gnn_gatv2_fused", ctypes.byref(fake_csr()), P(16), P(16), 1, P(16), 0, 32, ctypes.c_float(0.2), P(16), None, None, None), INV),
    ("gatv2 head of 130 slices", lambda: call("gnn_gatv2_fused", ctypes.byref(fake_csr()), P(16), P(16), 1, P(16), 1, 1040, ctypes.c_float(0.2), P(16), None, None, None), UNS),
    ("gatv2 head of 65 4-byte slices", lambda: call("gnn_gatv2_fused", ctypes.byref(fake_csr()), P(16), P(16), 1, P(16), 2, 130, ctypes.c_float(0.2), P(16), None, None, None), UNS),
    ("gt head of 129 f32", lambda: call("gnn_gt_fused", ctypes.byref(fake_csr()), P(16), P(16), P(16), 0, 2, 129, ctypes.c_float(0), 0, P(16), None, None, None), UNS),
    ("gatv2 H*D overflow", lambda: call("gnn_gatv2_fused", ctypes.byref(fake_csr()), P(16), P(16), 1, P(16), 2**28, 16, ctypes.c_float(0.2), P(16), None, None, None), OVF),
    ("gt H*D overflow", lambda: call("gnn_gt_fused", ctypes.byref(fake_csr()), P(16), P(16), P(16), 1, 2**28, 16, ctypes.c_float(0), 0, P(16), None, None, None), OVF),
    ("gt bad mode", lambda: call("gnn_gt_fused", ctypes.byref(fake_csr()), P(16), P(16), P(16), 1, 8, 64, ctypes.c_float(0), 5, P(16), None, None, None), INV),
    ("gt block16 f32", lambda: call("gnn_gt_fused", ctypes.byref(fake_csr()), P(16), P(16), P(16), 0, 8, 64, ctypes.c_float(0), 1, P(16), None, None, None), UNS),
    ("gt block16 D=48", lambda: call("gnn_gt_fused", ctypes.byref(fake_csr()), P(16), P(16), P(16), 1, 2, 48, ctypes.c_float(0), 1, P(16), None, None, None), UNS),
    ("gt block16 non-square", lambda: call("gnn_gt_fused", ctypes.byref(fake_csr(n_cols=5)), P(16), P(16), P(16), 1, 8, 64, ctypes.c_float(0), 1, P(16), None, None, None), INV),
    ("gt misaligned", lambda: call("gnn_gt_fused", ctypes.byref(fake_csr()), P(18), P(16), P(16), 1, 8, 64, ctypes.c_float(0), 0, P(16), None, None, None), UNS),
    ("reorder non-square", lambda: call("gnn_reorder", ctypes.byref(fake_csr(n_cols=3)), 0, P(8), None, None, None), INV),
    ("reorder null perm", lambda: call("gnn_reorder", ctypes.byref(fake_csr()), 0, None, None, None, None), INV),
    ("reorder one output", lambda: call("gnn_reorder", ctypes.byref(fake_csr()), 0, P(8), P(8), None, None), INV),
    ("reorder bad kind", lambda: call("gnn_reorder", ctypes.byref(fake_csr()), 4, P(8), None, None, None), INV),
    ("spmm bwd null dY", lambda: call("gnn_spmm_backward", ctypes.byref(fake_csr()), None, 4, 4, P(16), 4, 0, None, None), INV),
    ("spmm bwd ldx<F", lambda: call("gnn_spmm_backward", ctypes.byref(fake_csr()), P(16), 8, 8, P(16), 4, 0, None, None), INV),
    ("spmm bwd bad norm", lambda: call("gnn_spmm_backward", ctypes.byref(fake_csr()), P(16), 4, 4, P(16), 4, 7, None, None), INV),
    ("reduce bwd max without arg", lambda: call("gnn_reduce_backward", ctypes.byref(fake_csr()), 2, P(16), 4, 4, None, P(16), 4, None, None), INV),
    ("reduce bwd bad op", lambda: call("gnn_reduce_backward", ctypes.byref(fake_csr()), 9, P(16), 4, 4, None, P(16), 4, None, None), INV),
    ("gt bwd null lse", lambda: call("gnn_gt_backward", ctypes.byref(fake_csr()), P(16), P(16), P(16), 1, 8, 64, ctypes.c_float(0), P(16), None, P(16), P(16), P(16), P(16), None, None), INV),
    ("gt bwd head over 1 KB", lambda: call("gnn_gt_backward", ctypes.byref(fake_csr()), P(16), P(16), P(16), 1, 1, 1024, ctypes.c_float(0), P(16), P(16), P(16), P(16), P(16), P(16), None, None), UNS),
    ("gt bwd head not 16-byte slices", lambda: call("gnn_gt_backward", ctypes.byref(fake_csr()), P(16), P(16), P(16), 1, 8, 20, ctypes.c_float(0), P(16), P(16), P(16), P(16), P(16), P(16), None, None), UNS),
    ("gt bwd misaligned", lambda: call("gnn_gt_backward", ctypes.byref(fake_csr()), P(16), P(16), P(16), 1, 8, 64, ctypes.c_float(0), P(16), P(16), P(20), P(16), P(16), P(16), None, None), UNS),
    ("gatv2 bwd null datt", lambda: call("gnn_gatv2_backward", ctypes.byref(fake_csr()), P(16), P(16), 1, P(16), 4, 32, ctypes.c_float(0.2), P(16), P(16), P(16), P(16), P(16), None, None, None), INV),
    ("gatv2 bwd head over 1 KB", lambda: call("gnn_gatv2_backward", ctypes.byref(fake_csr()), P(16), P(16), 1, P(16), 2, 1024, ctypes.c_float(0.2), P(16), P(16), P(16), P(16), P(16), P(16), None, None), UNS),
    ("gatv2 bwd head not 16-byte slices", lambda: call("gnn_gatv2_backward", ctypes.byref(fake_csr()), P(16), P(16), 0, P(16), 4, 6, ctypes.c_float(0.2), P(16), P(16), P(16), P(16), P(16), P(16), None, None), UNS),
    ("gt bwd H*D overflow, wide heads", lambda: call("gnn_gt_backward", ctypes.byref(fake_csr()), P(16), P(16), P(16), 1, 1 << 20, 256, ctypes.c_float(0), P(16), P(16), P(16), P(16), P(16), P(16), None, None), OVF),
    ("spmm b16 non-square", lambda: call("gnn_spmm_block16", ctypes.byref(fake_csr(n_cols=5)), P(16), 1, 16, 16, P(16), 16, 0, None, None), INV),
    ("spmm b16 F not 16 B", lambda: call("gnn_spmm_block16", ctypes.byref(fake_csr()), P(16), 1, 12, 12, P(16), 12, 0, None, None), UNS),
    ("spmm b16 misaligned", lambda: call("gnn_spmm_block16", ctypes.byref(fake_csr()), P(24), 0, 16, 16, P(16), 16, 0, None, None), UNS),
    ("dot non-square", lambda: call("gnn_dot_aggr", ctypes.byref(fake_csr(n_cols=5)), P(16), 4, 4, 0, 0, P(16), None, None), INV),
    ("dot D=0", lambda: call("gnn_dot_aggr", ctypes.byref(fake_csr()), P(16), 0, 4, 0, 0, P(16), None, None), INV),
    ("dot ldx<D", lambda: call("gnn_dot_aggr", ctypes.byref(fake_csr()), P(16), 8, 4, 0, 0, P(16), None, None), INV),
    ("dot D>1024", lambda: call("gnn_dot_aggr", ctypes.byref(fake_csr()), P(16), 1028, 1028, 0, 0, P(16), None, None), UNS),
    ("dot bad map", lambda: call("gnn_dot_aggr", ctypes.byref(fake_csr()), P(16), 4, 4, 2, 0, P(16), None, None), INV),
    ("dot bad load", lambda: call("gnn_dot_aggr", ctypes.byref(fake_csr()), P(16), 4, 4, 0, 3, P(16), None, None), INV),
    ("dot null y", lambda: call("gnn_dot_aggr", ctypes.byref(fake_csr()), P(16), 4, 4, 0, 0, None, None, None), INV),
    ("dot vec16 D%4", lambda: call("gnn_dot_aggr", ctypes.byref(fake_csr()), P(16), 6, 8, 1, 1, P(16), None, None), INV),
    ("dot vec16 ldx%4", lambda: call("gnn_dot_aggr", ctypes.byref(fake_csr()), P(16), 4, 6, 1, 1, P(16), None, None), INV),
    ("dot vec16 misaligned", lambda: call("gnn_dot_aggr", ctypes.byref(fake_csr()), P(20), 4, 4, 0, 1, P(16), None, None), INV),
    ("dot edge values", lambda: call("gnn_dot_aggr", ctypes.byref(gnn._Csr(4, 4, 4, 0x1000, 0x2000, 0x3000)), P(16), 4, 4, 0, 0, P(16), None, None), INV),
    ("b16 bwd non-square", lambda: call("gnn_gt_backward_block16", ctypes.byref(fake_csr(n_cols=5)), P(16), P(16), P(16), 8, 64, 0.0, P(16), P(16), P(16), P(16), P(16), P(16), None, None), INV),
    ("b16 bwd D=96", lambda: call("gnn_gt_backward_block16", ctypes.byref(fake_csr()), P(16), P(16), P(16), 2, 96, 0.0, P(16), P(16), P(16), P(16), P(16), P(16), None, None), UNS),
    ("b16 bwd null dk", lambda: call("gnn_gt_backward_block16", ctypes.byref(fake_csr()), P(16), P(16), P(16), 8, 64, 0.0, P(16), P(16), P(16), P(16), None, P(16), None, None), INV),
    ("b16 bwd H*D overflow", lambda: call("gnn_gt_backward_block16", ctypes.byref(fake_csr()), P(16), P(16), P(16), 2**27, 32, 0.0, P(16), P(16), P(16), P(16), P(16), P(16), None, None), UNS),
    ("gt bwd H*D overflow", lambda: call("gnn_gt_backward", ctypes.byref(fake_csr()), P(16), P(16), P(16), 1, 2**28, 16, ctypes.c_float(0), P(16), P(16), P(16), P(16), P(16), P(16), None, None), OVF),
    ("b16 bwd misaligned", lambda: call("gnn_gt_backward_block16", ctypes.byref(fake_csr()), P(24), P(16), P(16), 8, 64, 0.0, P(16), P(16), P(16), P(16), P(16), P(16), None, None), UNS),
    ("plan null out", lambda: call("gnn_plan_create", ctypes.byref(fake_csr()), None, None, None), INV),
    ("plan bad opts", lambda: call("gnn_plan_create", ctypes.byref(fake_csr()),
                                   ctypes.byref(gnn._PlanOpts(2.0, 0, 0, 0, 0)), None, ctypes.byref(P())), INV),
    ("plan wsb non-square", lambda: call("gnn_plan_create", ctypes.byref(fake_csr(n_cols=9)),
                                         ctypes.byref(gnn._PlanOpts(0, 0, 0, 1, 0)), None, ctypes.byref(P())), INV),
    ("autotune null csr", lambda: call("gnn_plan_autotune", None, P(16), 0, 4, 4, 0, 3, ctypes.byref(gnn._PlanOpts()),
                                       ctypes.byref(ctypes.c_float()), None, None), INV),
    ("autotune reps=0", lambda: call("gnn_plan_autotune", ctypes.byref(fake_csr()), P(16), 0, 4, 4, 0, 0,
                                     ctypes.byref(gnn._PlanOpts()), ctypes.byref(ctypes.c_float()), None, None), INV),
    ("autotune bad op", lambda: call("gnn_plan_autotune", ctypes.byref(fake_csr()), P(16), 0, 4, 4, 7, 3,
                                     ctypes.byref(gnn._PlanOpts()), ctypes.byref(ctypes.c_float()), None, None), INV),
    ("autotune null best", lambda: call("gnn_plan_autotune", ctypes.byref(fake_csr()), P(16), 0, 4, 4, 0, 3, None,
                                        ctypes.byref(ctypes.c_float()), None, None), INV),
    ("autotune ldx<F", lambda: call("gnn_plan_autotune", ctypes.byref(fake_csr()), P(16), 0, 8, 4, 0, 3,
                                    ctypes.byref(gnn._PlanOpts()), ctypes.byref(ctypes.c_float()), None, None), INV),
    ("autotune att null csr", lambda: call("gnn_plan_autotune_attention", None, 1, P(16), P(16), P(16), 1, None, 8, 64, 3,
                                           ctypes.byref(gnn._PlanOpts()), ctypes.byref(ctypes.c_int()),
                                           ctypes.byref(ctypes.c_float()), None, None), INV),
    ("autotune att bad op", lambda: call("gnn_plan_autotune_attention", ctypes.byref(fake_csr()), 5, P(16), P(16), P(16), 1,
                                         None, 8, 64, 3, ctypes.byref(gnn._PlanOpts()), ctypes.byref(ctypes.c_int()),
                                         ctypes.byref(ctypes.c_float()), None, None), INV),
    ("autotune att gatv2 no att", lambda: call("gnn_plan_autotune_attention", ctypes.byref(fake_csr()), 0, P(16), P(16),
                                               None, 1, None, 4, 32, 3, ctypes.byref(gnn._PlanOpts()),
                                               ctypes.byref(ctypes.c_int()), ctypes.byref(ctypes.c_float()), None, None), INV),
    ("autotune att reps=0", lambda: call("gnn_plan_autotune_attention", ctypes.byref(fake_csr()), 1, P(16), P(16), P(16), 1,
                                         None, 8, 64, 0, ctypes.byref(gnn._PlanOpts()), ctypes.byref(ctypes.c_int()),
                                         ctypes.byref(ctypes.c_float()), None, None), INV),
    ("plan bad slot max", lambda: call("gnn_plan_create", ctypes.byref(fake_csr()),
                                       ctypes.byref(gnn._PlanOpts(0, 0, 0, 0, 0, -1)), None, ctypes.byref(P())), INV),
    ("stats null", lambda: call("gnn_plan_stats", None, None, 9), INV),
    ("permute bad F", lambda: call("gnn_permute_rows", P(8), 4, P(8), 0, 0, 4, P(8), 4, None), INV),
    ("copy negative", lambda: call("gnn_copy_bytes", P(8), P(8), -1, None), INV),
], ids=lambda c: c[0])
def test_validation_errors(case):
    name, fn, want = case
    rc, msg = fn()
    assert rc == want, (name, rc, msg)
    assert msg, "a message is recorded"


def test_empty_calls_are_noops():
    lib = gnn.load_library()
    empty = gnn._Csr(0, 0, 0, 0x1000, None, None)
    assert lib.gnn_spmm(ctypes.byref(empty), None, 0, 4, 4, P(8), 4, 0, None, None) == 0
    assert lib.gnn_copy_bytes(None, None, 0, None) == 0
    assert lib.gnn_dot_aggr(ctypes.byref(empty), None, 4, 4, 0, 1, None, None, None) == 0
    assert lib.gnn_plan_destroy(None) == 0
