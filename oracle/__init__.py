"""ORACLE — test infrastructure, not part of the library.

Plain fp64 CPU implementation (``oracle.c``) of what the aggregation kernels
compute.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg import this module; the library's own code path never does.

Every function here is a thin ctypes marshaller over ``liboracle.so``;
the arithmetic is in ``oracle.c``, which cites the passage each function
follows.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

NORM = {"none": 0, "left": 1, "right": 2, "both": 3}
OP = {"sum": 0, "mean": 1, "max": 2, "min": 3}


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (plain C, OpenMP over rows, no fast-math)."""
    import subprocess

    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-fno-fast-math",
           os.path.join(_HERE, "oracle.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i32, i64, vp, f32, ci = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    lib.oracle_degrees.argtypes = [i32, i32, vp, vp, vp, vp]
    lib.oracle_spmm.argtypes = [i32, i32, vp, vp, vp, ci, vp, ci, i32, i64, i64, vp, vp, vp]
    lib.oracle_reduce.argtypes = [i32, vp, vp, vp, i32, i64, ci, i64, vp, vp, vp, vp]
    lib.oracle_gatv2.argtypes = [i32, vp, vp, vp, vp, vp, i32, i32, f32, i64, vp, vp, vp, vp]
    lib.oracle_gt.argtypes = [i32, vp, vp, vp, vp, vp, i32, i32, f32, i64, vp, vp, vp, vp]
    lib.oracle_gatv2_f64.argtypes = [i32, vp, vp, vp, vp, vp, i32, i32, f32, i64, vp, vp, vp, vp]
    lib.oracle_project.argtypes = [i64, i32, vp, i32, vp, vp, vp]
    lib.oracle_degree_sort.argtypes = [i32, vp, vp]
    lib.oracle_rcm.argtypes = [i32, vp, vp, vp]
    lib.oracle_permute_csr.argtypes = [i32, vp, vp, vp, vp, vp]
    lib.oracle_wsb_build.argtypes = [i32, vp, vp, vp, vp, vp, vp]
    lib.oracle_spmm_backward.argtypes = [i32, i32, vp, vp, vp, ci, vp, i32, vp, vp]
    lib.oracle_spmm_backward_cols.argtypes = [i32, i32, vp, vp, vp, ci, vp, i32, i64, vp, vp, vp]
    lib.oracle_reduce_backward.argtypes = [i32, i32, vp, vp, ci, vp, vp, i32, vp, vp]
    lib.oracle_gt_backward.argtypes = [i32, i32, vp, vp, vp, vp, vp, i32, i32, f32, vp, vp, vp, vp, vp,
                                       vp, vp]
    lib.oracle_gatv2_backward.argtypes = [i32, i32, vp, vp, vp, vp, vp, i32, i32, f32, vp, vp, vp, vp,
                                          vp, vp, vp]
    lib.oracle_dot_aggr.argtypes = [i32, vp, vp, vp, i32, i64, i64, vp, vp, vp]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dt)


def _rc(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} returned {rc}")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_threads(n: int) -> None:
    """OpenMP threads of the following oracle calls."""
    _load().oracle_set_threads(int(n))


def _rows(rows, n):
    if rows is None:
        return None, n
    r = np.ascontiguousarray(rows, np.int32)
    return r, r.size


def degrees(row_ptr, col_idx, n_cols=None):
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    n = rp.size - 1
    n_cols = n if n_cols is None else n_cols
    din = np.empty(n, np.int32)
    dout = np.empty(n_cols, np.int32)
    _rc(_load().oracle_degrees(n, n_cols, _p(rp), _p(ci), _p(din), _p(dout)), "degrees")
    return din, dout


def spmm(row_ptr, col_idx, X, norm="none", edge_val=None, rows=None, n_cols=None,
         x_is_bf16=False, want_abs=True):
    """Y [n_sel, F] fp64 (and |.|-sum) of Y = A_norm X.  X is float32, or uint16 bf16 bits."""
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    n = rp.size - 1
    X = np.ascontiguousarray(X)
    if x_is_bf16:
        assert X.dtype == np.uint16
    else:
        X = np.ascontiguousarray(X, np.float32)
    F = X.shape[1]
    n_cols = X.shape[0] if n_cols is None else n_cols
    r, ns = _rows(rows, n)
    Y = np.empty((ns, F), np.float64)
    A = np.empty((ns, F), np.float64) if want_abs else None
    ev = _c(edge_val, np.float32)
    _rc(_load().oracle_spmm(n, n_cols, _p(rp), _p(ci), _p(ev), NORM[norm], _p(X), int(x_is_bf16),
                            F, F, ns, _p(r), _p(Y), _p(A)), "spmm")
    return (Y, A) if want_abs else Y


def reduce(row_ptr, col_idx, X, op, rows=None, want_abs=True):
    """(Y fp64 [n_sel, F], arg int32 [n_sel, F], Yabs)."""
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    n = rp.size - 1
    X = np.ascontiguousarray(X, np.float32)
    F = X.shape[1]
    r, ns = _rows(rows, n)
    Y = np.empty((ns, F), np.float64)
    arg = np.empty((ns, F), np.int32)
    A = np.empty((ns, F), np.float64) if want_abs else None
    _rc(_load().oracle_reduce(n, _p(rp), _p(ci), _p(X), F, F, OP[op], ns, _p(r), _p(Y), _p(arg),
                              _p(A)), "reduce")
    return Y, arg, A


def gatv2(row_ptr, col_idx, xl, xr, att, slope=0.2, rows=None):
    """(out [n_sel,H,D], lse [n_sel,H], vabs [n_sel,H,D]) in fp64; xl, xr bf16 bits [n,H,D]."""
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    n = rp.size - 1
    xl, xr = _c(xl, np.uint16), _c(xr, np.uint16)
    att = _c(att, np.float32)
    H, D = xl.shape[1], xl.shape[2]
    r, ns = _rows(rows, n)
    out = np.empty((ns, H, D), np.float64)
    lse = np.empty((ns, H), np.float64)
    va = np.empty((ns, H, D), np.float64)
    _rc(_load().oracle_gatv2(n, _p(rp), _p(ci), _p(xl), _p(xr), _p(att), H, D, slope, ns, _p(r),
                             _p(out), _p(lse), _p(va)), "gatv2")
    return out, lse, va


def gatv2_f64(row_ptr, col_idx, xl, xr, att, slope=0.2, rows=None):
    """As gatv2, from float64 per-vertex vectors xl [n_rows,H,D], xr [n_cols,H,D]."""
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    n = rp.size - 1
    xl, xr = _c(xl, np.float64), _c(xr, np.float64)
    att = _c(att, np.float32)
    H, D = xl.shape[1], xl.shape[2]
    r, ns = _rows(rows, n)
    out = np.empty((ns, H, D), np.float64)
    lse = np.empty((ns, H), np.float64)
    va = np.empty((ns, H, D), np.float64)
    _rc(_load().oracle_gatv2_f64(n, _p(rp), _p(ci), _p(xl), _p(xr), _p(att), H, D, slope, ns, _p(r),
                                 _p(out), _p(lse), _p(va)), "gatv2_f64")
    return out, lse, va


def project(X, W, want_abs=True):
    """Y = X W^T in float64 (and sum |x w|) from bf16 bits X [n, f_in], W [f_out, f_in]."""
    X, W = _c(X, np.uint16), _c(W, np.uint16)
    n, fi = X.shape
    fo = W.shape[0]
    assert W.shape[1] == fi
    Y = np.empty((n, fo), np.float64)
    A = np.empty((n, fo), np.float64) if want_abs else None
    _rc(_load().oracle_project(n, fi, _p(X), fo, _p(W), _p(Y), _p(A)), "project")
    return (Y, A) if want_abs else Y


def gatv2_layer(row_ptr, col_idx, X, W_l, W_r, att, H, D, slope=0.2, rows=None):
    """The GATv2 layer from node features: l = X W_l^T, r = X W_r^T taken exactly
    (float64), then the softmax aggregation.  X [n, f_in], W_* [H*D, f_in] bf16
    bits -> (out, lse, vabs) as gatv2."""
    n = np.asarray(row_ptr).size - 1
    L = project(X, W_l, want_abs=False).reshape(-1, H, D)
    R = project(X, W_r, want_abs=False).reshape(-1, H, D)
    return gatv2_f64(row_ptr, col_idx, L[:n], R, att, slope, rows)


def gt(row_ptr, col_idx, q, k, v, scale=0.0, rows=None):
    """(out [n_sel,H,D], lse [n_sel,H], vabs) in fp64; q, k, v bf16 bits [n,H,D]."""
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    n = rp.size - 1
    q, k, v = _c(q, np.uint16), _c(k, np.uint16), _c(v, np.uint16)
    H, D = q.shape[1], q.shape[2]
    r, ns = _rows(rows, n)
    out = np.empty((ns, H, D), np.float64)
    lse = np.empty((ns, H), np.float64)
    va = np.empty((ns, H, D), np.float64)
    _rc(_load().oracle_gt(n, _p(rp), _p(ci), _p(q), _p(k), _p(v), H, D, scale, ns, _p(r), _p(out),
                          _p(lse), _p(va)), "gt")
    return out, lse, va


def degree_sort(row_ptr):
    rp = _c(row_ptr, np.int32)
    n = rp.size - 1
    perm = np.empty(n, np.int32)
    _rc(_load().oracle_degree_sort(n, _p(rp), _p(perm)), "degree_sort")
    return perm


def rcm(row_ptr, col_idx):
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    n = rp.size - 1
    perm = np.empty(n, np.int32)
    _rc(_load().oracle_rcm(n, _p(rp), _p(ci), _p(perm)), "rcm")
    return perm


def permute_csr(row_ptr, col_idx, perm):
    rp, ci, pm = _c(row_ptr, np.int32), _c(col_idx, np.int32), _c(perm, np.int32)
    n = rp.size - 1
    rpo = np.empty(n + 1, np.int32)
    cio = np.empty(ci.size, np.int32)
    _rc(_load().oracle_permute_csr(n, _p(rp), _p(ci), _p(pm), _p(rpo), _p(cio)), "permute_csr")
    return rpo, cio


def wsb_build(row_ptr, col_idx):
    """(win_ptr [n_windows+1], tcb_col [n_tcb, 8], tcb_bits [n_tcb, 2] uint64)."""
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    n = rp.size - 1
    nw = (n + 15) // 16
    wp = np.empty(nw + 1, np.int32)
    nt = ctypes.c_int64(0)
    lib = _load()
    _rc(lib.oracle_wsb_build(n, _p(rp), _p(ci), _p(wp), None, None, ctypes.byref(nt)), "wsb sizes")
    tc = np.empty((nt.value, 8), np.int32)
    tb = np.empty((nt.value, 2), np.uint64)
    _rc(lib.oracle_wsb_build(n, _p(rp), _p(ci), _p(wp), _p(tc), _p(tb), ctypes.byref(nt)), "wsb")
    return wp, tc, tb


# ---------------------------------------------------------------------------
# backward passes
# ---------------------------------------------------------------------------

def spmm_backward(row_ptr, col_idx, dY, norm="none", edge_val=None, n_cols=None, cols=None):
    """(dX fp64 [n_cols, F], |.|-sum) of dX = A_norm^T dY; dY float32 [n_rows, F].
    cols: distinct column ids to evaluate (outputs packed [len(cols), F] in that order)."""
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    n = rp.size - 1
    n_cols = n if n_cols is None else n_cols
    dY = np.ascontiguousarray(dY, np.float32)
    F = dY.shape[1]
    ev = _p(_c(edge_val, np.float32))
    if cols is None:
        dX = np.empty((n_cols, F), np.float64)
        A = np.empty((n_cols, F), np.float64)
        _rc(_load().oracle_spmm_backward(n, n_cols, _p(rp), _p(ci), ev, NORM[norm], _p(dY), F, _p(dX), _p(A)),
            "spmm_backward")
        return dX, A
    c = np.ascontiguousarray(cols, np.int32)
    dX = np.empty((c.size, F), np.float64)
    A = np.empty((c.size, F), np.float64)
    _rc(_load().oracle_spmm_backward_cols(n, n_cols, _p(rp), _p(ci), ev, NORM[norm], _p(dY), F, c.size, _p(c),
                                          _p(dX), _p(A)), "spmm_backward_cols")
    return dX, A


def reduce_backward(row_ptr, col_idx, dY, op, arg=None, n_cols=None):
    """(dX fp64 [n_cols, F], |.|-sum); arg int32 [n_rows, F] for max / min."""
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    n = rp.size - 1
    n_cols = n if n_cols is None else n_cols
    dY = np.ascontiguousarray(dY, np.float32)
    F = dY.shape[1]
    dX = np.empty((n_cols, F), np.float64)
    A = np.empty((n_cols, F), np.float64)
    _rc(_load().oracle_reduce_backward(n, n_cols, _p(rp), _p(ci), OP[op], _p(dY), _p(_c(arg, np.int32)), F,
                                       _p(dX), _p(A)), "reduce_backward")
    return dX, A


def gt_backward(row_ptr, col_idx, q, k, v, dO, scale=0.0):
    """(dq, dk, dv, dq_abs, dk_abs, dv_abs) fp64; q, k, v bf16 bits [n, H, D], dO float32."""
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    n = rp.size - 1
    q, k, v = _c(q, np.uint16), _c(k, np.uint16), _c(v, np.uint16)
    dO = np.ascontiguousarray(dO, np.float32)
    H, D = q.shape[1], q.shape[2]
    nc = k.shape[0]
    outs = [np.empty((n, H, D)), np.empty((nc, H, D)), np.empty((nc, H, D)),
            np.empty((n, H, D)), np.empty((nc, H, D)), np.empty((nc, H, D))]
    _rc(_load().oracle_gt_backward(n, nc, _p(rp), _p(ci), _p(q), _p(k), _p(v), H, D, scale, _p(dO),
                                   *[_p(o) for o in outs]), "gt_backward")
    return tuple(outs)


def gatv2_backward(row_ptr, col_idx, xl, xr, att, dO, slope=0.2):
    """(dxl, dxr, datt, dxl_abs, dxr_abs, datt_abs) fp64; xl, xr bf16 bits [n, H, D]."""
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    n = rp.size - 1
    xl, xr = _c(xl, np.uint16), _c(xr, np.uint16)
    att = np.ascontiguousarray(att, np.float32)
    dO = np.ascontiguousarray(dO, np.float32)
    H, D = xl.shape[1], xl.shape[2]
    nc = xr.shape[0]
    outs = [np.empty((n, H, D)), np.empty((nc, H, D)), np.empty((H, D)),
            np.empty((n, H, D)), np.empty((nc, H, D)), np.empty((H, D))]
    _rc(_load().oracle_gatv2_backward(n, nc, _p(rp), _p(ci), _p(xl), _p(xr), _p(att), H, D, slope, _p(dO),
                                      *[_p(o) for o in outs]), "gatv2_backward")
    return tuple(outs)


def dot_aggr(row_ptr, col_idx, X, rows=None, want_abs=True):
    """(y [n_sel], yabs [n_sel]) in fp64: y_i = sum over row i's sources j of <X[i], X[j]>.
    X float32 [n, D] (rows of the square graph)."""
    rp, ci = _c(row_ptr, np.int32), _c(col_idx, np.int32)
    n = rp.size - 1
    X = np.ascontiguousarray(X, np.float32)
    assert X.ndim == 2 and X.shape[0] == n
    D = X.shape[1]
    r, ns = _rows(rows, n)
    y = np.empty(ns, np.float64)
    a = np.empty(ns, np.float64) if want_abs else None
    _rc(_load().oracle_dot_aggr(n, _p(rp), _p(ci), _p(X), D, D, ns, _p(r), _p(y), _p(a)), "dot_aggr")
    return (y, a) if want_abs else y
