"""Python binding of libgnn (MI355X / gfx950 GNN aggregation kernels).

Thin ctypes layer: it only marshals torch tensors (device memory) and the
current HIP stream into the C ABI declared in ``include/gnn.h``; every step
of the computation runs in libgnn's HIP kernels.  The function names are the
C names.  There is no CPU fallback: if ``libgnn.so`` is missing or cannot be
loaded, every call raises.

Graph convention: CSR with rows = destinations (row i lists the sources j of
edges j -> i), int32 indices, on the GPU.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgnn.so")

GNN_OK = 0
STATUS = {0: "GNN_OK", 1: "GNN_ERR_INVALID_VALUE", 2: "GNN_ERR_UNSUPPORTED",
          3: "GNN_ERR_OUT_OF_MEMORY", 4: "GNN_ERR_DEVICE", 5: "GNN_ERR_SIZE_OVERFLOW",
          6: "GNN_ERR_PLAN_MISMATCH"}
DTYPE = {"f32": 0, "bf16": 1}
NORM = {"none": 0, "left": 1, "right": 2, "both": 3}
REDUCE_OP = {"sum": 0, "mean": 1, "max": 2, "min": 3}
GT_MODE = {"csr": 0, "block16": 1, "auto": 2}
REORDER = {"degree": 0, "rcm": 1}
DOT_MAP = {"feature": 0, "neighbor": 1}
DOT_LOAD = {"scalar": 0, "vec16": 1}
TUNE_OP = {"spmm": 0, "sum": 1, "multi": 2}

# every symbol include/gnn.h declares
EXPORTS = ("gnn_plan_create", "gnn_plan_destroy", "gnn_plan_stats", "gnn_plan_wsb_export",
           "gnn_spmm", "gnn_reduce", "gnn_reduce_multi", "gnn_gatv2_fused", "gnn_gt_fused", "gnn_reorder",
           "gnn_permute_rows", "gnn_copy_bytes", "gnn_status_string", "gnn_last_error",
           "gnn_spmm_backward", "gnn_reduce_backward", "gnn_gatv2_backward", "gnn_gt_backward",
           "gnn_spmm_block16", "gnn_dot_aggr", "gnn_gt_backward_block16", "gnn_plan_autotune",
           "gnn_reduce_multi_noalloc", "gnn_project", "gnn_plan_verify", "gnn_plan_autotune_attention",
           "gnn_release_cached_memory")


class GnnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")


class _Csr(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int32), ("n_cols", ctypes.c_int32), ("nnz", ctypes.c_int64),
                ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
                ("edge_val", ctypes.c_void_p)]


class _PlanOpts(ctypes.Structure):
    _fields_ = [("heavy_quantile", ctypes.c_float), ("light_max_deg", ctypes.c_int32),
                ("chunk_edges", ctypes.c_int32), ("build_wsb", ctypes.c_int32),
                ("wsb_min_nnz", ctypes.c_int32), ("att_slot_max", ctypes.c_int32),
                ("reserved", ctypes.c_int32 * 3)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libgnn.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libgnn.so not found at {path}; build it with "
                          "`python -m graph_neural_network_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, ci = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_int)
    P = ctypes.POINTER
    sig = {
        "gnn_plan_create": [P(_Csr), P(_PlanOpts), vp, P(vp)],
        "gnn_plan_destroy": [vp],
        "gnn_plan_stats": [vp, P(ctypes.c_int64), i32],
        "gnn_plan_verify": [vp, P(_Csr), vp],
        "gnn_plan_autotune_attention": [P(_Csr), ci, vp, vp, vp, ci, vp, i32, i32, i32, P(_PlanOpts), P(ci),
                                        P(f32), P(f32), vp],
        "gnn_plan_wsb_export": [vp, vp, vp, vp, vp],
        "gnn_spmm": [P(_Csr), vp, ci, i32, i64, vp, i64, ci, vp, vp],
        "gnn_reduce": [P(_Csr), vp, ci, i32, i64, ci, vp, i64, vp, vp, vp],
        "gnn_reduce_multi": [P(_Csr), vp, ci, i32, i64, vp, vp, vp, vp, vp, vp, i64, vp, vp],
        "gnn_reduce_multi_noalloc": [P(_Csr), vp, ci, i32, i64, vp, vp, vp, vp, vp, vp, i64, vp, vp],
        "gnn_gatv2_fused": [P(_Csr), vp, vp, ci, vp, i32, i32, f32, vp, vp, vp, vp],
        "gnn_gt_fused": [P(_Csr), vp, vp, vp, ci, i32, i32, f32, ci, vp, vp, vp, vp],
        "gnn_reorder": [P(_Csr), ci, vp, vp, vp, vp],
        "gnn_permute_rows": [vp, i32, vp, ci, i32, i64, vp, i64, vp],
        "gnn_copy_bytes": [vp, vp, i64, vp],
        "gnn_spmm_backward": [P(_Csr), vp, i32, i64, vp, i64, ci, vp, vp],
        "gnn_spmm_block16": [P(_Csr), vp, ci, i32, i64, vp, i64, ci, vp, vp],
        "gnn_reduce_backward": [P(_Csr), ci, vp, i32, i64, vp, vp, i64, vp, vp],
        "gnn_gatv2_backward": [P(_Csr), vp, vp, ci, vp, i32, i32, f32, vp, vp, vp, vp, vp, vp, vp, vp],
        "gnn_gt_backward": [P(_Csr), vp, vp, vp, ci, i32, i32, f32, vp, vp, vp, vp, vp, vp, vp, vp],
        "gnn_dot_aggr": [P(_Csr), vp, i32, i64, ci, ci, vp, vp, vp],
        "gnn_gt_backward_block16": [P(_Csr), vp, vp, vp, i32, i32, f32, vp, vp, vp, vp, vp, vp, vp, vp],
        "gnn_plan_autotune": [P(_Csr), vp, ci, i32, i64, ci, i32, P(_PlanOpts), P(f32), P(f32), vp],
        "gnn_project": [vp, i32, i32, i64, i32, P(vp), i32, P(vp), vp],
        "gnn_release_cached_memory": [],
        "gnn_status_string": [ci],
        "gnn_last_error": [],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name in ("gnn_status_string", "gnn_last_error") else ci
    _lib = lib
    return lib


def _check(rc: int, where: str):
    if rc != GNN_OK:
        raise GnnError(rc, where, load_library().gnn_last_error().decode())


def _stream(stream=None):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


F32 = (torch.float32,)
FEAT = (torch.float32, torch.bfloat16)


def _need(t, name: str, rows: int, tail: tuple, dtypes: tuple, rows_strided: bool = False):
    """Check a tensor argument before its pointer reaches the library, which
    reads or writes rows [0, rows) at the layout it is told: at least `rows`
    rows, trailing sizes `tail` (None: any), a dtype of `dtypes`; contiguous,
    or (rows_strided) unit stride along the last dimension only.  The device
    is checked apart (_gpu), after every argument's shape."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")
    shape = t.shape
    ok = len(shape) == 1 + len(tail) and shape[0] >= rows
    if ok:
        for i, b in enumerate(tail):
            if b is not None and shape[i + 1] != b:
                ok = False
    if not ok:
        want = "x".join(str(x) for x in (f">={rows}",) + tuple("*" if b is None else b for b in tail))
        raise ValueError(f"{name} has shape {tuple(shape)}; expected [{want}]")
    if rows_strided:
        if len(shape) > 1 and t.stride(-1) != 1:
            raise ValueError(f"{name} must have unit stride along its last dimension")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _gpu(**tensors):
    """Every given tensor (None skipped) must live on a GPU."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DTYPE["f32"]
    if t.dtype == torch.bfloat16:
        return DTYPE["bf16"]
    raise TypeError(f"unsupported feature dtype {t.dtype} (float32 or bfloat16)")


class Csr:
    """A device CSR (rows = destinations).  Keeps the tensors alive."""

    def __init__(self, row_ptr: torch.Tensor, col_idx: torch.Tensor, n_cols: int | None = None,
                 edge_val: torch.Tensor | None = None):
        for name, t in (("row_ptr", row_ptr), ("col_idx", col_idx)):
            if t.dtype != torch.int32 or not t.is_contiguous():
                raise TypeError(f"{name} must be a contiguous int32 tensor")
        if edge_val is not None and (edge_val.dtype != torch.float32 or not edge_val.is_contiguous()
                                     or edge_val.numel() != col_idx.numel()):
            raise TypeError("edge_val must be a contiguous float32 tensor with one value per entry")
        self.row_ptr, self.col_idx, self.edge_val = row_ptr, col_idx, edge_val
        self.n_rows = row_ptr.numel() - 1
        self.n_cols = self.n_rows if n_cols is None else int(n_cols)
        self.nnz = col_idx.numel()
        self._s = _Csr(self.n_rows, self.n_cols, self.nnz, row_ptr.data_ptr(),
                       col_idx.data_ptr() if self.nnz else None,
                       edge_val.data_ptr() if edge_val is not None else None)

    @property
    def ref(self):
        return ctypes.byref(self._s)


class Plan:
    """Owns a gnn_plan*; destroyed with the object (or explicitly)."""

    def __init__(self, handle: int, csr: Csr):
        self.handle = ctypes.c_void_p(handle)
        self.csr = csr

    def destroy(self):
        if self.handle:
            _check(load_library().gnn_plan_destroy(self.handle), "gnn_plan_destroy")
            self.handle = ctypes.c_void_p(None)

    def __del__(self):
        try:
            if self.handle and _lib is not None:
                _lib.gnn_plan_destroy(self.handle)
        except Exception:
            pass


def gnn_plan_create(csr: Csr, heavy_quantile: float = 0.0, light_max_deg: int = 0,
                    chunk_edges: int = 0, build_wsb: bool = False, wsb_min_nnz: int = 0,
                    att_slot_max: int = 0, stream=None) -> Plan:
    o = _PlanOpts(heavy_quantile, light_max_deg, chunk_edges, int(build_wsb), wsb_min_nnz, att_slot_max)
    h = ctypes.c_void_p()
    _check(load_library().gnn_plan_create(csr.ref, ctypes.byref(o), _stream(stream),
                                          ctypes.byref(h)), "gnn_plan_create")
    return Plan(h.value, csr)


def gnn_plan_destroy(plan: Plan):
    plan.destroy()


def gnn_plan_autotune(csr: Csr, X: torch.Tensor, op: str = "multi", reps: int = 5, stream=None) -> dict:
    """Time the plan-option candidates for one aggregation on this graph and
    features; -> {"opts": {heavy_quantile, light_max_deg, chunk_edges},
    "best_ms": ..., "default_ms": ...}.  Pass opts to gnn_plan_create."""
    _need(X, "X", csr.n_cols, (None,), FEAT, rows_strided=True)
    _gpu(X=X)
    o = _PlanOpts()
    best, dflt = ctypes.c_float(0.0), ctypes.c_float(0.0)
    _check(load_library().gnn_plan_autotune(csr.ref, _ptr(X), _dtype_code(X), X.shape[1], X.stride(0),
                                            TUNE_OP[op], int(reps), ctypes.byref(o), ctypes.byref(best),
                                            ctypes.byref(dflt), _stream(stream)), "gnn_plan_autotune")
    return {"opts": {"heavy_quantile": round(o.heavy_quantile, 6), "light_max_deg": o.light_max_deg,
                     "chunk_edges": o.chunk_edges},
            "best_ms": best.value, "default_ms": dflt.value}


def gnn_plan_verify(plan: Plan, csr: Csr | None = None, stream=None):
    """Raise GnnError (PLAN_MISMATCH) if the plan's CSR changed since it was built
    (sizes, pointers, and sampled entries of row_ptr and col_idx)."""
    c = csr if csr is not None else plan.csr
    _check(load_library().gnn_plan_verify(plan.handle, c.ref, _stream(stream)), "gnn_plan_verify")


def gnn_plan_autotune_attention(csr: Csr, op: str, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor | None = None,
                                att: torch.Tensor | None = None, reps: int = 5, stream=None) -> dict:
    """Time the attention plan candidates on this graph and these inputs;
    op "gatv2" (q = xl, k = xr, att) or "gt" (q, k, v).  -> {"opts": {...},
    "mode": "csr" | "block16", "best_ms": ..., "default_ms": ...}."""
    _need(q, "q", csr.n_rows, (None, None), FEAT)
    H, D = q.shape[1], q.shape[2]
    _need(k, "k", csr.n_cols, (H, D), (q.dtype,))
    if op == "gt":
        _need(v, "v", csr.n_cols, (H, D), (q.dtype,))
    else:
        _need(att, "att", H, (D,), F32)
    _gpu(q=q, k=k, v=v, att=att)
    o = _PlanOpts()
    mode = ctypes.c_int(0)
    best, dflt = ctypes.c_float(0.0), ctypes.c_float(0.0)
    _check(load_library().gnn_plan_autotune_attention(
        csr.ref, 1 if op == "gt" else 0, _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(att), H, D, int(reps),
        ctypes.byref(o), ctypes.byref(mode), ctypes.byref(best), ctypes.byref(dflt), _stream(stream)),
        "gnn_plan_autotune_attention")
    return {"opts": {"heavy_quantile": round(o.heavy_quantile, 6), "chunk_edges": o.chunk_edges,
                     "att_slot_max": o.att_slot_max, "build_wsb": bool(o.build_wsb), "wsb_min_nnz": o.wsb_min_nnz},
            "mode": "block16" if mode.value == 1 else "csr", "best_ms": best.value, "default_ms": dflt.value}


def gnn_plan_stats(plan: Plan) -> dict:
    c = (ctypes.c_int64 * 9)()
    _check(load_library().gnn_plan_stats(plan.handle, c, 9), "gnn_plan_stats")
    keys = ("light_rows", "medium_rows", "heavy_rows", "items", "heavy_threshold",
            "wsb_windows", "wsb_blocks", "wsb_dense_tiles", "wsb_residual_edges")
    return dict(zip(keys, list(c)))


def gnn_plan_wsb_export(plan: Plan, stream=None):
    st = gnn_plan_stats(plan)
    dev = plan.csr.row_ptr.device
    wp = torch.empty(st["wsb_windows"] + 1, dtype=torch.int32, device=dev)
    bc = torch.empty((max(st["wsb_blocks"], 1), 8), dtype=torch.int32, device=dev)
    bb = torch.empty((max(st["wsb_blocks"], 1), 2), dtype=torch.int64, device=dev)
    _check(load_library().gnn_plan_wsb_export(plan.handle, _ptr(wp), _ptr(bc), _ptr(bb),
                                              _stream(stream)), "gnn_plan_wsb_export")
    return wp, bc[:st["wsb_blocks"]], bb[:st["wsb_blocks"]]


def _plan_h(plan):
    return plan.handle if plan is not None else None


def gnn_spmm(csr: Csr, X: torch.Tensor, norm: str = "none", Y: torch.Tensor | None = None,
             plan: Plan | None = None, stream=None) -> torch.Tensor:
    _need(X, "X", csr.n_cols, (None,), FEAT, rows_strided=True)
    F = X.shape[1]
    if Y is None:
        Y = torch.empty((csr.n_rows, F), dtype=torch.float32, device=X.device)
    _need(Y, "Y", csr.n_rows, (None,), F32, rows_strided=True)
    if Y.shape[1] < F:
        raise ValueError("Y must have at least as many columns as X")
    _gpu(X=X, Y=Y)
    _check(load_library().gnn_spmm(csr.ref, _ptr(X), _dtype_code(X), F, X.stride(0), _ptr(Y),
                                   Y.stride(0), NORM[norm], _plan_h(plan), _stream(stream)),
           "gnn_spmm")
    return Y


def gnn_spmm_block16(csr: Csr, X: torch.Tensor, norm: str = "none", Y: torch.Tensor | None = None,
                     plan: Plan | None = None, stream=None) -> torch.Tensor:
    """Y = A_norm X on the plan's 16 x 16 block-sparse tiles (plan built with build_wsb)."""
    _need(X, "X", csr.n_cols, (None,), FEAT, rows_strided=True)
    F = X.shape[1]
    if Y is None:
        Y = torch.empty((csr.n_rows, F), dtype=torch.float32, device=X.device)
    _need(Y, "Y", csr.n_rows, (None,), F32, rows_strided=True)
    if Y.shape[1] < F:
        raise ValueError("Y must have at least as many columns as X")
    _gpu(X=X, Y=Y)
    _check(load_library().gnn_spmm_block16(csr.ref, _ptr(X), _dtype_code(X), F, X.stride(0), _ptr(Y), Y.stride(0),
                                           NORM[norm], _plan_h(plan), _stream(stream)), "gnn_spmm_block16")
    return Y


def gnn_dot_aggr(csr: Csr, X: torch.Tensor, map: str = "feature", load: str = "scalar",
                 y: torch.Tensor | None = None, plan: Plan | None = None, stream=None) -> torch.Tensor:
    """dot-aggr micro-benchmark: y[i] = sum over row i's sources j of <X[i], X[j]> (float32 X);
    map "feature" | "neighbor", load "scalar" (4-byte) | "vec16" (16-byte per lane)."""
    _need(X, "X", max(csr.n_rows, csr.n_cols), (None,), F32, rows_strided=True)
    D = X.shape[1]
    if y is None:
        y = torch.empty(csr.n_rows, dtype=torch.float32, device=X.device)
    _need(y, "y", csr.n_rows, (), F32)
    _gpu(X=X, y=y)
    _check(load_library().gnn_dot_aggr(csr.ref, _ptr(X), D, X.stride(0), DOT_MAP[map], DOT_LOAD[load], _ptr(y),
                                       _plan_h(plan), _stream(stream)), "gnn_dot_aggr")
    return y


def gnn_reduce(csr: Csr, X: torch.Tensor, op: str = "sum", Y: torch.Tensor | None = None,
               arg: torch.Tensor | bool | None = None, plan: Plan | None = None, stream=None):
    """Returns (Y, arg); arg=True allocates the source-index output (max / min)."""
    _need(X, "X", csr.n_cols, (None,), FEAT, rows_strided=True)
    F = X.shape[1]
    if Y is None:
        Y = torch.empty((csr.n_rows, F), dtype=torch.float32, device=X.device)
    _need(Y, "Y", csr.n_rows, (None,), F32, rows_strided=True)
    if Y.shape[1] < F:
        raise ValueError("Y must have at least as many columns as X")
    if arg is True:
        arg = torch.empty((csr.n_rows, F), dtype=torch.int32, device=X.device)
    elif arg is False:
        arg = None
    if arg is not None:
        _need(arg, "arg", csr.n_rows, (F,), (torch.int32,))
    _gpu(X=X, Y=Y, arg=arg)
    _check(load_library().gnn_reduce(csr.ref, _ptr(X), _dtype_code(X), F, X.stride(0),
                                     REDUCE_OP[op], _ptr(Y), Y.stride(0), _ptr(arg),
                                     _plan_h(plan), _stream(stream)), "gnn_reduce")
    return Y, arg


def gnn_reduce_multi(csr: Csr, X: torch.Tensor, ops=("sum", "mean", "max", "min"), args: bool = True,
                     out: dict | None = None, plan: Plan | None = None, stream=None) -> dict:
    """One pass computing the requested reductions; returns {name: tensor} with
    keys among sum, mean, max, min, argmax, argmin (indices only with args)."""
    return _reduce_multi("gnn_reduce_multi", csr, X, ops, args, out, plan, stream)


def gnn_reduce_multi_noalloc(csr: Csr, X: torch.Tensor, out: dict, plan: Plan,
                             ops=("sum", "mean", "max", "min"), args: bool = True, stream=None) -> dict:
    """gnn_reduce_multi without any device allocation in the library: the plan
    (required) is built beforehand, split-row partials use the library's fixed
    per-GPU scratch array.  `out` must hold every requested output already
    (this wrapper allocates nothing either)."""
    if plan is None:
        raise ValueError("gnn_reduce_multi_noalloc needs a plan")
    want = set(ops) | ({"arg" + o for o in ("max", "min") if o in ops} if args else set())
    missing = want - set(out)
    if missing:
        raise ValueError(f"out lacks {sorted(missing)}")
    return _reduce_multi("gnn_reduce_multi_noalloc", csr, X, ops, args, out, plan, stream)


def _reduce_multi(fn: str, csr: Csr, X, ops, args, out, plan, stream) -> dict:
    _need(X, "X", csr.n_cols, (None,), FEAT, rows_strided=True)
    F = X.shape[1]
    out = dict(out or {})
    for op in ops:
        if op not in out:
            out[op] = torch.empty((csr.n_rows, F), dtype=torch.float32, device=X.device)
    if args:
        for op in ("max", "min"):
            if op in ops and "arg" + op not in out:
                out["arg" + op] = torch.empty((csr.n_rows, F), dtype=torch.int32, device=X.device)
    for k, o in out.items():
        if k.startswith("arg"):
            _need(o, k, csr.n_rows, (F,), (torch.int32,))
        else:
            _need(o, k, csr.n_rows, (None,), F32, rows_strided=True)
            if o.shape[1] < F:
                raise ValueError(f"{k} must have at least as many columns as X")
    lds = {o.stride(0) for k, o in out.items() if not k.startswith("arg")}
    if len(lds) != 1:
        raise ValueError("value outputs must share one row stride")
    _gpu(X=X, **out)
    _check(getattr(load_library(), fn)(
        csr.ref, _ptr(X), _dtype_code(X), F, X.stride(0), _ptr(out.get("sum")), _ptr(out.get("mean")),
        _ptr(out.get("max")), _ptr(out.get("argmax")), _ptr(out.get("min")), _ptr(out.get("argmin")),
        lds.pop(), _plan_h(plan), _stream(stream)), fn)
    return out


def gnn_gatv2_fused(csr: Csr, xl: torch.Tensor, xr: torch.Tensor, att: torch.Tensor,
                    neg_slope: float = 0.2, out: torch.Tensor | None = None,
                    lse: torch.Tensor | bool | None = True, plan: Plan | None = None, stream=None):
    """xl [n_rows, H, D], xr [n_cols, H, D] (bf16 or f32), att [H, D] f32 -> (out, lse)."""
    _need(xl, "xl", csr.n_rows, (None, None), FEAT)
    H, D = xl.shape[1], xl.shape[2]
    _need(xr, "xr", csr.n_cols, (H, D), (xl.dtype,))
    _need(att, "att", H, (D,), F32)
    if out is None:
        out = torch.empty((csr.n_rows, H, D), dtype=torch.float32, device=xl.device)
    if lse is True:
        lse = torch.empty((csr.n_rows, H), dtype=torch.float32, device=xl.device)
    elif lse is False:
        lse = None
    _need(out, "out", csr.n_rows, (H, D), F32)
    if lse is not None:
        _need(lse, "lse", csr.n_rows, (H,), F32)
    _gpu(xl=xl, xr=xr, att=att, out=out, lse=lse)
    _check(load_library().gnn_gatv2_fused(csr.ref, _ptr(xl), _ptr(xr), _dtype_code(xl), _ptr(att),
                                          H, D, float(neg_slope), _ptr(out), _ptr(lse),
                                          _plan_h(plan), _stream(stream)), "gnn_gatv2_fused")
    return out, lse


def gnn_gt_fused(csr: Csr, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float = 0.0,
                 mode: str = "csr", out: torch.Tensor | None = None,
                 lse: torch.Tensor | bool | None = True, plan: Plan | None = None, stream=None):
    """q [n_rows, H, D], k, v [n_cols, H, D] -> (out [n_rows, H, D] f32, lse [n_rows, H])."""
    _need(q, "q", csr.n_rows, (None, None), FEAT)
    H, D = q.shape[1], q.shape[2]
    _need(k, "k", csr.n_cols, (H, D), (q.dtype,))
    _need(v, "v", csr.n_cols, (H, D), (q.dtype,))
    if out is None:
        out = torch.empty((csr.n_rows, H, D), dtype=torch.float32, device=q.device)
    if lse is True:
        lse = torch.empty((csr.n_rows, H), dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    _need(out, "out", csr.n_rows, (H, D), F32)
    if lse is not None:
        _need(lse, "lse", csr.n_rows, (H,), F32)
    _gpu(q=q, k=k, v=v, out=out, lse=lse)
    _check(load_library().gnn_gt_fused(csr.ref, _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), H, D,
                                       float(scale), GT_MODE[mode], _ptr(out), _ptr(lse),
                                       _plan_h(plan), _stream(stream)), "gnn_gt_fused")
    return out, lse


def gnn_project(X: torch.Tensor, W, out=None, stream=None):
    """Y_m = X W_m^T for each bf16 weight W_m [f_out, f_in] (a tensor or a list of
    up to three), bf16 X [n, f_in]; -> list of bf16 [n, f_out] (bf16 matrix cores,
    fp32 accumulation, round to nearest even)."""
    Ws = [W] if isinstance(W, torch.Tensor) else list(W)
    if not 1 <= len(Ws) <= 3:
        raise ValueError("one to three weight matrices")
    _need(X, "X", 0, (None,), (torch.bfloat16,), rows_strided=True)
    n, fi = X.shape
    fo = Ws[0].shape[0]
    for k, w in enumerate(Ws):
        _need(w, f"W[{k}]", fo, (fi,), (torch.bfloat16,))
        if w.shape[0] != fo:
            raise ValueError("all weights need the same number of output features")
    if out is None:
        out = [torch.empty((n, fo), dtype=torch.bfloat16, device=X.device) for _ in Ws]
    if len(out) != len(Ws):
        raise ValueError("one output per weight")
    for k, y in enumerate(out):
        _need(y, f"Y[{k}]", n, (fo,), (torch.bfloat16,))
    _gpu(X=X, **{f"W{k}": w for k, w in enumerate(Ws)}, **{f"Y{k}": y for k, y in enumerate(out)})
    wp = (ctypes.c_void_p * len(Ws))(*[w.data_ptr() for w in Ws])
    yp = (ctypes.c_void_p * len(Ws))(*[y.data_ptr() for y in out])
    _check(load_library().gnn_project(_ptr(X), n, fi, X.stride(0), len(Ws), wp, fo, yp, _stream(stream)),
           "gnn_project")
    return out


def gnn_spmm_backward(csr: Csr, dY: torch.Tensor, norm: str = "none", dX: torch.Tensor | None = None,
                      plan: Plan | None = None, stream=None) -> torch.Tensor:
    """dX [n_cols, F] = A_norm^T dY (float32)."""
    _need(dY, "dY", csr.n_rows, (None,), F32, rows_strided=True)
    F = dY.shape[1]
    if dX is None:
        dX = torch.empty((csr.n_cols, F), dtype=torch.float32, device=dY.device)
    _need(dX, "dX", csr.n_cols, (None,), F32, rows_strided=True)
    if dX.shape[1] < F:
        raise ValueError("dX must have at least as many columns as dY")
    _gpu(dY=dY, dX=dX)
    _check(load_library().gnn_spmm_backward(csr.ref, _ptr(dY), F, dY.stride(0), _ptr(dX), dX.stride(0),
                                            NORM[norm], _plan_h(plan), _stream(stream)), "gnn_spmm_backward")
    return dX


def gnn_reduce_backward(csr: Csr, dY: torch.Tensor, op: str = "sum", arg: torch.Tensor | None = None,
                        dX: torch.Tensor | None = None, plan: Plan | None = None, stream=None) -> torch.Tensor:
    """dX [n_cols, F] (float32); arg: the forward's source indices (max / min)."""
    _need(dY, "dY", csr.n_rows, (None,), F32, rows_strided=True)
    F = dY.shape[1]
    if dX is None:
        dX = torch.empty((csr.n_cols, F), dtype=torch.float32, device=dY.device)
    _need(dX, "dX", csr.n_cols, (None,), F32, rows_strided=True)
    if dX.shape[1] < F:
        raise ValueError("dX must have at least as many columns as dY")
    if arg is not None:
        _need(arg, "arg", csr.n_rows, (F,), (torch.int32,))
    _gpu(dY=dY, dX=dX, arg=arg)
    _check(load_library().gnn_reduce_backward(csr.ref, REDUCE_OP[op], _ptr(dY), F, dY.stride(0), _ptr(arg),
                                              _ptr(dX), dX.stride(0), _plan_h(plan), _stream(stream)),
           "gnn_reduce_backward")
    return dX


def gnn_gatv2_backward(csr: Csr, xl: torch.Tensor, xr: torch.Tensor, att: torch.Tensor, out: torch.Tensor,
                       lse: torch.Tensor, dout: torch.Tensor, neg_slope: float = 0.2, plan: Plan | None = None,
                       stream=None):
    """-> (dxl [n_rows, H, D], dxr [n_cols, H, D], datt [H, D]), float32."""
    _need(xl, "xl", csr.n_rows, (None, None), FEAT)
    H, D = xl.shape[1], xl.shape[2]
    _need(xr, "xr", csr.n_cols, (H, D), (xl.dtype,))
    _need(att, "att", H, (D,), F32)
    for name, t in (("out", out), ("dout", dout)):
        _need(t, name, csr.n_rows, (H, D), F32)
    _need(lse, "lse", csr.n_rows, (H,), F32)
    dxl = torch.empty((csr.n_rows, H, D), dtype=torch.float32, device=xl.device)
    dxr = torch.empty((csr.n_cols, H, D), dtype=torch.float32, device=xl.device)
    datt = torch.empty((H, D), dtype=torch.float32, device=xl.device)
    _gpu(xl=xl, xr=xr, att=att, out=out, lse=lse, dout=dout)
    _check(load_library().gnn_gatv2_backward(csr.ref, _ptr(xl), _ptr(xr), _dtype_code(xl), _ptr(att), H, D,
                                             float(neg_slope), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dxl),
                                             _ptr(dxr), _ptr(datt), _plan_h(plan), _stream(stream)),
           "gnn_gatv2_backward")
    return dxl, dxr, datt


def gnn_gt_backward(csr: Csr, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                    lse: torch.Tensor, dout: torch.Tensor, scale: float = 0.0, plan: Plan | None = None,
                    stream=None):
    """-> (dq [n_rows, H, D], dk, dv [n_cols, H, D]), float32."""
    _need(q, "q", csr.n_rows, (None, None), FEAT)
    H, D = q.shape[1], q.shape[2]
    _need(k, "k", csr.n_cols, (H, D), (q.dtype,))
    _need(v, "v", csr.n_cols, (H, D), (q.dtype,))
    for name, t in (("out", out), ("dout", dout)):
        _need(t, name, csr.n_rows, (H, D), F32)
    _need(lse, "lse", csr.n_rows, (H,), F32)
    dq = torch.empty((csr.n_rows, H, D), dtype=torch.float32, device=q.device)
    dk = torch.empty((csr.n_cols, H, D), dtype=torch.float32, device=q.device)
    dv = torch.empty((csr.n_cols, H, D), dtype=torch.float32, device=q.device)
    _gpu(q=q, k=k, v=v, out=out, lse=lse, dout=dout)
    _check(load_library().gnn_gt_backward(csr.ref, _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), H, D, float(scale),
                                          _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                          _plan_h(plan), _stream(stream)), "gnn_gt_backward")
    return dq, dk, dv


def gnn_gt_backward_block16(csr: Csr, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                            lse: torch.Tensor, dout: torch.Tensor, scale: float = 0.0, plan: Plan | None = None,
                            stream=None):
    """Block-sparse (bf16 matrix cores) Graph Transformer backward; bf16 q, k, v.
    -> (dq, dk, dv), float32 [n, H, D]."""
    _need(q, "q", csr.n_rows, (None, None), (torch.bfloat16,))
    H, D = q.shape[1], q.shape[2]
    _need(k, "k", csr.n_cols, (H, D), (torch.bfloat16,))
    _need(v, "v", csr.n_cols, (H, D), (torch.bfloat16,))
    for name, t in (("out", out), ("dout", dout)):
        _need(t, name, csr.n_rows, (H, D), F32)
    _need(lse, "lse", csr.n_rows, (H,), F32)
    dq = torch.empty((csr.n_rows, H, D), dtype=torch.float32, device=q.device)
    dk = torch.empty((csr.n_cols, H, D), dtype=torch.float32, device=q.device)
    dv = torch.empty((csr.n_cols, H, D), dtype=torch.float32, device=q.device)
    _gpu(q=q, k=k, v=v, out=out, lse=lse, dout=dout)
    _check(load_library().gnn_gt_backward_block16(csr.ref, _ptr(q), _ptr(k), _ptr(v), H, D, float(scale),
                                                  _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                                  _plan_h(plan), _stream(stream)), "gnn_gt_backward_block16")
    return dq, dk, dv


def gnn_reorder(csr: Csr, kind: str = "degree", apply: bool = True, stream=None):
    """Returns perm (perm[new] = old) and, if apply, the relabelled (row_ptr, col_idx)."""
    dev = csr.row_ptr.device
    perm = torch.empty(csr.n_rows, dtype=torch.int32, device=dev)
    rp = ci = None
    if apply:
        rp = torch.empty(csr.n_rows + 1, dtype=torch.int32, device=dev)
        ci = torch.empty(max(csr.nnz, 1), dtype=torch.int32, device=dev)
    _check(load_library().gnn_reorder(csr.ref, REORDER[kind], _ptr(perm), _ptr(rp), _ptr(ci),
                                      _stream(stream)), "gnn_reorder")
    if apply:
        return perm, rp, ci[:csr.nnz]
    return perm


def gnn_permute_rows(perm: torch.Tensor, X: torch.Tensor, out: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    n, F = perm.numel(), X.shape[1]
    if out is None:
        out = torch.empty((n, F), dtype=X.dtype, device=X.device)
    _check(load_library().gnn_permute_rows(_ptr(perm), n, _ptr(X), _dtype_code(X), F, X.stride(0),
                                           _ptr(out), out.stride(0), _stream(stream)),
           "gnn_permute_rows")
    return out


def gnn_release_cached_memory():
    """Give the current device's cached stream-ordered temporaries back to the runtime."""
    _check(load_library().gnn_release_cached_memory(), "gnn_release_cached_memory")


def gnn_copy_bytes(src: torch.Tensor, dst: torch.Tensor, nbytes: int | None = None, stream=None):
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    _check(load_library().gnn_copy_bytes(_ptr(src), _ptr(dst), n, _stream(stream)),
           "gnn_copy_bytes")
    return dst
