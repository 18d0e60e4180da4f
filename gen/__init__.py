"""Seeded synthetic inputs (graphs in CSR, Gaussian features) for the kernels
and the oracle.

Holds none of the aggregation arithmetic: it only draws counter-based
random numbers (SplitMix64, Box-Muller, round-to-nearest-even bf16) and lays
the edge sets out as CSR with rows = destinations, columns sorted, no
duplicates.  See ``gen.c`` for the graph models and the trimming rule.

The workloads (sizes and distributions of the IO-aware GNN layers paper's
settings, with synthetic graphs standing in for its datasets):

=====  ======================================================================
 cfg   input
=====  ======================================================================
 1     Erdos-Renyi G(2000, 8000 pairs), symmetric + self loops; X 2000x64 f32
 2     R-MAT(0.57,0.19,0.19,0.05) 1,000,000 nodes, 16,000,000 edges;
       X 1,000,000x128 f32
 3     R-MAT 200,000 nodes, 4,000,000 edges + self loops; l, r [N,4,32] bf16;
       a [4,32] f32 ~ N(0, 1/32); LeakyReLU slope 0.2
 4     cluster graph 512,000 nodes (clusters of 64, p = 0.5, 1% inter edges)
       + self loops; Q, K, V [N,8,64] bf16 ~ N(0,1)
 5     R-MAT 16,000,000 nodes, 256,000,000 edges; X 16,000,000x256 bf16
=====  ======================================================================

Seeds: graph 0x5EED0000 + k, features 0xFEA70000 + k, weights 0x3E170000 + k.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgnngen.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile libgnngen.so with gcc (OpenMP)."""
    import subprocess

    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           os.path.join(_HERE, "gen.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class _Graph(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("m", ctypes.c_int64),
                ("row_ptr", ctypes.POINTER(ctypes.c_int32)),
                ("col_idx", ctypes.POINTER(ctypes.c_int32))]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i32, i64, u64, dbl, vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                              ctypes.c_double, ctypes.c_void_p)
    gp = ctypes.POINTER(_Graph)
    lib.gen_draw.argtypes = [u64, u64]
    lib.gen_draw.restype = u64
    lib.gen_uniform_u64.argtypes = [u64, i64, vp]
    lib.gen_gauss_f32.argtypes = [u64, i64, dbl, vp]
    lib.gen_gauss_bf16.argtypes = [u64, i64, dbl, vp]
    lib.gen_f32_to_bf16.argtypes = [i64, vp, vp]
    lib.gen_permutation.argtypes = [u64, i32, vp]
    lib.gen_rmat.argtypes = [u64, i32, i64, dbl, dbl, dbl, ctypes.c_int, ctypes.c_int, gp]
    lib.gen_er_undirected.argtypes = [u64, i32, i64, ctypes.c_int, gp]
    lib.gen_cluster.argtypes = [u64, i32, i32, dbl, dbl, ctypes.c_int, gp]
    lib.gen_from_edges.argtypes = [i32, i64, vp, vp, gp]
    lib.gen_graph_free.argtypes = [gp]
    for f in ("gen_rmat", "gen_er_undirected", "gen_cluster", "gen_from_edges", "gen_permutation"):
        getattr(lib, f).restype = ctypes.c_int
    lib.gen_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _take(g: _Graph):
    lib = _load()
    n, m = g.n, g.m
    rp = np.ctypeslib.as_array(g.row_ptr, shape=(n + 1,)).copy()
    ci = (np.ctypeslib.as_array(g.col_idx, shape=(m,)).copy() if m > 0
          else np.zeros(0, np.int32))
    lib.gen_graph_free(ctypes.byref(g))
    return rp, ci


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def draw(seed: int, counter: int) -> int:
    return int(_load().gen_draw(seed & (2**64 - 1), counter))


def uniform_u64(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint64)
    _load().gen_uniform_u64(seed, n, _ptr(out))
    return out


def gauss_f32(seed: int, shape, std: float = 1.0) -> np.ndarray:
    out = np.empty(shape, np.float32)
    _load().gen_gauss_f32(seed, out.size, std, _ptr(out))
    return out


def gauss_bf16(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of RNE(std * N(0,1))."""
    out = np.empty(shape, np.uint16)
    _load().gen_gauss_bf16(seed, out.size, std, _ptr(out))
    return out


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().gen_f32_to_bf16(x.size, _ptr(x), _ptr(out))
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns."""
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def permutation(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    _check(_load().gen_permutation(seed, n, _ptr(out)), "permutation")
    return out


def rmat(seed: int, n: int, m: int, a=0.57, b=0.19, c=0.19, relabel=True, self_loops=False):
    g = _Graph()
    _check(_load().gen_rmat(seed, n, m, a, b, c, int(relabel), int(self_loops), ctypes.byref(g)),
           "rmat")
    return _take(g)


def er_undirected(seed: int, n: int, m_pairs: int, self_loops=True):
    g = _Graph()
    _check(_load().gen_er_undirected(seed, n, m_pairs, int(self_loops), ctypes.byref(g)), "er")
    return _take(g)


def cluster(seed: int, n: int, csize: int = 64, p: float = 0.5, frac: float = 0.01,
            self_loops=True):
    g = _Graph()
    _check(_load().gen_cluster(seed, n, csize, p, frac, int(self_loops), ctypes.byref(g)),
           "cluster")
    return _take(g)


def grid2d(seed: int, k: int):
    """k x k four-neighbour grid, every undirected edge stored both ways, no
    self loops; vertex labels drawn by a seeded uniform permutation, so the
    stored numbering carries no locality (a road-network-like stand-in:
    degree at most 4)."""
    r, c = np.divmod(np.arange(k * k, dtype=np.int64), k)
    right = np.nonzero(c < k - 1)[0]
    down = np.nonzero(r < k - 1)[0]
    a = np.r_[right, down]
    b = np.r_[right + 1, down + k]
    lab = permutation(seed, k * k).astype(np.int64)
    src = lab[np.r_[a, b]]
    dst = lab[np.r_[b, a]]
    return from_edges(k * k, src, dst)


def from_edges(n: int, src, dst):
    """CSR (rows = destinations) from an explicit edge list src[k] -> dst[k]."""
    s = np.ascontiguousarray(src, np.int32)
    d = np.ascontiguousarray(dst, np.int32)
    assert s.shape == d.shape
    g = _Graph()
    _check(_load().gen_from_edges(n, s.size, _ptr(s), _ptr(d), ctypes.byref(g)), "from_edges")
    return _take(g)


def num_threads() -> int:
    return int(_load().gen_num_threads())


def degree_stats(row_ptr: np.ndarray) -> dict:
    """Descriptive statistics of the row lengths (for logs only)."""
    d = np.diff(row_ptr.astype(np.int64))
    n = d.size
    if n == 0:
        return {"n": 0, "m": 0}
    mean = float(d.mean())
    sd = float(d.std())
    skew = float(((d - mean) ** 3).mean() / sd ** 3) if sd > 0 else 0.0
    q = np.quantile(d, [0.5, 0.99, 0.999]) if n > 0 else [0, 0, 0]
    return {"n": int(n), "m": int(d.sum()), "empty_rows": int((d == 0).sum()),
            "max_deg": int(d.max()), "q50": float(q[0]), "q99": float(q[1]),
            "q999": float(q[2]), "skewness": skew}


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------

GRAPH_SEED = 0x5EED0000
FEAT_SEED = 0xFEA70000
WEIGHT_SEED = 0x3E170000


@dataclass
class Workload:
    name: str
    n: int
    row_ptr: np.ndarray
    col_idx: np.ndarray
    arrays: dict = field(default_factory=dict)
    params: dict = field(default_factory=dict)

    @property
    def nnz(self) -> int:
        return int(self.col_idx.size)


def gcn_small(n=2000, m_pairs=8000, F=64, k=1) -> Workload:
    rp, ci = er_undirected(GRAPH_SEED + k, n, m_pairs, self_loops=True)
    X = gauss_f32(FEAT_SEED + k, (n, F))
    return Workload("gcn_er2000_f64", n, rp, ci, {"X": X}, {"F": F, "norm": "both"})


def reduce_rmat(n=1_000_000, m=16_000_000, F=128, k=2, with_x=True) -> Workload:
    rp, ci = rmat(GRAPH_SEED + k, n, m)
    arrays = {"X": gauss_f32(FEAT_SEED + k, (n, F))} if with_x else {}
    return Workload(f"reduce_rmat{n}_{m}_f{F}", n, rp, ci, arrays, {"F": F})


def gatv2_rmat(n=200_000, m=4_000_000, H=4, D=32, k=3) -> Workload:
    rp, ci = rmat(GRAPH_SEED + k, n, m, self_loops=True)
    xl = gauss_bf16(FEAT_SEED + k, (n, H, D))
    xr = gauss_bf16(FEAT_SEED + 100 + k, (n, H, D))
    att = gauss_f32(WEIGHT_SEED + k, (H, D), std=(1.0 / D) ** 0.5)
    return Workload(f"gatv2_rmat{n}_{m}_h{H}d{D}", n, rp, ci,
                    {"xl": xl, "xr": xr, "att": att}, {"H": H, "D": D, "slope": 0.2})


def gatv2_layer_rmat(n=200_000, m=4_000_000, F_in=128, H=4, D=32, k=3) -> Workload:
    """The GATv2 layer as configured from node features: X [n, F_in] bf16 ~ N(0, 1),
    W_l, W_r [H*D, F_in] bf16 ~ N(0, 1/F_in) (variance 1/F_in, one row per output
    feature), attention vector a [H, D] fp32 ~ N(0, 1/D), on the same graph as
    gatv2_rmat."""
    rp, ci = rmat(GRAPH_SEED + k, n, m, self_loops=True)
    X = gauss_bf16(FEAT_SEED + 300 + k, (n, F_in))
    std = (1.0 / F_in) ** 0.5
    Wl = gauss_bf16(WEIGHT_SEED + 100 + k, (H * D, F_in), std=std)
    Wr = gauss_bf16(WEIGHT_SEED + 200 + k, (H * D, F_in), std=std)
    att = gauss_f32(WEIGHT_SEED + k, (H, D), std=(1.0 / D) ** 0.5)
    return Workload(f"gatv2_layer_rmat{n}_{m}_f{F_in}_h{H}d{D}", n, rp, ci,
                    {"X": X, "W_l": Wl, "W_r": Wr, "att": att}, {"F_in": F_in, "H": H, "D": D, "slope": 0.2})


def gt_cluster(n=512_000, csize=64, p=0.5, frac=0.01, H=8, D=64, k=4, with_x=True) -> Workload:
    rp, ci = cluster(GRAPH_SEED + k, n, csize, p, frac, self_loops=True)
    arrays = {}
    if with_x:
        arrays = {"q": gauss_bf16(FEAT_SEED + k, (n, H, D)), "k": gauss_bf16(FEAT_SEED + 100 + k, (n, H, D)),
                  "v": gauss_bf16(FEAT_SEED + 200 + k, (n, H, D))}
    return Workload(f"gt_cluster{n}_c{csize}_h{H}d{D}", n, rp, ci, arrays,
                    {"H": H, "D": D, "scale": 1.0 / D ** 0.5})


def spmm_rmat_large(n=16_000_000, m=256_000_000, F=256, k=5, with_x=True) -> Workload:
    rp, ci = rmat(GRAPH_SEED + k, n, m)
    arrays = {"X": gauss_bf16(FEAT_SEED + k, (n, F))} if with_x else {}
    return Workload(f"spmm_rmat{n}_{m}_f{F}_bf16", n, rp, ci, arrays, {"F": F})
