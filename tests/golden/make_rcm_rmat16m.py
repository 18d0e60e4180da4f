"""Write tests/golden/rcm_rmat16m.txt: SHA-256 digests of the reverse
Cuthill-McKee permutation and of the relabelled CSR of the 16,000,000-node /
256,000,000-edge R-MAT graph (a = 0.57, b = 0.19, c = 0.19), as the CPU
oracle computes them.

    python tests/golden/make_rcm_rmat16m.py

Only the seeded generator (gen) and the oracle run here; nothing from the
HIP library.  RCM follows the textbook steps on the symmetrised pattern
(Tang et al., "A High-Throughput Solver for Marginalized Graph Kernels on
GPU", graph reordering section, names RCM as its bandwidth-reducing order):
each component starts at its unvisited vertex of smallest (degree, id), a
FIFO queue appends unvisited neighbours in increasing (degree, id), and the
visit order is reversed.  The relabelled CSR is P A P^T with every row's
columns sorted ascending.

The digests are of the little-endian int32 bytes of each array.  The graph's
own arrays are digested too, so that a test can first confirm it generated
the same graph.  Takes a few minutes and about 12 GB of host memory.
"""
import hashlib
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import gen  # noqa: E402
import oracle  # noqa: E402

OUT = os.path.join(HERE, "rcm_rmat16m.txt")


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a, dtype="<i4").tobytes()).hexdigest()


def main():
    t0 = time.time()
    w = gen.spmm_rmat_large(with_x=False)
    print(f"graph {w.name}: n {w.n}, nnz {w.nnz} ({time.time() - t0:.0f} s)", flush=True)
    t1 = time.time()
    perm = oracle.rcm(w.row_ptr, w.col_idx)
    print(f"oracle rcm: {time.time() - t1:.0f} s", flush=True)
    t2 = time.time()
    rp2, ci2 = oracle.permute_csr(w.row_ptr, w.col_idx, perm)
    print(f"oracle permute_csr: {time.time() - t2:.0f} s", flush=True)
    lines = [
        "# Reverse Cuthill-McKee of the R-MAT graph of 16,000,000 nodes and 256,000,000",
        "# directed edges (a = 0.57, b = 0.19, c = 0.19, graph seed 0x5EED0005, vertices",
        "# relabelled by a seeded permutation), computed by the CPU oracle alone",
        "# (tests/golden/make_rcm_rmat16m.py).  RCM as in Tang et al., \"A High-Throughput",
        "# Solver for Marginalized Graph Kernels on GPU\", graph reordering section, with",
        "# the textbook steps on the symmetrised pattern.  SHA-256 of little-endian int32.",
        f"n {w.n}",
        f"nnz {w.nnz}",
        f"graph_row_ptr {digest(w.row_ptr)}",
        f"graph_col_idx {digest(w.col_idx)}",
        f"perm {digest(perm)}",
        f"row_ptr_out {digest(rp2)}",
        f"col_idx_out {digest(ci2)}",
        f"perm_head {' '.join(str(int(x)) for x in perm[:8])}",
        f"perm_tail {' '.join(str(int(x)) for x in perm[-8:])}",
    ]
    with open(OUT, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {OUT} ({time.time() - t0:.0f} s in all)", flush=True)


if __name__ == "__main__":
    main()
