"""GPU parity of the GT CSR forward and backward when K and V exceed 2 GB.

The one-slot attention walks gather rows through one buffer descriptor per
array while every gathered array is below 2^31 bytes, and through per-row
descriptors or per-lane addresses above that.  Here a rectangular CSR of
1,000 destination rows draws its sources from 2,200,000 columns, so K and V
([n_cols, 8, 64] bf16) take 2.25 GB each and the walks take the second path.
Only the referenced source rows hold data (the rest are zero and must get
zero gradients); the oracle runs on the compacted problem: sources renumbered
0 .. u-1, padded to a square graph with empty rows.
"""
import numpy as np
import pytest
import torch

import gen
import graph_neural_network_amd as gnn
import oracle
from gpu_util import dev, dev_bf16, dev_csr, host
from test_gpu_attention import check
from test_gpu_backward import TOL_ATT, bwd_err

pytestmark = pytest.mark.gpu

N_ROWS, N_COLS, PER_ROW, H, D = 1000, 2_200_000, 12, 8, 64


def test_gt_csr_forward_and_backward_above_2gb():
    assert N_COLS * H * D * 2 >= 1 << 31
    rp = (np.arange(N_ROWS + 1, dtype=np.int64) * PER_ROW).astype(np.int32)
    raw = gen.uniform_u64(0x5EED0A01, N_ROWS * PER_ROW) % np.uint64(N_COLS)
    ci = raw.astype(np.int32)
    # distinct, sorted sources per row
    segs = [np.unique(ci[rp[r]:rp[r + 1]]) for r in range(N_ROWS)]
    keep = np.concatenate(segs)
    lens = np.array([g.size for g in segs])
    rp = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ci = keep.astype(np.int32)
    cols, ci_sub = np.unique(ci, return_inverse=True)
    u = cols.size
    n_sq = max(N_ROWS, u)
    rp_sq = np.concatenate([rp, np.full(n_sq - N_ROWS, rp[-1], np.int32)])
    q = gen.gauss_bf16(0x4A01, (n_sq, H, D))
    k_sub = gen.gauss_bf16(0x4A02, (n_sq, H, D))
    v_sub = gen.gauss_bf16(0x4A03, (n_sq, H, D))
    dO = gen.gauss_f32(0xFEA70A01, (n_sq, H, D))
    print("rows", N_ROWS, "distinct sources", u, "entries", ci.size, flush=True)

    csr = dev_csr(rp, ci, n_cols=N_COLS)
    idx = torch.from_numpy(cols.astype(np.int64)).cuda()
    K = torch.zeros((N_COLS, H, D), dtype=torch.bfloat16, device="cuda")
    V = torch.zeros_like(K)
    K[idx] = dev_bf16(k_sub[:u])
    V[idx] = dev_bf16(v_sub[:u])
    Q = dev_bf16(q[:N_ROWS])
    out, lse = gnn.gnn_gt_fused(csr, Q, K, V)
    ro, rl, va = oracle.gt(rp_sq, ci_sub.astype(np.int32), q, k_sub, v_sub)
    check(host(out), host(lse), ro[:N_ROWS], rl[:N_ROWS], va[:N_ROWS])

    dq, dk, dv = gnn.gnn_gt_backward(csr, Q, K, V, out, lse, dev(dO[:N_ROWS]))
    rq, rk, rv, mq, mk, mv = oracle.gt_backward(rp_sq, ci_sub.astype(np.int32), q, k_sub, v_sub, dO)
    assert bwd_err(host(dq), rq[:N_ROWS], mq[:N_ROWS]) <= TOL_ATT, "dq"
    assert bwd_err(host(dk[idx]), rk[:u], mk[:u]) <= TOL_ATT, "dk"
    assert bwd_err(host(dv[idx]), rv[:u], mv[:u]) <= TOL_ATT, "dv"
    # sources no entry names get exactly zero
    dk[idx] = 0.0
    dv[idx] = 0.0
    assert float(dk.abs().max()) == 0.0 and float(dv.abs().max()) == 0.0
