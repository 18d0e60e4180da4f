"""GPU parity of the per-vertex projections (gnn_project) and of the GATv2
layer computed from node features: X -> (l = X W_l^T, r = X W_r^T) on the
bf16 matrix cores -> fused GATv2 (the IO-aware GNN layers paper, section 2.2:
e_ij = a^T LeakyReLU(W_l h_i + W_r h_j), v_j = W_r h_j; appendix D.2 feeds
the fused kernel the vectors precomputed per vertex).

Projection bar.  Products of two bf16 values are exact in fp32, so before the
final rounding the kernel's value differs from the exact sum by at most the
fp32 accumulation error, K * 2^-24 * sum_k |x w| over K = f_in terms; the
bf16 rounding (8 significant bits, round to nearest even) adds at most
2^-8 |y|.  Each output must lie within 2^-8 |y| + 2 K 2^-24 sum |x w| of the
oracle's exact float64 y, and within one bf16 step of RNE(y); almost all must
equal RNE(y) exactly.

Layer bar: the attention bar, max |out - ref| / sum_j alpha_ij |r_j| <= 2e-2,
against the oracle's layer with l and r kept exact in float64 (the kernel's
inputs are rounded to bf16, as the configuration states them).
"""
import numpy as np
import pytest
import torch

import gen
import graph_neural_network_amd as gnn
import oracle
from gpu_util import dev, dev_bf16, dev_csr, host, scaled_err

pytestmark = pytest.mark.gpu


def rne_bf16(y: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bf16 bits, round to nearest even (test-side)."""
    return gen.f32_to_bf16(y.astype(np.float32))


def to_bits(t: torch.Tensor) -> np.ndarray:
    return host(t.view(torch.int16)).view(np.uint16)


def check_projection(got_bits, y, yabs, K):
    g = gen.bf16_to_f32(got_bits).astype(np.float64)
    bound = 2.0 ** -8 * np.abs(y) + 2 * K * 2.0 ** -24 * yabs + 1e-30
    assert np.all(np.abs(g - y) <= bound), float(np.max(np.abs(g - y) / bound))
    want = rne_bf16(y)
    # where the fp32 accumulation error cannot reach a bf16 step, the result
    # is at most one step from the correctly rounded value
    clear = np.abs(y) * 2.0 ** -9 > 2 * K * 2.0 ** -24 * yabs
    steps = np.abs(got_bits.astype(np.int32) - want.astype(np.int32))[clear]
    assert steps.size == 0 or int(steps.max()) <= 1
    return float(np.mean(got_bits == want))


@pytest.mark.parametrize("n,fi,fo,nm", [(1000, 128, 128, 2), (3, 32, 16, 1), (64 * 4 + 5, 96, 48, 3),
                                        (777, 512, 272, 1), (2049, 256, 64, 2), (130, 160, 32, 3)])
def test_project_matches_oracle(n, fi, fo, nm):
    print(f"project n={n} f_in={fi} f_out={fo} n_mat={nm}", flush=True)
    X = gen.gauss_bf16(0xFEA70700 + fi, (n, fi))
    Ws = [gen.gauss_bf16(0x3E170700 + 31 * m + fo, (fo, fi), std=fi ** -0.5) for m in range(nm)]
    Ys = gnn.gnn_project(dev_bf16(X), [dev_bf16(W) for W in Ws])
    for W, Yd in zip(Ws, Ys):
        y, ya = oracle.project(X, W)
        exact = check_projection(to_bits(Yd), y, ya, fi)
        assert exact > 0.99, exact


def test_project_strided_input_and_identity():
    n, fi = 500, 64
    Xw = gen.gauss_bf16(0xFEA70711, (n, fi + 24))            # a row stride of 88 elements
    Xd = dev_bf16(Xw)[:, :fi]
    I = gen.f32_to_bf16(np.eye(fi, dtype=np.float32))
    Y, = gnn.gnn_project(Xd, [dev_bf16(I)])
    assert np.array_equal(to_bits(Y), np.ascontiguousarray(Xw[:, :fi]))  # identity weights: exact copy


def test_project_rejects_bad_shapes():
    X = torch.zeros((10, 48), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((16, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gnn.GnnError) as e:
        gnn.gnn_project(X, [W])
    assert e.value.status == 2  # f_in not a multiple of 32


@pytest.fixture(scope="module")
def layer():
    return gen.gatv2_layer_rmat()


def test_gatv2_layer_config3(layer):
    """The configured GATv2 layer end to end: 200,000-node R-MAT with self
    loops, X 200,000 x 128 bf16, W_l, W_r 128 x 128 bf16, 4 heads x 32;
    projection on the matrix cores, then the fused layer; sampled rows
    (uniform plus the 16 largest hubs) against the exact float64 layer."""
    w = layer
    n, H, D = w.n, w.params["H"], w.params["D"]
    X = dev_bf16(w.arrays["X"])
    Wl, Wr = dev_bf16(w.arrays["W_l"]), dev_bf16(w.arrays["W_r"])
    xl, xr = [t.view(n, H, D) for t in gnn.gnn_project(X, [Wl, Wr])]
    csr = dev_csr(w.row_ptr, w.col_idx)
    plan = gnn.gnn_plan_create(csr)
    out, lse = gnn.gnn_gatv2_fused(csr, xl, xr, dev(w.arrays["att"]), 0.2, plan=plan)
    d = np.diff(w.row_ptr)
    rng = np.random.default_rng(3)
    rows = np.unique(np.r_[rng.integers(0, n, 3000), np.argsort(-d, kind="stable")[:16]]).astype(np.int32)
    ro, rl, va = oracle.gatv2_layer(w.row_ptr, w.col_idx, w.arrays["X"], w.arrays["W_l"], w.arrays["W_r"],
                                    w.arrays["att"], H, D, 0.2, rows=rows)
    g_out, g_lse = host(out)[rows], host(lse)[rows]
    err = scaled_err(g_out, ro, va)
    assert err <= 2e-2, err
    lerr = float(np.max(np.abs(g_lse - rl) / np.maximum(1.0, np.abs(rl))))
    assert lerr <= 2e-2, lerr
    # the projections themselves, on the sampled rows and their sources
    L, La = oracle.project(w.arrays["X"][rows], w.arrays["W_l"])
    check_projection(to_bits(xl.reshape(n, H * D))[rows], L, La, 128)
    print(f"config-3 layer: out err {err:.2e}, lse err {lerr:.2e}", flush=True)
