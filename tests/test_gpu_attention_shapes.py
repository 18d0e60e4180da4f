"""GPU parity of the fused CSR attention kernels (GATv2, Graph Transformer)
over the head shapes beyond the configurations' own: the IO-aware GNN layers
paper measures H in {2, 4, 8} x D in {32, 64, 128, 256} (experimental setup)
and GATv2 at H = 8, D = 128 (the larger-hidden-size row of its GATv2 table),
and its appendix D.2 pairs head-dimension specialisations with a fallback.

Shapes covered here, each against the fp64 oracle at the CSR kernels' 1e-4
bar (the attention bar proper is 2e-2):
  - rows wider than one 64-lane slot, cut into head groups (GATv2 2-4 KB rows,
    GT 4 KB rows);
  - heads whose 16-byte slices fill a number of lanes that is not a power of
    two (D = 48, 96 bf16; D = 20, 80 f32), padded to the next power of two;
  - heads whose byte width is not a multiple of 16 (D = 20, 7, 100 bf16;
    D = 33 f32), on 8-, 4- or 2-byte slices with run-time lanes per head;
with and without a plan that splits rows into chunks.  Then the pages' grid
shapes on the configuration graphs (sampled rows), and the shapes no lane
mapping serves, which must be refused.
"""
import numpy as np
import pytest

import gen
import graph_neural_network_amd as gnn
import oracle
from gpu_util import dev, dev_bf16, dev_csr, host
from test_gpu_attention import SMALL_PLAN, TOL, check, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def graph():
    return gen.rmat(0x5EED0210, 6000, 60000, self_loops=True)


def inputs(n, H, D, seed, count, dt):
    raw = [gen.gauss_bf16(seed + i, (n, H, D)) for i in range(count)]
    devs = [dev_bf16(a) if dt == "bf16" else dev(gen.bf16_to_f32(a)) for a in raw]
    return raw, devs


SHAPES = [(8, 128, "bf16"), (8, 128, "f32"), (16, 64, "bf16"), (4, 48, "bf16"), (2, 96, "bf16"),
          (3, 20, "f32"), (2, 80, "f32"), (3, 20, "bf16"), (1, 7, "bf16"), (3, 100, "bf16"), (2, 33, "f32"),
          (5, 24, "bf16"), (4, 256, "bf16"), (2, 256, "f32")]


@pytest.mark.parametrize("H,D,dt", SHAPES)
@pytest.mark.parametrize("planned", [False, True])
def test_gatv2_shapes(graph, H, D, dt, planned):
    print(f"gatv2 H={H} D={D} {dt} planned={planned}", flush=True)
    rp, ci = graph
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    plan = gnn.gnn_plan_create(csr, **SMALL_PLAN) if planned else None
    (xl, xr), (dl, dr) = inputs(n, H, D, 0xFEA70800 + D, 2, dt)
    att = gen.gauss_f32(0x3E170800 + H, (H, D), std=(1.0 / D) ** 0.5)
    out, lse = gnn.gnn_gatv2_fused(csr, dl, dr, dev(att), 0.2, plan=plan)
    ro, rl, va = oracle.gatv2(rp, ci, xl, xr, att, 0.2)
    check(host(out), host(lse), ro, rl, va)


@pytest.mark.parametrize("H,D,dt", SHAPES + [(8, 256, "bf16"), (4, 256, "f32"), (2, 512, "bf16")])
@pytest.mark.parametrize("planned", [False, True])
def test_gt_shapes(graph, H, D, dt, planned):
    print(f"gt H={H} D={D} {dt} planned={planned}", flush=True)
    rp, ci = graph
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    plan = gnn.gnn_plan_create(csr, **SMALL_PLAN) if planned else None
    (q, k, v), (dq, dk, dv) = inputs(n, H, D, 0xFEA70900 + D, 3, dt)
    out, lse = gnn.gnn_gt_fused(csr, dq, dk, dv, plan=plan)
    ro, rl, va = oracle.gt(rp, ci, q, k, v)
    check(host(out), host(lse), ro, rl, va)


@pytest.mark.parametrize("kind,H,D,dt", [("gatv2", 2, 130, "bf16"), ("gt", 2, 129, "f32"),
                                         ("gt", 1, 1040, "bf16")])
def test_unmapped_shapes_are_refused(graph, kind, H, D, dt):
    """Heads of more than 64 slices at the widest slice that divides them."""
    rp, ci = graph
    n = rp.size - 1
    csr = dev_csr(rp, ci)
    _, ts = inputs(n, H, D, 0xFEA70A00, 3, dt)
    with pytest.raises(gnn.GnnError) as e:
        if kind == "gatv2":
            gnn.gnn_gatv2_fused(csr, ts[0], ts[1], dev(np.zeros((H, D), np.float32)))
        else:
            gnn.gnn_gt_fused(csr, *ts)
    assert e.value.status == 2


def test_gatv2_h8_d128_config3_graph():
    """GATv2 at H = 8, D = 128 bf16 (2-KB rows: two head groups) on the
    200,000-node R-MAT graph of the GATv2 configuration, sampled rows."""
    w = gen.gatv2_rmat(H=8, D=128)
    csr = dev_csr(w.row_ptr, w.col_idx)
    plan = gnn.gnn_plan_create(csr)
    xl, xr, att = w.arrays["xl"], w.arrays["xr"], w.arrays["att"]
    out, lse = gnn.gnn_gatv2_fused(csr, dev_bf16(xl), dev_bf16(xr), dev(att), 0.2, plan=plan)
    rows = sample_rows(w.row_ptr, 2000, 8)
    ro, rl, va = oracle.gatv2(w.row_ptr, w.col_idx, xl, xr, att, 0.2, rows=rows)
    check(host(out), host(lse), ro, rl, va, rows=rows)


@pytest.mark.parametrize("H,D", [(2, 256), (4, 128), (8, 64)])
def test_gt_grid_shapes_config4_graph(H, D):
    """GT at the pages' grid shapes on the 512,000-node cluster graph of the
    GT configuration, CSR mode, sampled rows."""
    w = gen.gt_cluster(H=H, D=D)
    csr = dev_csr(w.row_ptr, w.col_idx)
    plan = gnn.gnn_plan_create(csr)
    q, k, v = w.arrays["q"], w.arrays["k"], w.arrays["v"]
    out, lse = gnn.gnn_gt_fused(csr, dev_bf16(q), dev_bf16(k), dev_bf16(v), plan=plan)
    rows = sample_rows(w.row_ptr, 2000, 9)
    ro, rl, va = oracle.gt(w.row_ptr, w.col_idx, q, k, v, rows=rows)
    check(host(out), host(lse), ro, rl, va, rows=rows)
