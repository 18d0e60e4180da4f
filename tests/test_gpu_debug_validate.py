"""GNN_DEBUG_VALIDATE=1: plan creation and reorder check the CSR's contents on
the device (row_ptr starts at 0, ends at nnz, never decreases; every column in
[0, n_cols)) and return INVALID_VALUE before any other kernel reads them.  The
check kernel reads the two arrays within their sizes only, so the invalid
inputs below are safe to hand to the device."""
import pytest
import torch

import graph_neural_network_amd as gnn

pytestmark = pytest.mark.gpu


def csr(rp, ci, n_cols=4):
    return gnn.Csr(torch.tensor(rp, dtype=torch.int32, device="cuda"),
                   torch.tensor(ci, dtype=torch.int32, device="cuda"), n_cols=n_cols)


VALID = ([0, 2, 3, 3, 5], [0, 1, 2, 0, 3])
BAD = {
    "row_ptr decreases": ([0, 3, 2, 3, 5], [0, 1, 2, 0, 3]),
    "row_ptr[0] != 0": ([1, 2, 3, 3, 5], [0, 1, 2, 0, 3]),
    "row_ptr[n] != nnz": ([0, 2, 3, 3, 4], [0, 1, 2, 0, 3]),
    "column too large": ([0, 2, 3, 3, 5], [0, 1, 2, 0, 4]),
    "negative column": ([0, 2, 3, 3, 5], [0, -1, 2, 0, 3]),
}
MESSAGE = {"row_ptr decreases": "decreases", "row_ptr[0] != 0": "row_ptr[0]", "row_ptr[n] != nnz": "row_ptr[0]",
           "column too large": "column", "negative column": "column"}


def test_valid_csr_passes(monkeypatch):
    monkeypatch.setenv("GNN_DEBUG_VALIDATE", "1")
    c = csr(*VALID)
    plan = gnn.gnn_plan_create(c)
    X = torch.ones((4, 16), device="cuda")
    Y = gnn.gnn_spmm(c, X, plan=plan)
    assert torch.equal(Y.sum(1).cpu(), torch.tensor([32.0, 16.0, 0.0, 32.0]))
    perm = gnn.gnn_reorder(c, "degree", apply=False)
    assert sorted(perm.cpu().tolist()) == [0, 1, 2, 3]


@pytest.mark.parametrize("case", sorted(BAD))
def test_invalid_csr_rejected(monkeypatch, case):
    monkeypatch.setenv("GNN_DEBUG_VALIDATE", "1")
    c = csr(*BAD[case])
    with pytest.raises(gnn.GnnError) as e:
        gnn.gnn_plan_create(c)
    assert gnn.STATUS[e.value.status] == "GNN_ERR_INVALID_VALUE", str(e.value)
    assert MESSAGE[case] in str(e.value)
    with pytest.raises(gnn.GnnError) as e:
        gnn.gnn_spmm(c, torch.ones((4, 16), device="cuda"))  # a transient plan: the same check
    assert MESSAGE[case] in str(e.value)
    with pytest.raises(gnn.GnnError) as e:
        gnn.gnn_reorder(c, "rcm")
    assert MESSAGE[case] in str(e.value)
    torch.cuda.synchronize()


def test_check_is_off_by_default(monkeypatch):
    """Without the variable no check runs: a valid CSR builds a plan (an
    invalid one is not handed to the device here, since it would be read
    unchecked)."""
    monkeypatch.delenv("GNN_DEBUG_VALIDATE", raising=False)
    plan = gnn.gnn_plan_create(csr(*VALID))
    assert gnn.gnn_plan_stats(plan)["light_rows"] == 4
