"""Helpers shared by the GPU parity tests (test-side only)."""
import numpy as np
import torch

import graph_neural_network_amd as gnn


def cuda_ok() -> bool:
    return torch.cuda.is_available()


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def dev_bf16(u16: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16 numpy) -> torch.bfloat16 on the GPU, bit for bit."""
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).cuda().view(torch.bfloat16)


def dev_csr(rp, ci, n_cols=None, edge_val=None) -> gnn.Csr:
    ev = None if edge_val is None else dev(edge_val.astype(np.float32))
    return gnn.Csr(dev(rp.astype(np.int32)), dev(ci.astype(np.int32)) if ci.size else
                   torch.zeros(0, dtype=torch.int32, device="cuda"), n_cols=n_cols, edge_val=ev)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def scaled_err(got, ref, mag):
    """max |got - ref| / mag elementwise; where mag == 0 the result must be exactly ref."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    mag = np.asarray(mag, np.float64)
    zero = mag == 0
    if np.any(got[zero] != ref[zero]):
        return np.inf
    d = np.abs(got - ref)
    if (~zero).any():
        return float((d[~zero] / mag[~zero]).max())
    return 0.0


def bits_equal_f32(got, ref) -> bool:
    g = np.ascontiguousarray(np.asarray(got, np.float32))
    r = np.ascontiguousarray(np.asarray(ref, np.float64).astype(np.float32))
    return bool(np.array_equal(g.view(np.uint32), r.view(np.uint32)))


def plain_rel(got, ref, floor_frac=1e-6):
    """The plain relative error |got - ref| / |ref| over the outputs with |ref|
    above floor_frac * max |ref| (a sum that cancels to near zero has no useful
    relative error): {"median", "p99", "max", "n", "excluded"}."""
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    a = np.abs(ref)
    keep = a > floor_frac * (a.max() if a.size else 0.0)
    r = np.abs(got[keep] - ref[keep]) / a[keep]
    if r.size == 0:
        return {"median": 0.0, "p99": 0.0, "max": 0.0, "n": 0, "excluded": int((~keep).sum())}
    return {"median": float(np.median(r)), "p99": float(np.quantile(r, 0.99)), "max": float(r.max()),
            "n": int(r.size), "excluded": int((~keep).sum())}
