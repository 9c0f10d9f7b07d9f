"""Helpers shared by the GPU parity tests (host <-> device marshalling and
comparisons). Nothing here computes any part of the method."""
import numpy as np
import torch

DEV = "cuda"


def dev(a, dtype=None):
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    if a.dtype == np.uint64:
        return torch.from_numpy(a.view(np.int64)).to(DEV)
    t = torch.from_numpy(a).to(DEV)
    return t if dtype is None else t.to(dtype)


def host(t):
    """device tensor -> numpy; bf16 -> uint16 bit patterns."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def normwise_rel(got, ref):
    """max |got - ref| / max |ref| over the tensor, and the max elementwise error."""
    g, r = as_f64(got), as_f64(ref)
    err = np.abs(g - r)
    return float(err.max() / max(np.abs(r).max(), 1e-30)), float(err.max())
