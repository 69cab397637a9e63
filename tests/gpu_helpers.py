"""Helpers for the GPU parity tests: move seeded host inputs to the device and
bring results back.  No arithmetic of the layer lives here."""
import numpy as np
import torch


def dev(a, device="cuda"):
    """numpy -> device tensor; uint16 arrays are bfloat16 bits."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def host(t):
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def rel_err(got, want):
    want = np.asarray(want, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    scale = np.abs(want).max()
    return float(np.abs(got - want).max() / (scale if scale > 0 else 1.0))


def log(msg):
    print(msg, flush=True)
