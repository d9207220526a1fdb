"""Helpers shared by the GPU tests: move a synthetic case to the device and
measure the normwise error max|y - y*| / max|y*|."""
import numpy as np


def dev(case, name, device="cuda"):
    import torch
    if name in case.bits:
        t = torch.from_numpy(case.bits[name].view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(case.vals[name], dtype=np.float32))
    return t.to(device)


def nerr(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.isfinite(y).all(), "non-finite values in the GPU result"
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(y - ref)) / (den if den > 0 else 1.0))


def host(t):
    return t.detach().float().cpu().numpy()
