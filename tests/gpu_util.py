"""Helpers shared by the GPU tests: move a synthetic case to the device,
measure the normwise error max|y - y*| / max|y*| (the pass bar) and the
elementwise error max |y - y*| / max(|y*|, 1e-3) (printed as a diagnostic:
it shows where in a tensor the error sits, which the normwise figure hides)."""
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
    den = np.max(np.abs(ref)) if ref.size else 0.0
    return float(np.max(np.abs(y - ref)) / (den if den > 0 else 1.0)) if ref.size else 0.0


def eerr(y, ref, floor=1e-3):
    """Elementwise relative error with an absolute floor (diagnostic only)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not ref.size:
        return 0.0
    return float(np.max(np.abs(y - ref) / np.maximum(np.abs(ref), floor)))


def check(name, y, ref, tol):
    """Print both errors of one output and assert the normwise bar."""
    e = nerr(y, ref)
    print("  %-8s nerr=%.3e  elementwise=%.3e" % (name, e, eerr(y, ref)), flush=True)
    assert e <= tol, (name, e, tol)
    return e


def host(t):
    return t.detach().float().cpu().numpy()
