"""Helpers for the GPU parity tests: device upload of the seeded inputs and the
comparison metric.

Metric: for every slice (one value head of the prefill, one decode row / state
matrix), err = max|x - r| / max|r|; the bound is 1e-4 for fp32 compute and 2e-2
for bf16 compute, state compared in fp32.  A pure absolute bound would be
vacuous for the prefill outputs, whose magnitude is ~1e-2.
"""
import numpy as np

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def dev(arr, device="cuda"):
    """inputs.Arr -> torch tensor on the GPU holding exactly the same bits."""
    import torch
    if arr.dtype == "bf16":
        return torch.from_numpy(arr.data.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(arr.data).to(device)


def host(t):
    """torch tensor -> float64 numpy."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def rel_err_slices(x, r, nslice_dims):
    """max|x-r|/max|r| over each slice indexed by the leading `nslice_dims` axes."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    lead = int(np.prod(x.shape[:nslice_dims])) if nslice_dims else 1
    xd = np.abs(x - r).reshape(lead, -1).max(axis=1)
    rm = np.abs(r).reshape(lead, -1).max(axis=1)
    return xd / np.maximum(rm, 1e-30), rm


def assert_close(x, r, tol, nslice_dims, what):
    x = np.asarray(x, np.float64)
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    err, rm = rel_err_slices(x, r, nslice_dims)
    worst = int(np.argmax(err))
    assert float(err.max()) <= tol, (
        f"{what}: max slice error {err.max():.3e} > {tol:g} (slice {worst}, max|ref| {rm[worst]:.3e}, "
        f"abs err {np.abs(x - r).max():.3e})")
    return float(err.max())
