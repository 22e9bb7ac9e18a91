"""Helpers for the GPU parity tests (device upload, error metric)."""
import sys

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def torch_dev():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def up(x, dtype, dev):
    """Upload a float32 numpy array holding values of `dtype` exactly."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def down(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def rel_err(x, r, pair_axes):
    """max over (batch, head) slices of max|x - r| / max|r| (per-slice norm)."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    ax = tuple(i for i in range(r.ndim) if i not in pair_axes)
    num = np.max(np.abs(x - r), axis=ax)
    den = np.maximum(np.max(np.abs(r), axis=ax), 1e-30)
    return float(np.max(num / den))


def out_err(x, r):  # O: [B, T, H, dv] -> slices over (b, h)
    return rel_err(x, r, (0, 2))


def state_err(x, r):  # state: [B, H, dk, dv]
    return rel_err(x, r, (0, 1))


def note(*a):
    print(*a, flush=True)
    sys.stdout.flush()
