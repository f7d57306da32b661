"""Helpers for the GPU parity tests: device copies and ring views (test side only)."""
import numpy as np
import pytest
import torch

TOL = {"fp32": 1e-4, "bf16": 2e-2}
TDT = {"fp32": torch.float32, "bf16": torch.bfloat16}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(TDT[dtype]).cuda()


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def ring_logical(data, ring):
    """Logical content [B, len, D] of a ring (oldest first)."""
    idx = [(ring.start + t) % ring.capacity for t in range(ring.len)]
    return data[:, idx]


def max_err(got, want):
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))))
