"""Helpers for the GPU parity tests (device checks, conversions)."""

import numpy as np
import pytest
import torch

# Tolerances: max-abs on O / dQ / dK / dV and on LSE.  bf16 and fp32 values
# follow the stated targets: 2e-2 (outputs) and 1e-3 (LSE) for bf16, 1e-5 for
# fp32.
TOL = {
    torch.bfloat16: {"out": 2e-2, "lse": 1e-3},
    torch.float32: {"out": 1e-5, "lse": 1e-5},
}


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")


def f64(t):
    """Exact upcast of a CPU bf16/fp32 tensor to a float64 numpy array."""
    return t.detach().cpu().to(torch.float32).numpy().astype(np.float64)


def f32np(t):
    return t.detach().cpu().to(torch.float32).numpy()


def maxabs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))
