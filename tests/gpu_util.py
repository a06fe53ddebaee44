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


def bf16_half_ulp(x):
    """Half the bf16 spacing at |x| (8 significant bits): the error that
    rounding an exact result to bf16 can add by itself."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.where(ax > 0, 2.0 ** (e - 8), 0.0)


def check_half_ulp(got, want, slack, name=""):
    """|got - want| <= half a bf16 ulp of want + slack, element by element
    (for results that are exact before the final rounding to bf16)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    bound = bf16_half_ulp(want) + slack
    assert np.all(err <= bound), f"{name}: worst excess {np.max(err - bound)}"


# Outside the fwd+bwd configurations (scale 1/sqrt(d), magnitudes below ~5)
# the flat bound is scaled with the size of the exact result: bf16 operands
# (P and dS rounded before the matrix products) and the bf16 O that enters
# D_i = dO_i . O_i carry relative errors of order 2^-9, so for grouped heads
# (dK/dV summing 4..32 heads) or sharper softmaxes (|scale| far above
# 1/sqrt(d)) the absolute error grows with the magnitude of the gradients.
REL_BF16 = 5e-3


def check_close(got, want, base, rel=None, name="", own_ulp=False):
    """max |got - want| <= base, or <= max(base, rel * max|want|) when
    ``rel`` is given; with ``own_ulp`` each element may also differ by half a
    bf16 ulp of its exact value (the rounding of the stored bf16 result, on
    top of the error of the computation).  Returns the max-abs error."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if got.size == 0:
        return 0.0
    err = np.abs(got - want)
    top = float(np.max(np.abs(want)))
    bound = base if rel is None else max(base, rel * top)
    excess = err - bound - (bf16_half_ulp(want) if own_ulp else 0.0)
    worst = float(err.max())
    if float(excess.max()) > 0:
        i = np.unravel_index(np.argmax(excess), err.shape)
        raise AssertionError(f"{name}: error {err[i]} exceeds its bound by {excess[i]} at {i} (got {got[i]}, "
                             f"want {want[i]}, max|want| {top}, max-abs {worst})")
    return worst
