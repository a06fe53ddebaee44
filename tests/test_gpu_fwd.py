"""Forward pass on the GPU against the fp64 oracle, through the C ABI."""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, f32np, f64, maxabs, require_gpu
from io_aware_transformer_amd import FAError, fwd, inputs

pytestmark = pytest.mark.gpu


def _run(q, k, v, scale, causal):
    o, lse = fwd(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _check_full(B, Hq, Hkv, N, d, dtype, causal, seed, scale=None):
    require_gpu()
    q, k, v = inputs.make(B, Hq, Hkv, N, d, dtype, seed)
    scale = d ** -0.5 if scale is None else scale
    o, lse = _run(q, k, v, scale, causal)
    O, LSE = oracle.attention_forward(f64(q), f64(k), f64(v), scale, causal)
    tol = TOL[dtype]
    eo, el = maxabs(f64(o), O), maxabs(f64(lse), LSE)
    assert eo <= tol["out"], f"O max-abs {eo}"
    assert el <= tol["lse"], f"LSE max-abs {el}"
    return o, lse


# Small shapes: several tiles plus ragged tails, every head dim, grouped heads.
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 129, 300])
@pytest.mark.parametrize("heads", [(4, 4), (4, 2), (4, 1)])
def test_fwd_bf16_small(d, causal, N, heads):
    _check_full(2, heads[0], heads[1], N, d, torch.bfloat16, causal, seed=1000 + N + d)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 33, 200])
def test_fwd_fp32_small(d, causal, N):
    _check_full(2, 4, 2, N, d, torch.float32, causal, seed=2000 + N + d)


def test_fwd_fp32_config1():
    """fp32 non-causal, B=1 H=1 N=128 d=64, scale 1/8, whole output at 1e-5."""
    p = inputs.PRESETS["c1"]
    _check_full(p.B, p.Hq, p.Hkv, p.N, p.d, p.torch_dtype, p.causal, p.seed, p.scale)


@pytest.mark.parametrize("scale", [0.0, -0.3, 1.7])
def test_fwd_other_scales(scale):
    _check_full(1, 2, 2, 150, 128, torch.bfloat16, True, seed=7, scale=scale)
    _check_full(1, 2, 2, 70, 64, torch.float32, False, seed=8, scale=scale)


@pytest.mark.parametrize("name", ["c2", "c3a", "c3b", "c4a", "c4b", "c4c", "c5"])
def test_fwd_preset_sampled_rows(name):
    """Full-size presets: sampled rows of a few heads against the oracle's
    row-by-row forward, plus properties that hold for every row."""
    require_gpu()
    p = inputs.PRESETS[name]
    q, k, v = inputs.make_preset(p, with_grad=False)
    o, lse = _run(q, k, v, p.scale, p.causal)
    of, lf = f32np(o), lse.numpy()
    assert np.all(np.isfinite(of)) and np.all(np.isfinite(lf))
    # every output row is a convex combination of value rows
    vmax = float(np.max(np.abs(f32np(v))))
    assert float(np.max(np.abs(of))) <= vmax + 1e-2
    Q, K, V = f32np(q), f32np(k), f32np(v)
    rng = np.random.default_rng(p.seed)
    units = {(0, 0), (p.B - 1, p.Hq - 1), (int(rng.integers(p.B)), int(rng.integers(p.Hq)))}
    edge = [0, 1, 31, 32, 63, 64, 127, 128, 129, p.N // 2, p.N - 2, p.N - 1]
    rows = sorted(set(edge + [int(x) for x in rng.integers(0, p.N, 20)]))
    tol = TOL[p.torch_dtype]
    for b, h in sorted(units):
        O, LSE = oracle.attention_forward_rows(Q, K, V, p.scale, p.causal, b, h, rows)
        eo = maxabs(of[b, h, rows], O)
        el = maxabs(lf[b, h, rows], LSE)
        assert eo <= tol["out"], (b, h, eo)
        assert el <= tol["lse"], (b, h, el)


@pytest.mark.parametrize("name", ["c2", "c4a", "c4c", "c5"])
def test_fwd_equal_scores_full_size(name):
    """Q = 0: every score equal, so O_i is the mean of V_0..V_i and
    LSE_i = ln(i + 1) (causal) -- checked on every row at full size."""
    require_gpu()
    p = inputs.PRESETS[name]
    q, k, v = inputs.make_preset(p, with_grad=False)
    q = torch.zeros_like(q)
    o, lse = _run(q, k, v, p.scale, p.causal)
    G = p.Hq // p.Hkv
    V = f64(v)
    prefix = np.cumsum(V, axis=2) / np.arange(1, p.N + 1)[None, None, :, None]
    want = np.repeat(prefix, G, axis=1)
    assert maxabs(f64(o), want) <= TOL[p.torch_dtype]["out"]
    assert maxabs(lse.numpy(), np.broadcast_to(np.log(np.arange(1, p.N + 1)), lse.shape)) <= 1e-3
    # row 0 sees only key 0: its output is V_0 exactly
    assert torch.equal(o[:, :, 0], v.repeat_interleave(G, dim=1)[:, :, 0])


def test_fwd_deterministic():
    require_gpu()
    q, k, v = (t.cuda() for t in inputs.make(2, 8, 2, 1000, 128, torch.bfloat16, 5))
    o1, l1 = fwd(q, k, v, causal=True)
    o2, l2 = fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_gqa_equals_repeated_kv():
    require_gpu()
    q, k, v = (t.cuda() for t in inputs.make(2, 8, 2, 333, 128, torch.bfloat16, 6))
    o1, l1 = fwd(q, k, v, causal=True)
    o2, l2 = fwd(q, k.repeat_interleave(4, dim=1).contiguous(), v.repeat_interleave(4, dim=1).contiguous(),
                 causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("shape", [(0, 2, 2, 16, 64), (2, 2, 2, 0, 64), (0, 4, 1, 0, 128)])
def test_fwd_empty(shape):
    require_gpu()
    B, Hq, Hkv, N, d = shape
    q = torch.empty((B, Hq, N, d), device="cuda", dtype=torch.bfloat16)
    k = torch.empty((B, Hkv, N, d), device="cuda", dtype=torch.bfloat16)
    o, lse = fwd(q, k, k.clone(), causal=True)
    torch.cuda.synchronize()
    assert o.shape == q.shape and lse.shape == (B, Hq, N)


def test_fwd_bad_shape_raises():
    require_gpu()
    q = torch.zeros((1, 3, 16, 64), device="cuda", dtype=torch.bfloat16)
    k = torch.zeros((1, 2, 16, 64), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(FAError):
        fwd(q, k, k.clone())
