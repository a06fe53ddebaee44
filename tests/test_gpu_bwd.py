"""Backward pass on the GPU against the fp64 oracle, through the C ABI.

The GPU backward consumes the GPU forward's O and LSE (as the ABI requires);
the oracle recomputes everything from Q, K, V, dO in float64."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import REL_BF16, TOL, check_close, check_half_ulp, f64, maxabs, require_gpu
from io_aware_transformer_amd import FAError, bwd, bwd_workspace_size, fwd, inputs

pytestmark = pytest.mark.gpu


def _gpu_grads(q, k, v, do, scale, causal, workspace=None):
    q, k, v, do = (t.cuda() for t in (q, k, v, do))
    o, lse = fwd(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = bwd(q, k, v, o, lse, do, scale=scale, causal=causal, workspace=workspace)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 129, 300])
@pytest.mark.parametrize("heads", [(4, 4), (4, 2), (4, 1)])
def test_bwd_small(d, causal, N, heads):
    require_gpu()
    q, k, v, do = inputs.make(2, heads[0], heads[1], N, d, torch.bfloat16, 3000 + N + d, with_grad=True)
    scale = d ** -0.5
    dq, dk, dv = _gpu_grads(q, k, v, do, scale, causal)
    dQ, dK, dV = oracle.attention_backward(f64(q), f64(k), f64(v), f64(do), scale, causal)
    tol = TOL[torch.bfloat16]["out"]
    # One query head per key/value head at the default scale: the flat bound.
    # Grouped heads sum 2 or 4 heads into dK/dV: bound scaled with magnitude.
    rel = None if heads[0] == heads[1] else REL_BF16
    for name, got, want in (("dQ", dq, dQ), ("dK", dk, dK), ("dV", dv, dV)):
        check_close(f64(got), want, tol, rel, name)


@pytest.mark.parametrize("name,units,strict", [("c5", [(0, 0), (3, 15), (2, 7)], True),
                                               ("c2", [(0, 0), (7, 15)], True),
                                               ("c4a", [(1, 5)], False), ("c4b", [(3, 0)], False)])
def test_bwd_full_size_sampled_heads(name, units, strict):
    """Full-size shapes: complete dQ/dK/dV of sampled heads vs the oracle.
    ``units`` are (batch, kv head); every query head of the group is
    included so dK/dV sums are complete.  The fwd+bwd shapes (c5, and c2 at
    d=128) are held to the flat 2e-2 max-abs bound; grouped shapes, whose
    dK/dV sum 4 or 32 heads and exceed magnitude 8, get
    max(2e-2, 0.5% of the largest exact magnitude)."""
    require_gpu()
    p = inputs.PRESETS[name]
    q, k, v, do = inputs.make_preset(p, with_grad=True)
    dq, dk, dv = _gpu_grads(q, k, v, do, p.scale, p.causal)
    G = p.Hq // p.Hkv
    tol = TOL[torch.bfloat16]["out"]
    for b, g in units:
        dK = np.zeros((p.N, p.d))
        dV = np.zeros((p.N, p.d))
        for h in range(g * G, (g + 1) * G):
            hq, hk, hv = oracle.head_backward(f64(q[b, h]), f64(k[b, g]), f64(v[b, g]), f64(do[b, h]), p.scale,
                                              p.causal)
            dK += hk
            dV += hv
            if strict:
                assert maxabs(f64(dq[b, h]), hq) <= tol, ("dQ", b, h)
            else:
                check_close(f64(dq[b, h]), hq, tol, REL_BF16, f"dQ[{b},{h}]")
        if strict:
            assert maxabs(f64(dk[b, g]), dK) <= tol, ("dK", b, g, maxabs(f64(dk[b, g]), dK))
            assert maxabs(f64(dv[b, g]), dV) <= tol, ("dV", b, g, maxabs(f64(dv[b, g]), dV))
        else:
            check_close(f64(dk[b, g]), dK, tol, REL_BF16, f"dK[{b},{g}]")
            check_close(f64(dv[b, g]), dV, tol, REL_BF16, f"dV[{b},{g}]")


@pytest.mark.parametrize("name", ["c3a", "c3b"])
def test_fwd_bwd_long_context_complete_heads(name):
    """The long-context shapes (N = 8192; d = 128 with 16 heads, d = 64 with
    32 heads): complete O / LSE and complete dQ / dK / dV of two heads --
    every row, so every query block, key block and tail of the kernels'
    decompositions and the running-max rescaling on real data -- against the
    oracle at the flat bounds (2e-2, LSE 1e-3)."""
    require_gpu()
    p = inputs.PRESETS[name]
    assert p.N == 8192 and p.Hq == p.Hkv
    q, k, v, do = inputs.make_preset(p, with_grad=True)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fwd(qd, kd, vd, scale=p.scale, causal=p.causal)
    dq, dk, dv = bwd(qd, kd, vd, o, lse, dod, scale=p.scale, causal=p.causal)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (t.cpu() for t in (o, lse, dq, dk, dv))
    tol = TOL[torch.bfloat16]
    for b, h in ((0, 0), (p.B - 1, p.Hq - 1)):
        Q, K, V, dO = f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), f64(do[b, h])
        O, LSE = oracle.head_forward(Q, K, V, p.scale, p.causal)
        check_close(f64(o[b, h]), O, tol["out"], None, f"O[{b},{h}]")
        check_close(lse[b, h].numpy(), LSE, tol["lse"], None, f"LSE[{b},{h}]")
        gq, gk, gv = oracle.head_backward(Q, K, V, dO, p.scale, p.causal)
        for nm, got, want in (("dQ", dq, gq), ("dK", dk, gk), ("dV", dv, gv)):
            check_close(f64(got[b, h]), want, tol["out"], None, f"{nm}[{b},{h}]")


def test_bwd_single_token():
    """N = 1: P = 1, so dQ = dK = 0 and dV = dO (sum over the group).  On
    the GPU dS = dP - D is a difference of two fp32 dot products summed in
    different orders, so dQ and dK are zero up to fp32 rounding."""
    require_gpu()
    q, k, v, do = inputs.make(3, 4, 2, 1, 128, torch.bfloat16, 11, with_grad=True)
    dq, dk, dv = _gpu_grads(q, k, v, do, 0.1, True)
    assert float(dq.abs().max()) <= 1e-4 and float(dk.abs().max()) <= 1e-4
    want = do.float().reshape(3, 2, 2, 1, 128).sum(dim=2)  # exact in fp32: a sum of two bf16 values
    check_half_ulp(f64(dv), want.double().numpy(), 0.0, "dV")


def test_bwd_constant_v_full_size():
    """V constant: dP rows are constant so dS = P (dP - D) ~ 0, i.e. dQ and
    dK vanish up to the rounding of O to bf16 (c5 shape, every element)."""
    require_gpu()
    p = inputs.PRESETS["c5"]
    q, k, v, do = inputs.make_preset(p, with_grad=True)
    c = torch.linspace(-1, 1, p.d).to(torch.bfloat16)
    v = c.expand_as(v).contiguous()
    dq, dk, dv = _gpu_grads(q, k, v, do, p.scale, p.causal)
    assert float(dq.abs().max()) <= 2e-2 and float(dk.abs().max()) <= 2e-2
    # dV = P^T dO does not vanish: complete dV of two heads against the oracle
    for b, h in ((0, 0), (p.B - 1, p.Hq - 1)):
        _, _, want = oracle.head_backward(f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), f64(do[b, h]), p.scale,
                                          p.causal)
        check_close(f64(dv[b, h]), want, 2e-2, None, f"dV[{b},{h}]")


def fa_d_term_bytes(B, Hq, N):
    return (B * Hq * N * 4 + 255) // 256 * 256


def test_bwd_deterministic_and_workspace_contents_ignored():
    require_gpu()
    # grouped heads on a small grid: the query heads of each key/value head
    # are split over workgroups whose float partials sit in the workspace
    q, k, v, do = inputs.make(2, 8, 2, 777, 64, torch.bfloat16, 12, with_grad=True)
    need = bwd_workspace_size(2, 8, 2, 777, 64)
    assert need > fa_d_term_bytes(2, 8, 777)
    ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")
    a = _gpu_grads(q, k, v, do, 0.125, True)
    b = _gpu_grads(q, k, v, do, 0.125, True, workspace=ws)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_other_scales():
    require_gpu()
    for scale in (0.0, -0.2, 0.9):
        q, k, v, do = inputs.make(1, 2, 1, 150, 128, torch.bfloat16, 13, with_grad=True)
        dq, dk, dv = _gpu_grads(q, k, v, do, scale, True)
        dQ, dK, dV = oracle.attention_backward(f64(q), f64(k), f64(v), f64(do), scale, True)
        for name, got, want in (("dQ", dq, dQ), ("dK", dk, dK), ("dV", dv, dV)):
            check_close(f64(got), want, 2e-2, REL_BF16, f"{name} scale={scale}")


def test_bwd_d256_unsupported():
    require_gpu()
    q, k, v, do = (t.cuda() for t in inputs.make(1, 1, 1, 16, 256, torch.bfloat16, 1, with_grad=True))
    o, lse = fwd(q, k, v)
    with pytest.raises(FAError, match="UNSUPPORTED"):
        bwd(q, k, v, o, lse, do)


@pytest.mark.parametrize("shape", [(0, 2, 2, 16, 64), (2, 2, 1, 0, 128)])
def test_bwd_empty(shape):
    require_gpu()
    B, Hq, Hkv, N, d = shape
    q = torch.empty((B, Hq, N, d), device="cuda", dtype=torch.bfloat16)
    k = torch.empty((B, Hkv, N, d), device="cuda", dtype=torch.bfloat16)
    lse = torch.empty((B, Hq, N), device="cuda", dtype=torch.float32)
    dq, dk, dv = bwd(q, k, k.clone(), q.clone(), lse, q.clone())
    torch.cuda.synchronize()
    assert dq.shape == q.shape and dk.shape == k.shape
