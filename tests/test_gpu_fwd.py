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
    """Full-size presets: complete O / LSE of two heads and sampled rows of a
    third (every query-block edge of 32, 64, 128 and 256 rows among them)
    against the oracle, plus properties that hold for every row."""
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
    edge = [0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 256, 257, 511, 512, 513, p.N // 2, p.N - 257, p.N - 256,
            p.N - 2, p.N - 1]
    rows = sorted(set(edge + [int(x) for x in rng.integers(0, p.N, 20)]))
    tol = TOL[p.torch_dtype]
    G = p.Hq // p.Hkv
    for b, h in sorted(units)[:2]:
        O, LSE = oracle.head_forward(Q[b, h].astype(np.float64), K[b, h // G].astype(np.float64),
                                     V[b, h // G].astype(np.float64), p.scale, p.causal)
        eo, el = maxabs(of[b, h], O), maxabs(lf[b, h], LSE)
        assert eo <= tol["out"], ("complete head", b, h, eo)
        assert el <= tol["lse"], ("complete head", b, h, el)
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


# Launches with more (query block, head) items than compute units and short
# items (causal N up to about 3.8K, non-causal up to 2K, windows) run
# persistent: one workgroup per compute unit takes several items in a row.
# Every item's arithmetic is the same whichever workgroup runs it, so a head
# of such a launch equals, bit for bit, the same head computed in a launch
# of one item per workgroup (a few heads alone).
STREAMED = [  # B, Hq, Hkv, N, d, causal: B * Hq * ceil(N / 256) > 256 items
    (1, 96, 96, 1000, 128, True),
    (2, 64, 16, 700, 128, True),
    (1, 160, 40, 520, 64, True),
    (3, 48, 48, 600, 128, False),
    (1, 192, 12, 300, 64, False),
]


@pytest.mark.parametrize("shape", STREAMED, ids=lambda s: "B{}Hq{}Hkv{}N{}d{}{}".format(*s[:5], "c" if s[5] else "n"))
def test_fwd_streamed_launch(shape):
    require_gpu()
    B, Hq, Hkv, N, d, causal = shape
    G = Hq // Hkv
    q, k, v = (t.cuda() for t in inputs.make(B, Hq, Hkv, N, d, torch.bfloat16, 900 + N + d))
    o, lse = fwd(q, k, v, causal=causal)
    # the first and last key/value head's query heads, alone (one item per workgroup)
    for b, g in ((0, 0), (B - 1, Hkv - 1)):
        hs = slice(g * G, (g + 1) * G)
        o1, l1 = fwd(q[b:b + 1, hs].contiguous(), k[b:b + 1, g:g + 1].contiguous(), v[b:b + 1, g:g + 1].contiguous(),
                     causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1[0], o[b, hs]) and torch.equal(l1[0], lse[b, hs]), (b, g)
    # and the oracle on two heads
    for b, h in ((0, 0), (B - 1, Hq - 1)):
        g = h // G
        O, LSE = oracle.head_forward(f64(q[b, h]), f64(k[b, g]), f64(v[b, g]), d ** -0.5, causal)
        assert maxabs(f64(o[b, h]), O) <= TOL[torch.bfloat16]["out"]
        assert maxabs(lse[b, h].cpu().numpy(), LSE) <= TOL[torch.bfloat16]["lse"]


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_streamed_window_and_dropout(d):
    """The window and dropout kernels take the persistent launch as well."""
    require_gpu()
    from io_aware_transformer_amd import fwd_dropout, fwd_window

    B, H, N = 2, 96, 900
    q, k, v = (t.cuda() for t in inputs.make(B, H, H, N, d, torch.bfloat16, 950 + d))
    ow, lw = fwd_window(q, k, v, (300, 0))
    od, ld = fwd_dropout(q, k, v, 0.2, 77, 3)
    hs = slice(H - 3, H)
    ow1, lw1 = fwd_window(q[1:, hs].contiguous(), k[1:, hs].contiguous(), v[1:, hs].contiguous(), (300, 0))
    torch.cuda.synchronize()
    assert torch.equal(ow1[0], ow[1, hs]) and torch.equal(lw1[0], lw[1, hs])
    # dropout: the keep mask depends on (b, h) of the full batch, so compare with the oracle
    h = H - 1
    O, LSE = oracle.dropout_head_forward(f64(q[1, h]), f64(k[1, h]), f64(v[1, h]), d ** -0.5, True, 0.2, 77, 3,
                                         1 * H + h)
    assert maxabs(f64(od[1, h]), O) <= TOL[torch.bfloat16]["out"]
    assert maxabs(ld[1, h].cpu().numpy(), LSE) <= TOL[torch.bfloat16]["lse"]
    Ow, LSEw = oracle.window_forward(f64(q[:1, 5:6]), f64(k[:1, 5:6]), f64(v[:1, 5:6]), d ** -0.5, 300, 0)
    assert maxabs(f64(ow[:1, 5:6]), Ow) <= TOL[torch.bfloat16]["out"]
    assert maxabs(lw[:1, 5:6].cpu().numpy(), LSEw) <= TOL[torch.bfloat16]["lse"]


def test_fwd_streamed_launch_beyond_item_table():
    """More (query block, head) items than 512 per compute unit: the launch
    grows its grid past one workgroup per compute unit so that no workgroup
    holds more items than its LDS table (B3 H65535 N256 d64 causal: 196605
    items).  Heads of that launch equal, bit for bit, the same heads in
    launches of one item per workgroup.  Inputs are drawn on the device
    (26 GB of Q, K, V and O)."""
    require_gpu()
    B, H, N, d = 3, 65535, 256, 64
    g = torch.Generator(device="cuda").manual_seed(4242)
    q = torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16)
    o, lse = fwd(q, k, v, causal=True)
    for b, h in ((0, 0), (1, 31337), (2, H - 4)):
        hs = slice(h, h + 4)
        o1, l1 = fwd(q[b:b + 1, hs].contiguous(), k[b:b + 1, hs].contiguous(), v[b:b + 1, hs].contiguous(),
                     causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o1[0], o[b, hs]) and torch.equal(l1[0], lse[b, hs]), (b, h)
    O, LSE = oracle.head_forward(f64(q[2, H - 1]), f64(k[2, H - 1]), f64(v[2, H - 1]), d ** -0.5, True)
    assert maxabs(f64(o[2, H - 1]), O) <= TOL[torch.bfloat16]["out"]
    assert maxabs(lse[2, H - 1].cpu().numpy(), LSE) <= TOL[torch.bfloat16]["lse"]
    del q, k, v, o, lse
    torch.cuda.empty_cache()
