"""Split key/value forward (fa_fwd_split) and the merge of partials
(fa_lse_merge) against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, check_half_ulp, f64, maxabs, require_gpu
from io_aware_transformer_amd import fwd, fwd_split, fwd_split_parts, inputs, lse_merge

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF = torch.bfloat16


def run_and_check(B, Hq, Hkv, Nq, Nk, d, causal, splits, seed, scale=None):
    require_gpu()
    q, k, v = inputs.make_split(B, Hq, Hkv, Nq, Nk, d, BF, seed)
    sc = d ** -0.5 if scale is None else scale
    o, lse = fwd_split(q.to(DEV), k.to(DEV), v.to(DEV), scale=sc, causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    want_o, want_l = oracle.cross_forward(f64(q), f64(k), f64(v), sc, causal)
    got_o, got_l = f64(o), lse.cpu().numpy().astype(np.float64)
    live = np.isfinite(want_l)
    # rows that see no key: output exactly 0, LSE -inf
    assert np.array_equal(np.isfinite(got_l), live)
    assert np.all(got_o[~live] == 0)
    err_o = maxabs(got_o[live], want_o[live])
    err_l = maxabs(got_l[live], want_l[live])
    assert err_o <= TOL[BF]["out"], f"O max-abs {err_o}"
    assert err_l <= TOL[BF]["lse"], f"LSE max-abs {err_l}"
    return o, lse


SHAPES = [
    # B, Hq, Hkv, Nq, Nk, d
    (1, 1, 1, 1, 1, 64),
    (2, 4, 2, 1, 100, 128),
    (1, 8, 1, 3, 257, 64),
    (2, 4, 4, 17, 300, 128),
    (1, 2, 1, 40, 33, 64),      # N_q > N_k: under the causal mask the first rows see nothing
    (1, 32, 8, 1, 1000, 128),   # grouped heads: 4 query heads per kv head packed in one block
    (1, 4, 1, 9, 2049, 128),    # 36 packed rows: two row blocks, ragged key tail
    (1, 64, 1, 1, 513, 64),     # 64 query heads on one kv head: two full row blocks
]


@pytest.mark.parametrize("splits", [1, 3, 0])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}Hq{}Hkv{}Nq{}Nk{}d{}".format(*s))
def test_split_small(shape, causal, splits):
    run_and_check(*shape, causal=causal, splits=splits, seed=hash((shape, causal, splits)) % 1000)


def test_split_more_parts_than_tiles():
    # 40 key ranges over 70 keys: most ranges are empty and merge as nothing
    run_and_check(2, 4, 2, 2, 70, 64, causal=True, splits=40, seed=5)


@pytest.mark.parametrize("scale", [0.0, -0.3, 1.1])
def test_split_other_scales(scale):
    run_and_check(1, 8, 2, 5, 400, 128, causal=True, splits=4, seed=6, scale=scale)


def test_split_matches_square_forward():
    # N_q = N_k: the same attention as fa_fwd; both within tolerance of the oracle, and of each other
    require_gpu()
    q, k, v = inputs.make_split(2, 4, 2, 150, 150, 128, BF, 7)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, l1 = fwd_split(qd, kd, vd, causal=True, num_splits=3)
    o2, l2 = fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    want_o, want_l = oracle.cross_forward(f64(q), f64(k), f64(v), 128 ** -0.5, True)
    assert maxabs(f64(o1), want_o) <= TOL[BF]["out"] and maxabs(f64(o2), want_o) <= TOL[BF]["out"]
    assert maxabs(l1.cpu().numpy(), want_l) <= TOL[BF]["lse"]
    assert maxabs(f64(o1), f64(o2)) <= 2 * TOL[BF]["out"]


def test_split_deterministic():
    require_gpu()
    q, k, v = (t.to(DEV) for t in inputs.make_split(2, 16, 4, 2, 3000, 128, BF, 8))
    a = fwd_split(q, k, v, causal=True, num_splits=0)
    b = fwd_split(q, k, v, causal=True, num_splits=0)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("name", sorted(inputs.SPLIT_PRESETS))
def test_split_presets_full(name):
    """Full-size decoding presets, every row against the oracle (N_q is small,
    so the fp64 reference over all (batch, head) units is cheap)."""
    require_gpu()
    p = inputs.SPLIT_PRESETS[name]
    q, k, v = inputs.make_split_preset(p)
    o, lse = fwd_split(q.to(DEV), k.to(DEV), v.to(DEV), scale=p.scale, causal=p.causal, num_splits=0)
    torch.cuda.synchronize()
    parts = fwd_split_parts(p.B, p.Hq, p.Hkv, p.Nq, p.Nk, p.d, 0)
    assert parts >= 1
    qq, kk, vv = f64(q), f64(k), f64(v)
    for b in range(p.B):
        want_o, want_l = oracle.cross_forward(qq[b:b + 1], kk[b:b + 1], vv[b:b + 1], p.scale, p.causal)
        assert maxabs(f64(o[b:b + 1]), want_o) <= TOL[BF]["out"], (name, b)
        assert maxabs(lse[b:b + 1].cpu().numpy(), want_l) <= TOL[BF]["lse"], (name, b)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("parts,rows", [(1, 1), (2, 5), (7, 300), (8, 4), (37, 300), (128, 40)])
@pytest.mark.parametrize("dtype", [torch.float32, BF], ids=["fp32", "bf16"])
def test_merge(d, parts, rows, dtype):
    require_gpu()
    g = torch.Generator().manual_seed(d * 1000 + parts * 10 + rows)
    o_parts = torch.randn((parts, rows, d), generator=g, dtype=torch.float32)
    lse_parts = torch.randn((parts, rows), generator=g, dtype=torch.float32) * 20.0
    # some parts saw no key; row 0 of the first part set, and (with >1 part) a row where every part is empty
    lse_parts[0, 0] = -float("inf")
    o_parts[0, 0] = 0.0
    if rows > 3:
        lse_parts[:, 3] = -float("inf")
        o_parts[:, 3] = 0.0
    o, lse = lse_merge(o_parts.to(DEV), lse_parts.to(DEV), dtype=dtype)
    torch.cuda.synchronize()
    want_o, want_l = oracle.merge_partials(o_parts.numpy(), lse_parts.numpy())
    got_l = lse.cpu().numpy().astype(np.float64)
    live = np.isfinite(want_l)
    assert np.array_equal(np.isfinite(got_l), live)
    assert maxabs(got_l[live], want_l[live]) <= 1e-5 * max(1.0, float(np.max(np.abs(want_l[live]), initial=0)))
    got_o = f64(o)
    assert np.all(got_o[~live] == 0)
    if dtype == torch.float32:
        assert maxabs(got_o, want_o) <= 1e-5
    else:
        check_half_ulp(got_o, want_o, 2e-6, "merged O")
