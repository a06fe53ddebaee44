"""Block-sparse attention, forward and backward, against the fp64 oracle,
through the C ABI (fa_fwd_blocksparse / fa_bwd_blocksparse)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import REL_BF16, TOL, check_close, f64, maxabs, require_gpu
from io_aware_transformer_amd import FAError, bwd_blocksparse, fwd, fwd_blocksparse, inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF = torch.bfloat16
BLOCK = 128


def _map(nb, density, seed, diag=False):
    rng = np.random.default_rng(seed)
    m = (rng.random((nb, nb)) < density).astype(np.uint8)
    if diag:
        np.fill_diagonal(m, 1)
    return m


def _check_lse(got, want, tol):
    """Finite entries within tol; rows that see nothing are -inf on both sides."""
    got = np.asarray(got, dtype=np.float64)
    inf = np.isinf(want)
    assert np.array_equal(np.isinf(got), inf) and np.all(got[inf] < 0)
    if (~inf).any():
        assert maxabs(got[~inf], want[~inf]) <= tol


SHAPES = [(1, 2, 1, 129), (2, 4, 4, 300), (1, 4, 2, 520), (1, 2, 2, 1000)]  # B, Hq, Hkv, N
MAPS = [("half", 0.5, False), ("sparse", 0.25, False), ("banded", 0.3, True), ("ones", 1.0, False)]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", MAPS, ids=lambda m: m[0])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}Hq{}Hkv{}N{}".format(*s))
def test_blocksparse_fwd_bwd(shape, kind, causal, d):
    require_gpu()
    B, Hq, Hkv, N = shape
    nb = (N + BLOCK - 1) // BLOCK
    name, density, diag = kind
    mask = _map(nb, density, 97 * N + d + int(causal), diag)
    q, k, v, do = inputs.make(B, Hq, Hkv, N, d, BF, 5000 + N + d, with_grad=True)
    sc = d ** -0.5
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    md = torch.from_numpy(mask).to(DEV)
    o, lse = fwd_blocksparse(qd, kd, vd, md, scale=sc, causal=causal)
    dq, dk, dv = bwd_blocksparse(qd, kd, vd, o, lse, dod, md, scale=sc, causal=causal)
    torch.cuda.synchronize()
    want_o, want_l = oracle.blocksparse_forward(f64(q), f64(k), f64(v), mask, sc, causal)
    check_close(f64(o), want_o, TOL[BF]["out"], None, "O")
    _check_lse(lse.cpu().numpy(), want_l, TOL[BF]["lse"])
    gq, gk, gv = oracle.blocksparse_backward(f64(q), f64(k), f64(v), f64(do), mask, sc, causal)
    if Hq == Hkv and not (causal and name == "banded"):
        for nm, got, want in (("dQ", dq, gq), ("dK", dk, gk), ("dV", dv, gv)):
            check_close(f64(got), want, TOL[BF]["out"], None, nm)
        return
    # Grouped heads sum the group into dK / dV; a banded map with causal
    # leaves the first rows of a visible diagonal block seeing only a few
    # keys (as a narrow window does), so P concentrates near 1 and dV / dK
    # reach magnitude 4 and more with few summands: the bound adds each
    # element's own bf16 half ulp to the magnitude-scaled one (worst seen:
    # B2 Hq4 Hkv4 N300 banded causal d 128, dV[1, 3, 0, 89] = 4.28125
    # against 4.26086).
    check_close(f64(dq), gq, TOL[BF]["out"], REL_BF16, "dQ", own_ulp=True)
    check_close(f64(dk), gk, TOL[BF]["out"], REL_BF16, "dK", own_ulp=True)
    check_close(f64(dv), gv, TOL[BF]["out"], REL_BF16, "dV", own_ulp=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_blocksparse_all_ones_forward_equals_dense(d, causal):
    """An all-ones map visits the same tiles in the same order as the dense
    forward kernels: O and LSE are bit-identical to fa_fwd."""
    require_gpu()
    B, Hq, Hkv, N = 2, 4, 2, 700
    q, k, v = (t.to(DEV) for t in inputs.make(B, Hq, Hkv, N, d, BF, 61 + d))
    nb = (N + BLOCK - 1) // BLOCK
    ones = torch.ones((nb, nb), dtype=torch.uint8, device=DEV)
    a = fwd_blocksparse(q, k, v, ones, causal=causal)
    b = fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("d", [64, 128])
def test_blocksparse_rows_that_see_nothing(d):
    """Query blocks whose map row is empty: O = 0 and LSE = -inf exactly, dQ =
    0 there, and keys no query sees get dK = dV = 0."""
    require_gpu()
    B, Hq, Hkv, N = 1, 2, 2, 500
    mask = np.array([[1, 0, 0, 1], [0, 0, 0, 0], [1, 1, 0, 0], [0, 0, 0, 1]], dtype=np.uint8)  # key block 2 unseen
    q, k, v, do = (t.to(DEV) for t in inputs.make(B, Hq, Hkv, N, d, BF, 77, with_grad=True))
    md = torch.from_numpy(mask).to(DEV)
    for causal in (False, True):
        o, lse = fwd_blocksparse(q, k, v, md, causal=causal)
        dq, dk, dv = bwd_blocksparse(q, k, v, o, lse, do, md, causal=causal)
        torch.cuda.synchronize()
        assert torch.all(o[:, :, 128:256] == 0) and torch.all(torch.isneginf(lse[:, :, 128:256]))
        assert torch.all(dq[:, :, 128:256] == 0)
        assert torch.all(dk[:, :, 256:384] == 0) and torch.all(dv[:, :, 256:384] == 0)
        assert torch.isfinite(o).all() and torch.isfinite(dq).all() and torch.isfinite(dk).all()
        want_o, want_l = oracle.blocksparse_forward(f64(q), f64(k), f64(v), mask, d ** -0.5, causal)
        check_close(f64(o), want_o, TOL[BF]["out"], None, "O")
        _check_lse(lse.cpu().numpy(), want_l, TOL[BF]["lse"])


def test_blocksparse_long_sequence_sampled():
    """N = 8192, d = 128, a local band of three blocks plus the first key
    block for every query (a sliding window with a global block): complete
    O / LSE and dQ / dK / dV of one head against the oracle."""
    require_gpu()
    B, H, N, d = 1, 4, 8192, 128
    nb = N // BLOCK
    mask = np.zeros((nb, nb), dtype=np.uint8)
    for i in range(nb):
        mask[i, max(0, i - 2):i + 1] = 1
        mask[i, 0] = 1
    q, k, v, do = inputs.make(B, H, H, N, d, BF, 8100, with_grad=True)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    md = torch.from_numpy(mask).to(DEV)
    o, lse = fwd_blocksparse(qd, kd, vd, md, causal=True)
    dq, dk, dv = bwd_blocksparse(qd, kd, vd, o, lse, dod, md, causal=True)
    torch.cuda.synchronize()
    h = 3
    sc = d ** -0.5
    want_o, want_l = oracle.blocksparse_forward(f64(q[:, h:h + 1]), f64(k[:, h:h + 1]), f64(v[:, h:h + 1]), mask, sc,
                                                True)
    check_close(f64(o[:, h:h + 1]), want_o, TOL[BF]["out"], None, "O")
    _check_lse(lse[:, h:h + 1].cpu().numpy(), want_l, TOL[BF]["lse"])
    gq, gk, gv = oracle.blocksparse_backward(f64(q[:, h:h + 1]), f64(k[:, h:h + 1]), f64(v[:, h:h + 1]),
                                             f64(do[:, h:h + 1]), mask, sc, True)
    for name, got, want in (("dQ", dq, gq), ("dK", dk, gk), ("dV", dv, gv)):
        check_close(f64(got[:, h:h + 1]), want, TOL[BF]["out"], None, name)


def test_blocksparse_rejects():
    require_gpu()
    q, k, v = (t.to(DEV) for t in inputs.make(1, 2, 1, 200, 128, BF, 1))
    good = torch.ones((2, 2), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        fwd_blocksparse(q, k, v, torch.ones((3, 3), dtype=torch.uint8, device=DEV))
    q2, k2, v2 = (t.to(DEV) for t in inputs.make(1, 2, 1, 200, 256, BF, 1))
    with pytest.raises(FAError, match="UNSUPPORTED"):
        fwd_blocksparse(q2, k2, v2, good)
    qf, kf, vf = (t.to(DEV) for t in inputs.make(1, 2, 1, 200, 64, torch.float32, 1))
    with pytest.raises(FAError, match="UNSUPPORTED"):
        fwd_blocksparse(qf, kf, vf, good)
