"""Python binding checks that need no GPU: every entry point that takes a
caller-supplied output buffer (``out=``, ``lse=``) rejects one that is not
exactly what the kernels write, before anything reaches the C ABI.  CPU
tensors pass every check up to the final device check, so a valid call
fails only with "must be on a HIP device"."""

import pytest
import torch

from io_aware_transformer_amd import fwd, fwd_split, fwd_varlen, fwd_window, lse_merge

BF = torch.bfloat16


def _qkv(B=1, Hq=2, Hkv=1, N=16, d=64, dtype=BF):
    q = torch.zeros((B, Hq, N, d), dtype=dtype)
    k = torch.zeros((B, Hkv, N, d), dtype=dtype)
    return q, k, k.clone()


def _bad_outs(shape, dtype):
    """Wrong dtype, wrong shape, missing dimension, non-contiguous view."""
    good = torch.zeros(shape, dtype=dtype)
    other = torch.float32 if dtype != torch.float32 else BF
    yield torch.zeros(shape, dtype=other)
    yield torch.zeros((*shape[:-1], shape[-1] + 1), dtype=dtype)
    yield torch.zeros(shape[1:], dtype=dtype)
    big = torch.zeros((*shape[:-1], 2 * shape[-1]), dtype=dtype)
    yield big[..., ::2]
    assert good.is_contiguous()


def _calls():
    q, k, v = _qkv()
    B, Hq, N, d = q.shape
    qs = torch.zeros((1, 2, 3, 64), dtype=BF)
    cu = torch.tensor([0, 16], dtype=torch.int32)
    qv, kv, vv = q[0], k[0], v[0]
    o_parts, l_parts = torch.zeros((3, 5, 64)), torch.zeros((3, 5))
    return [
        ("fwd", lambda out, lse: fwd(q, k, v, out=out, lse=lse), q.shape, (B, Hq, N), BF),
        ("fwd_window", lambda out, lse: fwd_window(q, k, v, (4, 0), out=out, lse=lse), q.shape, (B, Hq, N), BF),
        ("fwd_split", lambda out, lse: fwd_split(qs, k, v, out=out, lse=lse), qs.shape, (1, 2, 3), BF),
        ("fwd_varlen", lambda out, lse: fwd_varlen(qv, kv, vv, cu, 16, out=out, lse=lse), qv.shape, (2, 16), BF),
        ("lse_merge", lambda out, lse: lse_merge(o_parts, l_parts, BF, out=out, lse=lse), (5, 64), (5,), BF),
    ]


@pytest.mark.parametrize("i", range(5))
def test_bad_out_rejected(i):
    name, call, oshape, lshape, dt = _calls()[i]
    for bad in _bad_outs(oshape, dt):
        with pytest.raises(ValueError, match="out must be"):
            call(bad, None)


@pytest.mark.parametrize("i", range(5))
def test_bad_lse_rejected(i):
    name, call, oshape, lshape, dt = _calls()[i]
    for bad in _bad_outs(lshape, torch.float32):
        with pytest.raises(ValueError, match="lse must be"):
            call(None, bad)


@pytest.mark.parametrize("i", range(5))
def test_good_buffers_reach_the_device_check(i):
    name, call, oshape, lshape, dt = _calls()[i]
    with pytest.raises(ValueError, match="HIP device"):
        call(torch.zeros(oshape, dtype=dt), torch.zeros(lshape, dtype=torch.float32))
    with pytest.raises(ValueError, match="HIP device"):
        call(None, None)


def test_block_mask_validated_before_the_device_check():
    from io_aware_transformer_amd import bwd_blocksparse, fwd_blocksparse

    q, k, v = _qkv(N=300)
    good = torch.ones((3, 3), dtype=torch.uint8)
    for bad in (torch.ones((2, 2), dtype=torch.uint8), torch.ones((3, 3), dtype=torch.int32),
                torch.ones((3, 6), dtype=torch.uint8)[:, ::2]):
        with pytest.raises(ValueError, match="block_mask"):
            fwd_blocksparse(q, k, v, bad)
    with pytest.raises(ValueError, match="HIP device"):
        fwd_blocksparse(q, k, v, good)
    lse = torch.zeros((1, 2, 300))
    with pytest.raises(ValueError, match="block_mask"):
        bwd_blocksparse(q, k, v, q, lse, q, torch.ones((4, 4), dtype=torch.uint8))
