"""The allocation-free backward (fa_bwd_noalloc) against fa_bwd, through
the C ABI: the same kernels with the D_i term in the library's fixed
per-device buffer instead of a caller workspace, so the gradients must be
bit-identical.  Two calls in a row, the second smaller, on one stream."""

import pytest
import torch

from gpu_util import require_gpu
from io_aware_transformer_amd import _lib, bwd, fwd, inputs

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _noalloc(q, k, v, o, lse, do, scale, causal):
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = _lib.load().fa_bwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
        dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, N, d, float(scale), int(causal), _lib.FA_BF16,
        torch.cuda.current_stream().cuda_stream)
    _lib.check(st, "fa_bwd_noalloc")
    return dq, dk, dv


@pytest.mark.parametrize("d", [64, 128])
def test_noalloc_equals_bwd_two_calls(d):
    require_gpu()
    # second call smaller than the first: the shared buffer keeps the first
    # call's D terms, which the second must not read
    shapes = [(2, 8, 2, 1000, True), (1, 4, 4, 300, False)]
    for i, (B, Hq, Hkv, N, causal) in enumerate(shapes):
        q, k, v, do = (t.cuda() for t in inputs.make(B, Hq, Hkv, N, d, BF, 4100 + 10 * i + d, with_grad=True))
        scale = d ** -0.5
        o, lse = fwd(q, k, v, scale=scale, causal=causal)
        want = bwd(q, k, v, o, lse, do, scale=scale, causal=causal)
        got = _noalloc(q, k, v, o, lse, do, scale, causal)
        torch.cuda.synchronize()
        assert torch.equal(got[0], want[0]), ("dQ", B, Hq, Hkv, N, d)
        for name, x, y in zip(("dK", "dV"), got[1:], want[1:]):
            if Hq == Hkv:
                assert torch.equal(x, y), (name, B, Hq, Hkv, N, d)
            else:
                # fa_bwd splits a grouped head's query heads over several
                # workgroups and sums their float partials; the buffer-free
                # call sums the group in one workgroup.  Both round one float
                # sum to bf16, so they differ by at most one bf16 ulp.
                x, y = x.float(), y.float()
                assert torch.all((x - y).abs() <= 2.0 ** -7 * torch.maximum(x.abs(), y.abs()) + 1e-6), (name, B, Hq,
                                                                                                     Hkv, N, d)


def test_noalloc_rejects_sizes_past_the_buffer():
    require_gpu()
    lib = _lib.load()
    fake = 0x10000  # never dereferenced: the size check fails first
    N = _lib.FA_NOALLOC_MAX_ROWS // 16 + 1
    st = lib.fa_bwd_noalloc(*([fake] * 9), 1, 16, 16, N, 128, 0.1, 1, _lib.FA_BF16, None)
    assert _lib.STATUS[st] == "FA_ERR_WORKSPACE"
    # at the limit the size check passes and validation reaches the pointers
    st = lib.fa_bwd_noalloc(*([None] * 9), 1, 16, 16, N - 1, 128, 0.1, 1, _lib.FA_BF16, None)
    assert _lib.STATUS[st] == "FA_ERR_NULL"
