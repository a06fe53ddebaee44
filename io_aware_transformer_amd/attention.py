"""Torch-facing binding of the C ABI: argument marshalling only.

``fwd`` and ``bwd`` check devices, dtypes, shapes and contiguity, allocate
outputs with torch on the tensors' device, and pass raw device pointers plus
the current HIP stream to ``fa_fwd`` / ``fa_bwd``.  Every step of the
computation runs in the HIP kernels of libfa.so.
"""

import math

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.FA_BF16, torch.float32: _lib.FA_FP32}


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _on_device(t):
    """Checked last, after every shape / dtype / buffer check, so that all
    argument validation can be exercised without a GPU."""
    if not t.is_cuda:
        raise ValueError("tensors must be on a HIP device")


def _buffer(t, shape, dtype, device, name):
    """A caller-supplied output buffer (``out=``, ``lse=``) must be exactly
    what the kernels write: contiguous, of this shape, dtype and device;
    None allocates one."""
    shape = tuple(int(x) for x in shape)
    if t is None:
        return torch.empty(shape, device=device, dtype=dtype)
    if tuple(t.shape) != shape or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {shape} on {device} "
                         f"(got {t.dtype} {tuple(t.shape)} on {t.device}, contiguous={t.is_contiguous()})")
    return t


def _check(q, k, v, *extra):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for t in (k, v, *extra):
        if t.device != q.device:
            raise ValueError("all tensors must be on the same device")
        if t.dtype != q.dtype:
            raise TypeError("all tensors must share one dtype")
    for t in (q, k, v, *extra):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, d]")
    B, Hq, N, d = q.shape
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("k, v must be [B, H_kv, N, d] matching q")
    return B, Hq, k.shape[1], N, d


def fwd(q, k, v, scale=None, causal=True, out=None, lse=None):
    """Forward pass: returns (o, lse).  o like q; lse float32 [B, H_q, N]."""
    B, Hq, Hkv, N, d = _check(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = _buffer(out, q.shape, q.dtype, q.device, "out")
    lse = _buffer(lse, (B, Hq, N), torch.float32, q.device, "lse")
    _on_device(q)
    lib = _lib.load()
    st = lib.fa_fwd(
        q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None, o.data_ptr() or None,
        lse.data_ptr() or None, B, Hq, Hkv, N, d, float(scale), int(bool(causal)), _DTYPES[q.dtype],
        _stream(q.device),
    )
    _lib.check(st, "fa_fwd")
    return o, lse


def bwd_workspace_size(B, Hq, Hkv, N, d, dtype=torch.bfloat16):
    return int(_lib.load().fa_bwd_workspace_size(B, Hq, Hkv, N, d, _DTYPES[dtype]))


def bwd(q, k, v, o, lse, do, scale=None, causal=True, workspace=None):
    """Backward pass: returns (dq, dk, dv) shaped like q, k, v."""
    B, Hq, Hkv, N, d = _check(q, k, v, o, do)
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, N) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H_q, N]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = bwd_workspace_size(B, Hq, Hkv, N, d, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=q.device, dtype=torch.uint8)
    _on_device(q)
    lib = _lib.load()
    st = lib.fa_bwd(
        q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None, o.data_ptr() or None,
        do.data_ptr() or None, lse.data_ptr() or None, dq.data_ptr() or None, dk.data_ptr() or None,
        dv.data_ptr() or None, workspace.data_ptr() or None, workspace.numel(),
        B, Hq, Hkv, N, d, float(scale), int(bool(causal)), _DTYPES[q.dtype], _stream(q.device),
    )
    _lib.check(st, "fa_bwd")
    return dq, dk, dv


def _check_split(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for t in (k, v):
        if t.device != q.device:
            raise ValueError("all tensors must be on the same device")
        if t.dtype != q.dtype:
            raise TypeError("all tensors must share one dtype")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, d]")
    B, Hq, Nq, d = q.shape
    if k.shape[0] != B or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("k, v must be [B, H_kv, N_k, d] matching q")
    return B, Hq, k.shape[1], Nq, k.shape[2], d


def fwd_split_parts(B, Hq, Hkv, Nq, Nk, d, num_splits=0):
    return int(_lib.load().fa_fwd_split_parts(B, Hq, Hkv, Nq, Nk, d, int(num_splits)))


def fwd_split_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits=0, dtype=torch.bfloat16):
    return int(_lib.load().fa_fwd_split_workspace_size(B, Hq, Hkv, Nq, Nk, d, int(num_splits), _DTYPES[dtype]))


def fwd_split(q, k, v, scale=None, causal=True, num_splits=0, out=None, lse=None, workspace=None):
    """Split key/value forward: q [B, H_q, N_q, d] against k, v [B, H_kv, N_k, d].

    Returns (o like q, lse float32 [B, H_q, N_q]).  ``num_splits`` key
    ranges (0: the library's default); causal aligns the queries with the
    last N_q key positions.
    """
    B, Hq, Hkv, Nq, Nk, d = _check_split(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = _buffer(out, q.shape, q.dtype, q.device, "out")
    lse = _buffer(lse, (B, Hq, Nq), torch.float32, q.device, "lse")
    ws_bytes = fwd_split_workspace_size(B, Hq, Hkv, Nq, Nk, d, num_splits, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=q.device, dtype=torch.uint8)
    _on_device(q)
    lib = _lib.load()
    st = lib.fa_fwd_split(
        q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None, o.data_ptr() or None,
        lse.data_ptr() or None, B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), int(num_splits),
        workspace.data_ptr() or None, workspace.numel(), _DTYPES[q.dtype], _stream(q.device),
    )
    _lib.check(st, "fa_fwd_split")
    return o, lse


def lse_merge(o_parts, lse_parts, dtype=torch.bfloat16, out=None, lse=None):
    """Merge partial results: o_parts float32 [P, ..., d], lse_parts float32
    [P, ...] -> (o [..., d] of ``dtype``, lse float32 [...])."""
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise TypeError("partials must be float32")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()) or lse_parts.device != o_parts.device:
        raise ValueError("partials must be contiguous tensors on one device")
    if o_parts.shape[:-1] != lse_parts.shape or o_parts.dim() < 2:
        raise ValueError("o_parts must be [P, ..., d] and lse_parts [P, ...]")
    P, d = o_parts.shape[0], o_parts.shape[-1]
    rows = lse_parts[0].numel()
    if dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {dtype}")
    o = _buffer(out, o_parts.shape[1:], dtype, o_parts.device, "out")
    lse = _buffer(lse, lse_parts.shape[1:], torch.float32, o_parts.device, "lse")
    _on_device(o_parts)
    st = _lib.load().fa_lse_merge(
        o_parts.data_ptr() or None, lse_parts.data_ptr() or None, P, rows, d, o.data_ptr() or None,
        lse.data_ptr() or None, _DTYPES[dtype], _stream(o_parts.device),
    )
    _lib.check(st, "fa_lse_merge")
    return o, lse


def fwd_window(q, k, v, window, scale=None, out=None, lse=None):
    """Local-attention forward: query i sees keys i - window[0] .. i + window[1]
    (-1: unbounded on that side).  Returns (o, lse) as ``fwd``."""
    B, Hq, Hkv, N, d = _check(q, k, v)
    left, right = (int(x) for x in window)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = _buffer(out, q.shape, q.dtype, q.device, "out")
    lse = _buffer(lse, (B, Hq, N), torch.float32, q.device, "lse")
    _on_device(q)
    st = _lib.load().fa_fwd_window(
        q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None, o.data_ptr() or None,
        lse.data_ptr() or None, B, Hq, Hkv, N, d, float(scale), left, right, _DTYPES[q.dtype], _stream(q.device),
    )
    _lib.check(st, "fa_fwd_window")
    return o, lse


def bwd_window(q, k, v, o, lse, do, window, scale=None, workspace=None):
    """Backward of ``fwd_window`` with the same window: returns (dq, dk, dv)."""
    B, Hq, Hkv, N, d = _check(q, k, v, o, do)
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, N) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H_q, N]")
    left, right = (int(x) for x in window)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = bwd_workspace_size(B, Hq, Hkv, N, d, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=q.device, dtype=torch.uint8)
    _on_device(q)
    st = _lib.load().fa_bwd_window(
        q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None, o.data_ptr() or None,
        do.data_ptr() or None, lse.data_ptr() or None, dq.data_ptr() or None, dk.data_ptr() or None,
        dv.data_ptr() or None, workspace.data_ptr() or None, workspace.numel(),
        B, Hq, Hkv, N, d, float(scale), left, right, _DTYPES[q.dtype], _stream(q.device),
    )
    _lib.check(st, "fa_bwd_window")
    return dq, dk, dv


def _check_varlen(q, k, v, cu_seqlens, *extra):
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be packed [H, total, d]")
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for t in (k, v, *extra):
        if t.device != q.device:
            raise ValueError("all tensors must be on the same device")
        if t.dtype != q.dtype:
            raise TypeError("all tensors must share one dtype")
    for t in (q, k, v, *extra):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [H, total, d]")
    Hq, total, d = q.shape
    if k.shape[1] != total or k.shape[2] != d or v.shape != k.shape:
        raise ValueError("k, v must be [H_kv, total, d] matching q")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of batch + 1 offsets")
    if cu_seqlens.device != q.device or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous tensor on the tensors' device")
    return cu_seqlens.numel() - 1, total, Hq, k.shape[0], d


def fwd_varlen(q, k, v, cu_seqlens, max_seqlen, scale=None, causal=True, out=None, lse=None):
    """Forward over packed sequences of different lengths.

    q [H_q, total, d], k, v [H_kv, total, d]; sequence b is rows
    cu_seqlens[b] .. cu_seqlens[b+1]-1 (int32, on the device) of every head;
    max_seqlen bounds every length.  Returns (o like q, lse float32
    [H_q, total]).
    """
    batch, total, Hq, Hkv, d = _check_varlen(q, k, v, cu_seqlens)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = _buffer(out, q.shape, q.dtype, q.device, "out")
    lse = _buffer(lse, (Hq, total), torch.float32, q.device, "lse")
    _on_device(q)
    st = _lib.load().fa_fwd_varlen(
        q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None, o.data_ptr() or None,
        lse.data_ptr() or None, cu_seqlens.data_ptr() or None, batch, total, int(max_seqlen), Hq, Hkv, d,
        float(scale), int(bool(causal)), _DTYPES[q.dtype], _stream(q.device),
    )
    _lib.check(st, "fa_fwd_varlen")
    return o, lse


def bwd_varlen_workspace_size(total, Hq, Hkv, d, dtype=torch.bfloat16):
    return int(_lib.load().fa_bwd_varlen_workspace_size(total, Hq, Hkv, d, _DTYPES[dtype]))


def bwd_varlen(q, k, v, o, lse, do, cu_seqlens, max_seqlen, scale=None, causal=True, workspace=None):
    """Backward of ``fwd_varlen``: returns (dq, dk, dv) shaped like q, k, v."""
    batch, total, Hq, Hkv, d = _check_varlen(q, k, v, cu_seqlens, o, do)
    if lse.dtype != torch.float32 or lse.shape != (Hq, total) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [H_q, total]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = bwd_varlen_workspace_size(total, Hq, Hkv, d, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=q.device, dtype=torch.uint8)
    _on_device(q)
    st = _lib.load().fa_bwd_varlen(
        q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None, o.data_ptr() or None,
        do.data_ptr() or None, lse.data_ptr() or None, dq.data_ptr() or None, dk.data_ptr() or None,
        dv.data_ptr() or None, workspace.data_ptr() or None, workspace.numel(), cu_seqlens.data_ptr() or None,
        batch, total, int(max_seqlen), Hq, Hkv, d, float(scale), int(bool(causal)), _DTYPES[q.dtype],
        _stream(q.device),
    )
    _lib.check(st, "fa_bwd_varlen")
    return dq, dk, dv


def _check_block_mask(mask, N, device):
    nb = (N + _lib.FA_SPARSE_BLOCK - 1) // _lib.FA_SPARSE_BLOCK
    if mask.dtype not in (torch.uint8, torch.bool) or tuple(mask.shape) != (nb, nb):
        raise ValueError(f"block_mask must be a uint8 or bool tensor of shape ({nb}, {nb}) for N = {N}")
    if mask.device != device or not mask.is_contiguous():
        raise ValueError("block_mask must be a contiguous tensor on the tensors' device")
    return mask


def fwd_blocksparse(q, k, v, block_mask, scale=None, causal=False, out=None, lse=None):
    """Block-sparse forward: query i sees key j when
    block_mask[i // 128, j // 128] is nonzero (and j <= i with causal).
    Rows that see nothing get o = 0, lse = -inf.  Returns (o, lse) as ``fwd``."""
    B, Hq, Hkv, N, d = _check(q, k, v)
    _check_block_mask(block_mask, N, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = _buffer(out, q.shape, q.dtype, q.device, "out")
    lse = _buffer(lse, (B, Hq, N), torch.float32, q.device, "lse")
    _on_device(q)
    st = _lib.load().fa_fwd_blocksparse(
        q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None, o.data_ptr() or None,
        lse.data_ptr() or None, block_mask.data_ptr() or None, B, Hq, Hkv, N, d, float(scale), int(bool(causal)),
        _DTYPES[q.dtype], _stream(q.device),
    )
    _lib.check(st, "fa_fwd_blocksparse")
    return o, lse


def bwd_blocksparse(q, k, v, o, lse, do, block_mask, scale=None, causal=False, workspace=None):
    """Backward of ``fwd_blocksparse`` with the same map: returns (dq, dk, dv)."""
    B, Hq, Hkv, N, d = _check(q, k, v, o, do)
    _check_block_mask(block_mask, N, q.device)
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, N) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H_q, N]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = bwd_workspace_size(B, Hq, Hkv, N, d, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=q.device, dtype=torch.uint8)
    _on_device(q)
    st = _lib.load().fa_bwd_blocksparse(
        q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None, o.data_ptr() or None,
        do.data_ptr() or None, lse.data_ptr() or None, dq.data_ptr() or None, dk.data_ptr() or None,
        dv.data_ptr() or None, workspace.data_ptr() or None, workspace.numel(), block_mask.data_ptr() or None,
        B, Hq, Hkv, N, d, float(scale), int(bool(causal)), _DTYPES[q.dtype], _stream(q.device),
    )
    _lib.check(st, "fa_bwd_blocksparse")
    return dq, dk, dv


def fwd_dropout(q, k, v, dropout_p, seed, offset=0, scale=None, causal=True, out=None, lse=None):
    """Forward with dropout on the attention probabilities (inverted: kept
    terms scaled by 256 / (256 - t8), t8 = round(dropout_p * 256)); the keep
    mask is a function of (seed, offset, batch, head, query, key).  LSE is
    that of the softmax without dropout.  Returns (o, lse) as ``fwd``."""
    B, Hq, Hkv, N, d = _check(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = _buffer(out, q.shape, q.dtype, q.device, "out")
    lse = _buffer(lse, (B, Hq, N), torch.float32, q.device, "lse")
    _on_device(q)
    st = _lib.load().fa_fwd_dropout(
        q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None, o.data_ptr() or None,
        lse.data_ptr() or None, B, Hq, Hkv, N, d, float(scale), int(bool(causal)), float(dropout_p),
        int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 32 - 1), _DTYPES[q.dtype], _stream(q.device),
    )
    _lib.check(st, "fa_fwd_dropout")
    return o, lse


def bwd_dropout(q, k, v, o, lse, do, dropout_p, seed, offset=0, scale=None, causal=True, workspace=None):
    """Backward of ``fwd_dropout`` with the same dropout_p, seed and offset:
    returns (dq, dk, dv)."""
    B, Hq, Hkv, N, d = _check(q, k, v, o, do)
    if lse.dtype != torch.float32 or lse.shape != (B, Hq, N) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H_q, N]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = bwd_workspace_size(B, Hq, Hkv, N, d, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=q.device, dtype=torch.uint8)
    _on_device(q)
    st = _lib.load().fa_bwd_dropout(
        q.data_ptr() or None, k.data_ptr() or None, v.data_ptr() or None, o.data_ptr() or None,
        do.data_ptr() or None, lse.data_ptr() or None, dq.data_ptr() or None, dk.data_ptr() or None,
        dv.data_ptr() or None, workspace.data_ptr() or None, workspace.numel(), B, Hq, Hkv, N, d, float(scale),
        int(bool(causal)), float(dropout_p), int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 32 - 1),
        _DTYPES[q.dtype], _stream(q.device),
    )
    _lib.check(st, "fa_bwd_dropout")
    return dq, dk, dv
