"""Block-sparse attention, forward and backward, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the HIP library never
imports this module, and this module imports nothing from the HIP library.

Sources (cited by page title and section):

* "Flash attention: fast and memory-efficient exact attention with
  IO-awareness -- a deep dive", closing paragraph: block-sparse
  FlashAttention is named as a variant the page does not cover.
* FlashAttention interview Q&A (app.wittybyte.ai, "FlashAttention1"),
  answer on the challenges of scaling to very long sequences: the method can
  be combined with sparse attention patterns (local or dilated attention),
  and sparse FlashAttention is among the listed future directions.
* The attention itself is the definition of ``oracle.attention`` (standard
  attention Steps 1-3 of the deep-dive page) with more scores hidden.

Reading taken where the pages are silent (listed in the design notes): the
sequence is cut into blocks of ``BLOCK`` = 128 positions; a map
``mask[nb][nb]`` (nb = ceil(N / 128), nonzero = visible), shared by every
batch entry and head, lets query i see key j exactly when
mask[i // 128][j // 128] != 0, and with ``causal`` also j <= i.  A row that
sees no key has no softmax: its output is 0, its LSE is -inf, and it adds
nothing to any gradient (its P row is all zeros).

Everything is float64 and unblocked.
"""

import numpy as np

from .attention import _check_shapes, kv_head_of

__all__ = ["BLOCK", "blocksparse_visible", "blocksparse_forward", "blocksparse_backward"]

BLOCK = 128


def blocksparse_visible(n, mask, causal):
    """Boolean [n, n]: key j visible to query i."""
    mask = np.asarray(mask)
    nb = (n + BLOCK - 1) // BLOCK
    if mask.shape != (nb, nb):
        raise ValueError(f"mask must be [{nb}, {nb}] for N = {n}")
    blk = np.arange(n) // BLOCK
    vis = mask[blk[:, None], blk[None, :]] != 0
    if causal:
        vis &= np.arange(n)[None, :] <= np.arange(n)[:, None]
    return vis


def _probs(q, k, scale, vis):
    """Row softmax of the visible scores; all-hidden rows give P = 0 and
    LSE = -inf instead of 0/0."""
    s = np.where(vis, scale * (q @ k.T), -np.inf)
    any_vis = vis.any(axis=1)
    m = np.where(any_vis, s.max(axis=1), 0.0)
    e = np.where(vis, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    p = np.where(any_vis[:, None], e / np.where(any_vis, l, 1.0)[:, None], 0.0)
    lse = np.where(any_vis, m + np.log(np.where(any_vis, l, 1.0)), -np.inf)
    return p, lse


def blocksparse_forward(Q, K, V, mask, scale, causal):
    """Q [B, H_q, N, d], K/V [B, H_kv, N, d], mask [nb, nb]
    -> (O [B, H_q, N, d_v], LSE [B, H_q, N])."""
    Q, K, V = (np.asarray(x, dtype=np.float64) for x in (Q, K, V))
    B, Hq, Hkv, N, d = _check_shapes(Q, K, V)
    vis = blocksparse_visible(N, mask, causal)
    O = np.zeros((B, Hq, N, V.shape[3]))
    LSE = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            p, lse = _probs(Q[b, h], K[b, g], scale, vis)
            O[b, h] = p @ V[b, g]
            LSE[b, h] = lse
    return O, LSE


def blocksparse_backward(Q, K, V, dO, mask, scale, causal):
    """Analytic backward of ``blocksparse_forward`` -> (dQ, dK, dV): the chain
    rule of ``oracle.attention.head_backward`` with this P (hidden scores and
    rows that see nothing have P = 0)."""
    Q, K, V, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, dO))
    B, Hq, Hkv, N, d = _check_shapes(Q, K, V)
    vis = blocksparse_visible(N, mask, causal)
    dQ = np.zeros(Q.shape)
    dK = np.zeros(K.shape)
    dV = np.zeros(V.shape)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            p, _ = _probs(Q[b, h], K[b, g], scale, vis)
            dp = dO[b, h] @ V[b, g].T
            d_row = (p * dp).sum(axis=1)
            ds = p * (dp - d_row[:, None])
            dQ[b, h] = scale * (ds @ K[b, g])
            dK[b, g] += scale * (ds.T @ Q[b, h])
            dV[b, g] += p.T @ dO[b, h]
    return dQ, dK, dV
