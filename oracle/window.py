"""Local (sliding-window) attention, forward and backward, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the HIP library never
imports this module, and this module imports nothing from the HIP library.

Sources (cited by page title and section):

* FlashAttention interview Q&A (app.wittybyte.ai, "FlashAttention1"): among
  the challenges of very long sequences it proposes combining the method
  with sparse attention such as local attention, and it lists sparse
  FlashAttention among future directions.  The deep-dive page ("Flash
  attention: fast and memory-efficient exact attention with IO-awareness")
  only names block-sparse FlashAttention as a topic it does not cover.
  Neither page defines a pattern.
* The attention itself is the definition of ``oracle.attention`` (standard
  attention Steps 1-3 of the deep-dive page) with more scores hidden.

Reading taken where the pages are silent (listed in the design notes): a
window (left, right) lets query i see key j exactly when
i - left <= j <= i + right, a negative bound meaning unbounded on that side.
(-1, 0) is the causal mask of ``oracle.attention``, (-1, -1) no mask.  With
both bounds >= 0 every row sees at least its own key.

Everything is float64 and unblocked.
"""

import numpy as np

from .attention import _check_shapes, _row_softmax, kv_head_of

__all__ = ["window_visible", "window_forward", "window_backward"]


def window_visible(n, left, right):
    """Boolean [n, n]: key j visible to query i under the window (left, right)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    vis = np.ones((n, n), dtype=bool)
    if left >= 0:
        vis &= j >= i - left
    if right >= 0:
        vis &= j <= i + right
    return vis


def _head_probs(q, k, scale, vis):
    s = np.where(vis, scale * (q @ k.T), -np.inf)
    return _row_softmax(s)


def window_forward(Q, K, V, scale, left, right):
    """Forward with a sliding window: Q [B, H_q, N, d], K/V [B, H_kv, N, d]
    -> (O [B, H_q, N, d_v], LSE [B, H_q, N])."""
    Q, K, V = (np.asarray(x, dtype=np.float64) for x in (Q, K, V))
    B, Hq, Hkv, N, d = _check_shapes(Q, K, V)
    vis = window_visible(N, left, right)
    O = np.zeros((B, Hq, N, V.shape[3]))
    LSE = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            if N == 0:
                continue
            p, m, l = _head_probs(Q[b, h], K[b, g], scale, vis)
            O[b, h] = p @ V[b, g]
            LSE[b, h] = m + np.log(l)
    return O, LSE


def window_backward(Q, K, V, dO, scale, left, right):
    """Analytic backward of ``window_forward`` -> (dQ, dK, dV); the chain rule
    of ``oracle.attention.head_backward`` with the window's P (hidden scores
    have P = 0 and contribute nothing)."""
    Q, K, V, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, dO))
    B, Hq, Hkv, N, d = _check_shapes(Q, K, V)
    vis = window_visible(N, left, right)
    dQ = np.zeros(Q.shape)
    dK = np.zeros(K.shape)
    dV = np.zeros(V.shape)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            if N == 0:
                continue
            p, _, _ = _head_probs(Q[b, h], K[b, g], scale, vis)
            dp = dO[b, h] @ V[b, g].T
            d_row = (p * dp).sum(axis=1)
            ds = p * (dp - d_row[:, None])
            dQ[b, h] = scale * (ds @ K[b, g])
            dK[b, g] += scale * (ds.T @ Q[b, h])
            dV[b, g] += p.T @ dO[b, h]
    return dQ, dK, dV
