"""Attention over split key ranges and the merge of partial results, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the HIP library never
imports this module, and this module imports nothing from the HIP library.

Sources (cited by page title and section):

* FlashAttention interview Q&A (app.wittybyte.ai, problem "FlashAttention1"),
  the answer on how softmax is handled: each block keeps its own maximum and
  sum of exponentials, and two blocks combine by rescaling both sums to the
  larger maximum.  The same page's list of what the method makes possible
  names combining partial results computed over different blocks, and
  incremental (streaming) attention.  A partial result over a block of keys
  is (O_p, LSE_p) with LSE_p = m_p + ln l_p; the combine rule is that
  recurrence applied to whole partials:
      LSE = ln sum_p exp(LSE_p),   O = sum_p exp(LSE_p - LSE) O_p.
* Deep-dive page ("Flash attention: fast and memory-efficient exact
  attention with IO-awareness"), standard attention Steps 1-3: the result
  being combined is plain attention over the union of the blocks.

Readings taken where the pages are silent (listed in the design notes):

* queries and keys of different lengths: under the causal mask the N_q
  queries are the LAST N_q positions of the N_k-long key sequence, so key j
  is hidden from query i when j > i + (N_k - N_q).  With N_q = N_k this is
  the square rule of ``oracle.attention``; a single query (decoding) sees
  every key.
* a row with no visible key (only possible when N_q > N_k under the causal
  mask, or for a key block that lies wholly in a row's future) has output 0
  and LSE = -inf; it contributes nothing when merged.

Everything is float64 and unblocked: one score matrix per (batch, query
head), exactly as in ``oracle.attention``.
"""

import numpy as np

from .attention import kv_head_of

__all__ = ["cross_forward", "partial_forward", "merge_partials"]


def _visible(n_q, n_k, causal, k_begin=0, k_end=None):
    """Boolean [n_q, n_k] matrix: key j is visible to query i.

    Causal reading (bottom-right alignment): visible when j <= i + n_k - n_q.
    Keys outside [k_begin, k_end) are not visible (partial results).
    """
    k_end = n_k if k_end is None else k_end
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    vis = np.broadcast_to((j >= k_begin) & (j < k_end), (n_q, n_k))
    if causal:
        vis = vis & (j <= i + (n_k - n_q))
    return vis


def _head(q, k, v, scale, vis):
    """Softmax attention of one unit over the visible keys of each row.

    Rows with no visible key get output 0 and LSE -inf.
    """
    s = np.where(vis, scale * (q @ k.T), -np.inf)
    o = np.zeros((q.shape[0], v.shape[1]))
    lse = np.full(q.shape[0], -np.inf)
    live = vis.any(axis=1)
    if live.any():
        sl = s[live]
        m = sl.max(axis=1)
        e = np.exp(sl - m[:, None])
        l = e.sum(axis=1)
        o[live] = (e / l[:, None]) @ v
        lse[live] = m + np.log(l)
    return o, lse


def _check(Q, K, V):
    if Q.ndim != 4 or K.ndim != 4 or V.ndim != 4:
        raise ValueError("expected [B, H, N, d] arrays")
    B, Hq, n_q, d = Q.shape
    if K.shape[0] != B or K.shape[3] != d or V.shape[:3] != K.shape[:3]:
        raise ValueError("K must be [B, H_kv, N_k, d] and V [B, H_kv, N_k, d_v], matching Q")
    if Hq % K.shape[1] != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    return B, Hq, K.shape[1], n_q, K.shape[2]


def partial_forward(Q, K, V, scale, causal, k_begin, k_end):
    """Attention of every query over the keys in [k_begin, k_end) only.

    Q [B, H_q, N_q, d], K/V [B, H_kv, N_k, d] -> (O_p [B, H_q, N_q, d_v],
    LSE_p [B, H_q, N_q]).  The causal rule uses global key positions.  This
    is the partial result a block of keys contributes.
    """
    Q, K, V = (np.asarray(x, dtype=np.float64) for x in (Q, K, V))
    B, Hq, Hkv, n_q, n_k = _check(Q, K, V)
    vis = _visible(n_q, n_k, causal, k_begin, k_end)
    O = np.zeros((B, Hq, n_q, V.shape[3]))
    LSE = np.full((B, Hq, n_q), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            O[b, h], LSE[b, h] = _head(Q[b, h], K[b, g], V[b, g], scale, vis)
    return O, LSE


def cross_forward(Q, K, V, scale, causal):
    """Plain attention with N_q queries against N_k keys -> (O, LSE).

    The definition (deep-dive page, standard attention Steps 1-3) with the
    causal reading of this module; N_q = N_k gives ``attention_forward``.
    """
    K = np.asarray(K)
    return partial_forward(Q, K, V, scale, causal, 0, K.shape[2])


def merge_partials(O_parts, LSE_parts):
    """Combine partial results over disjoint key blocks.

    O_parts [P, ..., d_v] and LSE_parts [P, ...] -> (O [..., d_v], LSE [...]).
    Interview Q&A softmax answer, applied to whole partials: with
    M = max_p LSE_p, LSE = M + ln sum_p exp(LSE_p - M) and
    O = sum_p exp(LSE_p - LSE) O_p.  Parts with LSE_p = -inf contribute
    nothing; if every part is -inf the result is (0, -inf).
    """
    O_parts = np.asarray(O_parts, dtype=np.float64)
    LSE_parts = np.asarray(LSE_parts, dtype=np.float64)
    M = LSE_parts.max(axis=0)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(LSE_parts), np.exp(LSE_parts - Ms[None]), 0.0)
    tot = w.sum(axis=0)
    LSE = np.where(finite, Ms + np.log(np.where(finite, tot, 1.0)), -np.inf)
    scale = np.where(finite, 1.0 / np.where(finite, tot, 1.0), 0.0)
    O = (w[..., None] * O_parts).sum(axis=0) * scale[..., None]
    return O, LSE
