"""Attention over a batch of sequences of different lengths, packed, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the HIP library never
imports this module, and this module imports nothing from the HIP library.

Sources (cited by page title and section):

* FlashAttention interview Q&A (app.wittybyte.ai, "FlashAttention1"): the
  answer on scaling challenges names uneven work across the GPU's cores for
  variable sequence lengths, to be met by dynamic load balancing or sequence
  bucketing; the integration answer asks for inputs formatted for block-wise
  processing.  The pages give no layout.
* Each sequence is attended to on its own with the definition of
  ``oracle.attention`` (deep-dive page, standard attention Steps 1-3):
  no query sees a key of another sequence.

Reading taken where the pages are silent (listed in the design notes): the
sequences of a batch are packed back to back per head, Q [H_q, total, d],
K and V [H_kv, total, d], with cumulative offsets cu_seqlens [B + 1]
(cu[0] = 0, cu[B] = total); sequence b occupies rows cu[b] .. cu[b+1]-1 of
every head.  The causal mask applies within each sequence.

Everything is float64 and unblocked.
"""

import numpy as np

from .attention import head_backward, head_forward, kv_head_of

__all__ = ["varlen_forward", "varlen_backward"]


def _check(Q, K, V, cu):
    if Q.ndim != 3 or K.ndim != 3 or V.ndim != 3:
        raise ValueError("expected packed [H, total, d] arrays")
    Hq, total, d = Q.shape
    if K.shape[1] != total or K.shape[2] != d or V.shape[:2] != K.shape[:2] or Hq % K.shape[0] != 0:
        raise ValueError("K, V must be [H_kv, total, d] with H_q a multiple of H_kv")
    cu = [int(x) for x in cu]
    if cu[0] != 0 or cu[-1] != total or any(b < a for a, b in zip(cu[:-1], cu[1:])):
        raise ValueError("cu_seqlens must start at 0, end at total and not decrease")
    return Hq, K.shape[0], cu


def varlen_forward(Q, K, V, cu_seqlens, scale, causal):
    """Packed forward -> (O [H_q, total, d_v], LSE [H_q, total]): each
    sequence is plain attention over its own keys."""
    Q, K, V = (np.asarray(x, dtype=np.float64) for x in (Q, K, V))
    Hq, Hkv, cu = _check(Q, K, V, cu_seqlens)
    O = np.zeros((Hq, Q.shape[1], V.shape[2]))
    LSE = np.zeros((Hq, Q.shape[1]))
    for a, b in zip(cu[:-1], cu[1:]):
        if b == a:
            continue
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            O[h, a:b], LSE[h, a:b] = head_forward(Q[h, a:b], K[g, a:b], V[g, a:b], scale, causal)
    return O, LSE


def varlen_backward(Q, K, V, dO, cu_seqlens, scale, causal):
    """Packed backward -> (dQ, dK, dV), sequence by sequence; dK and dV of a
    kv head sum over the query heads of its group."""
    Q, K, V, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, dO))
    Hq, Hkv, cu = _check(Q, K, V, cu_seqlens)
    dQ, dK, dV = np.zeros(Q.shape), np.zeros(K.shape), np.zeros(V.shape)
    for a, b in zip(cu[:-1], cu[1:]):
        if b == a:
            continue
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            dq, dk, dv = head_backward(Q[h, a:b], K[g, a:b], V[g, a:b], dO[h, a:b], scale, causal)
            dQ[h, a:b] = dq
            dK[g, a:b] += dk
            dV[g, a:b] += dv
    return dQ, dK, dV
