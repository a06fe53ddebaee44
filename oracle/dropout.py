"""Attention with dropout on the attention probabilities, forward and
backward, fp64, with the keep mask drawn from a counter-based generator.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the HIP library never
imports this module, and this module imports nothing from the HIP library.

Sources:

* "Flash attention: fast and memory-efficient exact attention with
  IO-awareness -- a deep dive", section "Computing and memory basics",
  quantitative evidence: in unfused attention, softmax, dropout and masking
  take most of the time -- dropout is applied to the attention weights
  between the softmax and the product with V.  The pages give no formula or
  generator.
* The generator is Philox-4x32 with 10 rounds from J. K. Salmon,
  M. A. Moraes, R. O. Dror and D. E. Shaw, "Parallel random numbers: as easy
  as 1, 2, 3" (SC 2011): a 128-bit counter and a 64-bit key; each round
  multiplies counter words 0 and 2 by 0xD2511F53 and 0xCD9E8D57 (full 64-bit
  products), and forms (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key is
  bumped by the Weyl constants (0x9E3779B9, 0xBB67AE85) between rounds.

Readings taken where the pages are silent (listed in the design notes):

* Inverted dropout on P: O = (P o Z) V / (1 - p), Z in {0, 1}; LSE is that
  of the softmax without dropout; the backward is the chain rule with the
  same Z: dV = (P o Z)^T dO / (1 - p), dP = (dO V^T) o Z / (1 - p),
  D_i = sum_j P_ij dP_ij (= dO_i . O_i), dS = P o (dP - D), dQ = scale dS K,
  dK = scale dS^T Q.
* Keep decision: 8-bit random values.  t8 = round(p * 256) (round half to
  even), the effective drop probability is t8 / 256 and element (i, j) is
  kept when its byte u >= t8, so 1 / (1 - p) is read as 256 / (256 - t8).
* Bytes of element (b, h_q, i, j): Philox with key (seed & 0xFFFFFFFF,
  seed >> 32) and counter (j // 4, i // 4, b * H_q + h_q, offset) gives four
  32-bit words for the 4 x 4 block of queries 4(i // 4) .. +3 and keys
  4(j // 4) .. +3; word i % 4 holds the block's row i, and its byte j % 4
  (bits 8 (j % 4) .. +7) is element (i, j)'s u.

Everything is float64 and unblocked.
"""

import numpy as np

from .attention import _check_shapes, _row_softmax, _scores, kv_head_of

__all__ = ["philox4x32_10", "dropout_threshold", "keep_mask", "dropout_head_forward", "dropout_head_backward",
           "dropout_forward", "dropout_backward"]

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox-4x32-10 of counters (c0, c1, c2, c3) (uint32 arrays, broadcast)
    under the key (k0, k1) (Python ints); returns four uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK32 for x in (c0, c1, c2, c3)]
    c = list(np.broadcast_arrays(*c))
    k0, k1 = int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF
    for _ in range(10):
        p0 = _M0 * c[0]  # < 2^64: exact in uint64
        p1 = _M1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
        k0 = (k0 + _W0) & 0xFFFFFFFF
        k1 = (k1 + _W1) & 0xFFFFFFFF
    return [x.astype(np.uint32) for x in c]


def dropout_threshold(p):
    """t8 = round(p * 256), half to even; p must give t8 <= 255."""
    t8 = int(np.round(np.float64(p) * 256.0))
    if not 0 <= t8 <= 255:
        raise ValueError("dropout probability must round to 0 .. 255 / 256")
    return t8


def keep_mask(n_q, n_k, bh, p, seed, offset):
    """Boolean [n_q, n_k]: element (i, j) of unit bh = b * H_q + h_q kept."""
    t8 = dropout_threshold(p)
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    words = philox4x32_10(j // 4, i // 4, bh, offset, seed & 0xFFFFFFFF, seed >> 32)
    w = np.choose(i % 4, words) if n_q and n_k else np.zeros((n_q, n_k), dtype=np.uint32)
    u = (w >> (8 * (j % 4)).astype(np.uint32)) & np.uint32(0xFF)
    return u >= t8


def _unit(q, k, scale, causal, keep, t8):
    p, m, l = _row_softmax(_scores(q, k, scale, causal))
    pz = np.where(keep, p, 0.0) * (256.0 / (256.0 - t8))
    return p, pz, m + np.log(l)


def dropout_head_forward(q, k, v, scale, causal, p, seed, offset, bh):
    """One (batch, query head) unit with unit index bh = b * H_q + h:
    (O [N, d], LSE [N])."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    t8 = dropout_threshold(p)
    keep = keep_mask(q.shape[0], k.shape[0], bh, p, seed, offset)
    _, pz, lse = _unit(q, k, scale, causal, keep, t8)
    return pz @ v, lse


def dropout_head_backward(q, k, v, do, scale, causal, p, seed, offset, bh):
    """Backward of one unit: (dQ, dK, dV) of its query head (dK, dV before
    the sum over a grouped head's query heads)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    t8 = dropout_threshold(p)
    keep = keep_mask(q.shape[0], k.shape[0], bh, p, seed, offset)
    pr, pz, _ = _unit(q, k, scale, causal, keep, t8)
    dp = np.where(keep, do @ v.T, 0.0) * (256.0 / (256.0 - t8))
    d_row = (pr * dp).sum(axis=1)
    ds = pr * (dp - d_row[:, None])
    return scale * (ds @ k), scale * (ds.T @ q), pz.T @ do


def dropout_forward(Q, K, V, scale, causal, p, seed, offset=0):
    """Q [B, H_q, N, d], K/V [B, H_kv, N, d] -> (O, LSE); LSE without dropout."""
    Q, K, V = (np.asarray(x, dtype=np.float64) for x in (Q, K, V))
    B, Hq, Hkv, N, d = _check_shapes(Q, K, V)
    dropout_threshold(p)
    O = np.zeros((B, Hq, N, V.shape[3]))
    LSE = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            O[b, h], LSE[b, h] = dropout_head_forward(Q[b, h], K[b, g], V[b, g], scale, causal, p, seed, offset,
                                                      b * Hq + h)
    return O, LSE


def dropout_backward(Q, K, V, dO, scale, causal, p, seed, offset=0):
    """Analytic backward of ``dropout_forward`` with the same keep mask."""
    Q, K, V, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, dO))
    B, Hq, Hkv, N, d = _check_shapes(Q, K, V)
    dropout_threshold(p)
    dQ, dK, dV = np.zeros(Q.shape), np.zeros(K.shape), np.zeros(V.shape)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            dq, dk, dv = dropout_head_backward(Q[b, h], K[b, g], V[b, g], dO[b, h], scale, causal, p, seed, offset,
                                               b * Hq + h)
            dQ[b, h] = dq
            dK[b, g] += dk
            dV[b, g] += dv
    return dQ, dK, dV
