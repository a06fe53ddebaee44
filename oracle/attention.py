"""Plain fp64 definition of exact attention, forward and backward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the HIP library never
imports this module, and this module imports nothing from the HIP library.

Sources (cited by page title and section; the pages are web articles about
FlashAttention):

* "Flash attention: fast and memory-efficient exact attention with
  IO-awareness -- a deep dive" (technicalterrence.com), the walk-through of
  standard attention, Steps 1-3: the score matrix is the product of the
  queries with the transposed keys (N x N), a softmax normalises each row,
  and the normalised matrix multiplies V.  The same page, "What is the
  mathematical aspect of softmax? / Intuition", keeps for every row its
  maximum together with the sum of its exponentials; the result of the
  blocked method is stated to be exact, not approximate.
* "Optimizing memory usage on GPUs with flash attention mechanisms"
  (logicnest.cc), "Mechanics of Flash Attention": the dot-product scores are
  multiplied by a scale factor before the softmax (scaled dot product).
* FlashAttention interview Q&A (app.wittybyte.ai, problem "FlashAttention1"),
  the answer on how softmax is handled: the log-sum-exp form subtracts the
  row maximum before exponentiating, for numerical stability.
* "The Future of AI: How FlashAttention Revolutionizes Deep Learning"
  (networkstorageforum.com), "FlashAttention-2: Enhanced Performance",
  bullet on multi-query / grouped-query attention: several query heads share
  one key/value head.  Same page, "Understanding FlashAttention", bullet on
  recomputation: the backward pass recomputes the attention matrix instead
  of storing it.  The pages print no backward formulas; the backward here is
  the analytic derivative of the forward definition.
* ai5.artificialintelligencearticle.com (4-token example [A, B, C, D]):
  scores form a 4 x 4 matrix, a softmax turns them into weights, and the
  weights form a weighted sum of the values.

Readings taken where the pages are silent (each is listed with its reason in
the project's design notes):

* causal mask: the pages never define one; key j is hidden from query i when
  j > i (queries and keys have the same length N, diagonal kept).
* LSE: natural logarithm of the sum of exponentials of the scaled, masked
  scores of a row: LSE_i = m_i + ln(l_i).
* head grouping: query head h reads key/value head h // (H_q / H_kv)
  (contiguous groups); dK and dV of a key/value head sum over its group.

Everything is float64.  Inputs are upcast exactly (bf16 and fp32 values are
all representable in float64).  No blocking, tiling or online recurrence is
used here: that lives in the kernels, and in one test that checks the pages'
recurrence against this definition.
"""

import numpy as np

__all__ = [
    "kv_head_of",
    "head_forward",
    "head_backward",
    "attention_forward",
    "attention_backward",
    "attention_forward_rows",
]


def kv_head_of(h_q, n_heads_q, n_heads_kv):
    """Key/value head read by query head ``h_q``.

    Grouped-query attention ("The Future of AI: How FlashAttention
    Revolutionizes Deep Learning", "FlashAttention-2: Enhanced Performance",
    multi-query bullet): H_q / H_kv query heads share one key/value head.
    Reading: contiguous groups, so h_kv = h_q // (H_q / H_kv).
    """
    if n_heads_q % n_heads_kv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    return h_q // (n_heads_q // n_heads_kv)


def _scores(q, k, scale, causal):
    """Scaled, masked score matrix S (rows: queries, columns: keys).

    Deep-dive page, Step 2: S = Q K^T, one row per query token.  The
    logicnest page ("Mechanics of Flash Attention") multiplies the scores
    by a scale.  Causal reading: S[i, j] = -inf for j > i.
    """
    s = scale * (q @ k.T)
    if causal:
        i = np.arange(q.shape[0])[:, None]
        j = np.arange(k.shape[0])[None, :]
        s = np.where(j > i, -np.inf, s)
    return s


def _row_softmax(s):
    """Stable row softmax and per-row statistics.

    Interview Q&A, softmax answer (log-sum-exp, stability): subtract the row
    maximum m before exponentiating.  Returns P = exp(S - m) / l, the row
    maximum m and the row sum l = sum_j exp(S_ij - m_i).
    """
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def head_forward(q, k, v, scale, causal):
    """One (batch, query-head) unit: returns (O [N, d], LSE [N]).

    Deep-dive page, standard attention Steps 1-3: O = softmax(S) V with S the
    scaled, masked scores; LSE_i = m_i + ln l_i keeps the row statistics of
    the "Intuition" paragraph in one number per row.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    if n == 0:
        return np.zeros((0, v.shape[1])), np.zeros((0,))
    p, m, l = _row_softmax(_scores(q, k, scale, causal))
    return p @ v, m + np.log(l)


def head_backward(q, k, v, do, scale, causal):
    """Analytic backward of one unit: returns (dQ, dK, dV).

    The pages give no backward formulas, only that the backward recomputes
    the attention matrix ("The Future of AI ...", "Understanding
    FlashAttention", recomputation bullet).  This is the textbook chain rule
    through O = P V, P = rowsoftmax(S), S = scale Q K^T:
        dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
        dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
    P is recomputed here from Q and K; no forward output is taken as input.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    if q.shape[0] == 0:
        return np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    p, _, _ = _row_softmax(_scores(q, k, scale, causal))
    dv = p.T @ do
    dp = do @ v.T
    d_row = (p * dp).sum(axis=1)
    ds = p * (dp - d_row[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def _check_shapes(Q, K, V):
    if Q.ndim != 4 or K.ndim != 4 or V.ndim != 4:
        raise ValueError("expected [B, H, N, d] arrays")
    B, Hq, N, d = Q.shape
    if K.shape[0] != B or K.shape[2] != N or K.shape[3] != d or V.shape[:3] != K.shape[:3]:
        raise ValueError("K must be [B, H_kv, N, d] and V [B, H_kv, N, d_v], matching Q")
    if Hq % K.shape[1] != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    return B, Hq, K.shape[1], N, d


def attention_forward(Q, K, V, scale, causal):
    """Full forward: Q [B, H_q, N, d], K/V [B, H_kv, N, d] -> (O, LSE).

    O is [B, H_q, N, d_v] (d_v = V's last axis, normally d), LSE is
    [B, H_q, N]; both float64.  One unit per
    (b, h_q), reading key/value head ``kv_head_of(h_q, H_q, H_kv)``.
    """
    B, Hq, Hkv, N, d = _check_shapes(Q, K, V)
    O = np.zeros((B, Hq, N, V.shape[3]))
    LSE = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            O[b, h], LSE[b, h] = head_forward(Q[b, h], K[b, g], V[b, g], scale, causal)
    return O, LSE


def attention_backward(Q, K, V, dO, scale, causal):
    """Full backward -> (dQ [B, H_q, N, d], dK, dV [B, H_kv, N, d]).

    dK and dV of a key/value head are the sums over the query heads of its
    group (the derivative of a shared input is the sum of the derivatives of
    its uses).
    """
    B, Hq, Hkv, N, d = _check_shapes(Q, K, V)
    dQ = np.zeros((B, Hq, N, d))
    dK = np.zeros((B, Hkv, N, d))
    dV = np.zeros(V.shape)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            dq, dk, dv = head_backward(Q[b, h], K[b, g], V[b, g], dO[b, h], scale, causal)
            dQ[b, h] = dq
            dK[b, g] += dk
            dV[b, g] += dv
    return dQ, dK, dV


def attention_forward_rows(Q, K, V, scale, causal, b, h, rows):
    """Selected rows of one unit's forward, for spot checks at full size.

    Each requested query row i is computed on its own from the definition:
    s_j = scale q_i . k_j (j > i hidden if causal), o_i = sum_j softmax(s)_j
    v_j, lse_i = max_j s_j + ln sum_j exp(s_j - max).  Costs N d per row.
    Returns (O_rows [len(rows), d], LSE_rows [len(rows)]).
    """
    B, Hq, Hkv, N, d = _check_shapes(Q, K, V)
    g = kv_head_of(h, Hq, Hkv)
    k = np.asarray(K[b, g], dtype=np.float64)
    v = np.asarray(V[b, g], dtype=np.float64)
    rows = [int(r) for r in rows]
    o = np.zeros((len(rows), v.shape[1]))
    lse = np.zeros((len(rows),))
    for t, i in enumerate(rows):
        q = np.asarray(Q[b, h, i], dtype=np.float64)
        s = scale * (k @ q)
        if causal:
            s = s[: i + 1]
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        o[t] = (e / l) @ v[: s.shape[0]]
        lse[t] = m + np.log(l)
    return o, lse
