"""Pins that tie the fp64 oracle to facts fixed by the pages and by mathematics.

Each ``check_*`` function raises AssertionError when the oracle disagrees
with the fact it pins.  ``test_oracle_pins.py`` runs them against the oracle
as written; ``test_oracle_mutants.py`` runs them against deliberately broken
copies of the oracle's internals (a dropped scale, a wrong mask, a missing
term, a transposed operand ...) and requires each break to be caught.

The checks look the oracle up through the ``oracle.attention`` and
``oracle.splitkv`` modules at call time, so a patched module attribute is
what they exercise.
"""

import math
import os

import numpy as np

import oracle.attention as OA
import oracle.blocksparse as OB
import oracle.dropout as ODR
import oracle.splitkv as OS
import oracle.varlen as OV
import oracle.window as OW

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_four_token_example():
    """Parse tests/golden/four_token_scores.txt -> dict name -> int matrix."""
    blocks, name = {}, None
    with open(os.path.join(GOLDEN, "four_token_scores.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line[0].isalpha():
                name = line
                blocks[name] = []
            else:
                blocks[name].append([int(x) for x in line.split()])
    return {k: np.array(v, dtype=np.float64) for k, v in blocks.items()}


def online_recurrence(scores, values, block):
    """The pages' block recurrence, written independently of the oracle.

    Interview Q&A (app.wittybyte.ai, "FlashAttention1"), softmax answer: for
    block i, m_i = max(m_{i-1}, local_max_i) and
    l_i = l_{i-1} exp(m_{i-1} - m_i) + local_sum_i exp(local_max_i - m_i),
    with local_sum_i read as sum exp(s - local_max_i) over the block.  The
    deep-dive page ("Intuition") rescales the numerator (the running output)
    by the same factor as the denominator.  Start: m = -inf, l = 0, o = 0; a
    block whose entries are all -inf (masked) contributes nothing.
    Returns (O rows, LSE) for a score matrix ``scores`` [n, n_k] and values
    ``values`` [n_k, d].
    """
    n, nk = scores.shape
    d = values.shape[1]
    O = np.zeros((n, d))
    LSE = np.zeros(n)
    for i in range(n):
        m, l, o = -math.inf, 0.0, np.zeros(d)
        for j0 in range(0, nk, block):
            s = scores[i, j0 : j0 + block]
            local_max = s.max()
            if local_max == -math.inf:
                continue
            e = np.exp(s - local_max)
            local_sum = e.sum()
            local_o = e @ values[j0 : j0 + block]
            m_new = max(m, local_max)
            a_old = math.exp(m - m_new) if m != -math.inf else 0.0
            a_new = math.exp(local_max - m_new)
            l = l * a_old + local_sum * a_new
            o = o * a_old + local_o * a_new
            m = m_new
        O[i] = o / l
        LSE[i] = m + math.log(l)
    return O, LSE


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# softmax of a row that is a permutation of [1, 2, 3, 4]: e^(x-4) / sum,
# sum = 1 + e^-1 + e^-2 + e^-3 = 1.5530018...; values rounded to 7 digits.
SOFTMAX_1234 = {1.0: 0.0320586, 2.0: 0.0871443, 3.0: 0.2368828, 4.0: 0.6439143}
LSE_1234 = 4.4401897  # 4 + ln(1.5530018)
L_MERGED = 1.5530018  # tile (A,B) then tile (C,D): 1.3678794 e^-2 + 1.3678794
L_TILE = 1.3678794  # 1 + e^-1 for a 2-wide tile holding {x, x-1}


def check_four_token_tiles_consistent():
    ex = load_four_token_example()
    s = ex["scores"]
    assert np.array_equal(ex["tile1"], s[0:2, 0:2])
    assert np.array_equal(ex["tile2"], s[0:2, 2:4])
    assert np.array_equal(ex["tile3"], s[2:4, 0:2])
    assert np.array_equal(ex["tile4"], s[2:4, 2:4])


def check_four_token_recurrence_values():
    """Row A through the pages' recurrence with 2-wide tiles, by hand."""
    s = load_four_token_example()["scores"]
    row = s[0]
    # tile 1: local max 2, local sum 1 + e^-1; tile 2: local max 4, same sum
    t1 = np.exp(row[:2] - row[:2].max()).sum()
    t2 = np.exp(row[2:] - row[2:].max()).sum()
    assert abs(t1 - L_TILE) < 1e-7 and abs(t2 - L_TILE) < 1e-7
    m = max(row[:2].max(), row[2:].max())
    l = t1 * math.exp(row[:2].max() - m) + t2 * math.exp(row[2:].max() - m)
    assert m == 4.0 and abs(l - L_MERGED) < 1e-7
    assert abs(m + math.log(l) - LSE_1234) < 1e-7


def check_four_token_oracle():
    """Oracle on the printed scores: Q = scores, K = I, V = I, scale 1."""
    s = load_four_token_example()["scores"]
    eye = np.eye(4)
    Q, K, V = s[None, None], eye[None, None], eye[None, None]
    O, LSE = OA.attention_forward(Q, K, V, 1.0, False)
    for i in range(4):
        want = np.array([SOFTMAX_1234[x] for x in s[i]])
        assert np.max(np.abs(O[0, 0, i] - want)) < 1e-7, (i, O[0, 0, i], want)
        assert abs(LSE[0, 0, i] - LSE_1234) < 1e-7
    # the same with every score shifted by 1000: weights unchanged, LSE + 1000
    # (softmax is invariant to a per-row constant; the stable form must not
    # overflow)
    O2, LSE2 = OA.attention_forward((s + 1000.0)[None, None] * 1.0, K, V, 1.0, False)
    assert np.all(np.isfinite(O2)) and np.all(np.isfinite(LSE2))
    assert np.max(np.abs(O2 - O)) < 1e-12
    assert np.max(np.abs(LSE2 - (LSE + 1000.0))) < 1e-9
    # the pages' recurrence over the printed 2 x 2 tiling gives the same
    O3, LSE3 = online_recurrence(s, eye, 2)
    assert np.max(np.abs(O3 - O[0, 0])) < 1e-14
    assert np.max(np.abs(LSE3 - LSE[0, 0])) < 1e-14


def check_blocked_recurrence_matches(seed=7):
    rng = np.random.default_rng(seed)
    n, d, scale = 13, 5, 0.37
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    for causal in (False, True):
        O, LSE = OA.attention_forward(q[None, None], k[None, None], v[None, None], scale, causal)
        s = scale * (q @ k.T)
        if causal:
            s = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, s)
        for block in (1, 2, 3, 7, n):
            Ob, LSEb = online_recurrence(s, v, block)
            assert np.max(np.abs(Ob - O[0, 0])) < 1e-12, (causal, block)
            assert np.max(np.abs(LSEb - LSE[0, 0])) < 1e-12, (causal, block)


def check_rows_sum_to_one(seed=8):
    rng = np.random.default_rng(seed)
    n = 11
    q, k = _rand(rng, n, 6), _rand(rng, n, 6)
    eye = np.eye(n)
    for causal in (False, True):
        O, _ = OA.attention_forward(q[None, None], k[None, None], eye[None, None], 0.5, causal)
        P = O[0, 0]
        assert np.all(P >= 0)
        assert np.max(np.abs(P.sum(axis=1) - 1.0)) < 1e-14
        if causal:
            assert np.all(P[np.triu_indices(n, 1)] == 0.0)


def check_constant_v(seed=9):
    rng = np.random.default_rng(seed)
    n, d = 10, 4
    q, k, do = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    c = rng.standard_normal(d)
    v = np.tile(c, (n, 1))
    for causal in (False, True):
        O, _ = OA.attention_forward(q[None, None], k[None, None], v[None, None], 0.8, causal)
        assert np.max(np.abs(O[0, 0] - c)) < 1e-14
        dQ, dK, dV = OA.attention_backward(q[None, None], k[None, None], v[None, None], do[None, None], 0.8, causal)
        assert np.max(np.abs(dQ)) < 1e-13 and np.max(np.abs(dK)) < 1e-13


def check_equal_scores(seed=10):
    rng = np.random.default_rng(seed)
    n, d = 9, 3
    k, v = _rand(rng, n, d), _rand(rng, n, d)
    q = np.zeros((n, d))
    O, LSE = OA.attention_forward(q[None, None], k[None, None], v[None, None], 1.3, False)
    assert np.max(np.abs(O[0, 0] - v.mean(axis=0))) < 1e-14
    assert np.max(np.abs(LSE[0, 0] - math.log(n))) < 1e-14
    O, LSE = OA.attention_forward(q[None, None], k[None, None], v[None, None], 1.3, True)
    prefix_mean = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.max(np.abs(O[0, 0] - prefix_mean)) < 1e-14
    assert np.max(np.abs(LSE[0, 0] - np.log(np.arange(1, n + 1)))) < 1e-14
    # scale = 0 makes every score equal as well
    q2 = _rand(rng, n, d)
    O, LSE = OA.attention_forward(q2[None, None], k[None, None], v[None, None], 0.0, True)
    assert np.max(np.abs(O[0, 0] - prefix_mean)) < 1e-14


def check_single_token(seed=11):
    rng = np.random.default_rng(seed)
    d, scale = 5, 0.6
    q, k, v, do = (_rand(rng, 1, d) for _ in range(4))
    for causal in (False, True):
        O, LSE = OA.attention_forward(q[None, None], k[None, None], v[None, None], scale, causal)
        assert np.array_equal(O[0, 0], v)
        assert abs(LSE[0, 0, 0] - scale * float(q[0] @ k[0])) < 1e-15
        dQ, dK, dV = OA.attention_backward(q[None, None], k[None, None], v[None, None], do[None, None], scale, causal)
        assert np.max(np.abs(dQ)) < 1e-15 and np.max(np.abs(dK)) < 1e-15
        assert np.max(np.abs(dV[0, 0] - do)) < 1e-15


def check_causal_prefix(seed=12):
    rng = np.random.default_rng(seed)
    n, d, scale = 8, 4, 0.7
    q, k, v = _rand(rng, n, d), _rand(rng, n, d), _rand(rng, n, d)
    O, LSE = OA.attention_forward(q[None, None], k[None, None], v[None, None], scale, True)
    for i in range(n):
        Oi, LSEi = OA.attention_forward(
            q[None, None, : i + 1], k[None, None, : i + 1], v[None, None, : i + 1], scale, False
        )
        assert np.max(np.abs(O[0, 0, i] - Oi[0, 0, i])) < 1e-14
        assert abs(LSE[0, 0, i] - LSEi[0, 0, i]) < 1e-14
    assert np.array_equal(O[0, 0, 0], v[0])


def _loss(Q, K, V, dO, scale, causal):
    O, _ = OA.attention_forward(Q, K, V, scale, causal)
    return float((O * dO).sum())


def check_backward_finite_differences(seed=13):
    """Central differences of L = <dO, O> against the analytic backward."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, n, d, scale = 1, 2, 1, 6, 3, 0.45
    Q = rng.standard_normal((B, Hq, n, d))
    K = rng.standard_normal((B, Hkv, n, d))
    V = rng.standard_normal((B, Hkv, n, d))
    dO = rng.standard_normal((B, Hq, n, d))
    h = 1e-6
    for causal in (False, True):
        grads = OA.attention_backward(Q, K, V, dO, scale, causal)
        for which, X in enumerate((Q, K, V)):
            G = grads[which]
            num = np.zeros_like(X)
            it = np.nditer(X, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                old = X[idx]
                X[idx] = old + h
                lp = _loss(Q, K, V, dO, scale, causal)
                X[idx] = old - h
                lm = _loss(Q, K, V, dO, scale, causal)
                X[idx] = old
                num[idx] = (lp - lm) / (2 * h)
            err = np.max(np.abs(num - G)) / max(1.0, np.max(np.abs(G)))
            assert err < 1e-7, (causal, which, err)


def check_against_torch_sdpa(seed=14):
    """Library cross-check: torch's CPU float64 scaled_dot_product_attention
    (and its autograd) on the same inputs, including grouped heads."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(seed)
    B, Hq, Hkv, n, d, scale = 2, 4, 2, 7, 5, 0.31
    Q = rng.standard_normal((B, Hq, n, d))
    K = rng.standard_normal((B, Hkv, n, d))
    V = rng.standard_normal((B, Hkv, n, d))
    dO = rng.standard_normal((B, Hq, n, d))
    for causal in (False, True):
        O, LSE = OA.attention_forward(Q, K, V, scale, causal)
        dQ, dK, dV = OA.attention_backward(Q, K, V, dO, scale, causal)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
        to = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=True)
        to.backward(torch.tensor(dO))
        assert np.max(np.abs(O - to.detach().numpy())) < 1e-12
        assert np.max(np.abs(dQ - tq.grad.numpy())) < 1e-12
        assert np.max(np.abs(dK - tk.grad.numpy())) < 1e-12
        assert np.max(np.abs(dV - tv.grad.numpy())) < 1e-12
        # LSE: torch.logsumexp over the scaled, masked scores of each head
        kk = torch.tensor(K).repeat_interleave(Hq // Hkv, dim=1)
        s = torch.tensor(Q) @ kk.transpose(-1, -2) * scale
        if causal:
            s = s.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
        assert np.max(np.abs(LSE - torch.logsumexp(s, dim=-1).numpy())) < 1e-12


def check_grouped_heads(seed=15):
    """GQA equals MHA over K/V repeated per group; dK/dV are group sums."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, n, d, scale = 1, 6, 2, 5, 3, 0.5
    G = Hq // Hkv
    Q = rng.standard_normal((B, Hq, n, d))
    K = rng.standard_normal((B, Hkv, n, d))
    V = rng.standard_normal((B, Hkv, n, d))
    dO = rng.standard_normal((B, Hq, n, d))
    Kr, Vr = np.repeat(K, G, axis=1), np.repeat(V, G, axis=1)
    for causal in (False, True):
        O, LSE = OA.attention_forward(Q, K, V, scale, causal)
        Or, LSEr = OA.attention_forward(Q, Kr, Vr, scale, causal)
        assert np.max(np.abs(O - Or)) < 1e-14 and np.max(np.abs(LSE - LSEr)) < 1e-14
        dQ, dK, dV = OA.attention_backward(Q, K, V, dO, scale, causal)
        dQr, dKr, dVr = OA.attention_backward(Q, Kr, Vr, dO, scale, causal)
        assert np.max(np.abs(dQ - dQr)) < 1e-14
        assert np.max(np.abs(dK - dKr.reshape(B, Hkv, G, n, d).sum(axis=2))) < 1e-13
        assert np.max(np.abs(dV - dVr.reshape(B, Hkv, G, n, d).sum(axis=2))) < 1e-13
    assert [OA.kv_head_of(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]


def check_forward_rows(seed=16):
    """Row-sampled forward equals the full forward and the closed forms."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, n, d, scale = 2, 4, 2, 9, 4, 0.4
    Q = rng.standard_normal((B, Hq, n, d))
    K = rng.standard_normal((B, Hkv, n, d))
    V = rng.standard_normal((B, Hkv, n, d))
    for causal in (False, True):
        O, LSE = OA.attention_forward(Q, K, V, scale, causal)
        rows = [0, 3, n - 1]
        Or, LSEr = OA.attention_forward_rows(Q, K, V, scale, causal, 1, 3, rows)
        assert np.max(np.abs(Or - O[1, 3, rows])) < 1e-14
        assert np.max(np.abs(LSEr - LSE[1, 3, rows])) < 1e-14
    Z = np.zeros_like(Q)
    Or, LSEr = OA.attention_forward_rows(Z, K, V, scale, True, 0, 2, [0, 4, 8])
    g = OA.kv_head_of(2, Hq, Hkv)
    for t, i in enumerate([0, 4, 8]):
        assert np.max(np.abs(Or[t] - V[0, g, : i + 1].mean(axis=0))) < 1e-14
        assert abs(LSEr[t] - math.log(i + 1)) < 1e-14


# ---------------------------------------------------------------- split keys


def _qkv(rng, B, Hq, Hkv, n_q, n_k, d):
    return (rng.standard_normal((B, Hq, n_q, d)), rng.standard_normal((B, Hkv, n_k, d)),
            rng.standard_normal((B, Hkv, n_k, d)))


def check_cross_square(seed=17):
    """N_q = N_k reproduces the square definition of oracle.attention."""
    rng = np.random.default_rng(seed)
    Q, K, V = _qkv(rng, 2, 4, 2, 11, 11, 8)
    for causal in (False, True):
        O, LSE = OS.cross_forward(Q, K, V, 0.3, causal)
        Or, LSEr = OA.attention_forward(Q, K, V, 0.3, causal)
        assert np.max(np.abs(O - Or)) < 1e-14 and np.max(np.abs(LSE - LSEr)) < 1e-13


def check_cross_suffix(seed=18):
    """Bottom-right causal alignment: N_q queries against N_k keys are the last
    N_q rows of the square problem whose queries extend them to N_k rows."""
    rng = np.random.default_rng(seed)
    n_k, d = 13, 6
    Qf, K, V = _qkv(rng, 1, 2, 1, n_k, n_k, d)
    Of, LSEf = OA.attention_forward(Qf, K, V, 0.45, True)
    for n_q in (1, 2, 5, n_k):
        O, LSE = OS.cross_forward(Qf[:, :, n_k - n_q:], K, V, 0.45, True)
        assert np.max(np.abs(O - Of[:, :, n_k - n_q:])) < 1e-14
        assert np.max(np.abs(LSE - LSEf[:, :, n_k - n_q:])) < 1e-13
    # one query (decoding) sees every key: causal equals non-causal
    O1, L1 = OS.cross_forward(Qf[:, :, :1], K, V, 0.45, True)
    O0, L0 = OS.cross_forward(Qf[:, :, :1], K, V, 0.45, False)
    assert np.max(np.abs(O1 - O0)) < 1e-15 and np.max(np.abs(L1 - L0)) < 1e-15
    # more queries than keys: the first N_q - N_k rows see nothing
    Q2, K2, V2 = _qkv(rng, 1, 1, 1, 7, 4, 3)
    O2, L2 = OS.cross_forward(Q2, K2, V2, 1.0, True)
    assert np.all(O2[0, 0, :3] == 0) and np.all(L2[0, 0, :3] == -np.inf)
    O2s, L2s = OA.attention_forward(Q2[:, :, 3:], K2, V2, 1.0, True)
    assert np.max(np.abs(O2[:, :, 3:] - O2s)) < 1e-14 and np.max(np.abs(L2[:, :, 3:] - L2s)) < 1e-13


def check_merge_four_token():
    """The printed example merged from its two key tiles: row A's tile (A, B)
    holds scores {1, 2}, tile (C, D) holds {3, 4}; merged LSE = 4 + ln
    1.5530018 and the merged weights are the softmax of [1, 2, 3, 4]."""
    s = load_four_token_example()["scores"]
    eye = np.eye(4)
    Q, K, V = s[None, None], eye[None, None], eye[None, None]
    parts = [OS.partial_forward(Q, K, V, 1.0, False, 0, 2), OS.partial_forward(Q, K, V, 1.0, False, 2, 4)]
    assert abs(parts[0][1][0, 0, 0] - (2 + math.log(L_TILE))) < 1e-7
    assert abs(parts[1][1][0, 0, 0] - (4 + math.log(L_TILE))) < 1e-7
    O, LSE = OS.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    for i in range(4):
        want = np.array([SOFTMAX_1234[x] for x in s[i]])
        assert np.max(np.abs(O[0, 0, i] - want)) < 1e-7
        assert abs(LSE[0, 0, i] - LSE_1234) < 1e-7


def check_merge_partition(seed=19):
    """Merging the partial results of any partition of the keys (empty blocks
    included) gives attention over all keys, causal or not, N_q <> N_k."""
    rng = np.random.default_rng(seed)
    for n_q, n_k in ((1, 37), (5, 37), (37, 37), (9, 4)):
        Q, K, V = _qkv(rng, 2, 4, 2, n_q, n_k, 5)
        for causal in (False, True):
            want_o, want_l = OS.cross_forward(Q, K, V, 0.7, causal)
            for cuts in ([0, n_k], [0, 0, n_k], [0, 1, n_k // 2, n_k], list(range(0, n_k + 1, 3)) + [n_k]):
                cuts = sorted(set(min(c, n_k) for c in cuts))
                parts = [OS.partial_forward(Q, K, V, 0.7, causal, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
                parts.append(OS.partial_forward(Q, K, V, 0.7, causal, n_k, n_k))  # an empty block
                O, LSE = OS.merge_partials([p[0] for p in parts], [p[1] for p in parts])
                live = np.isfinite(want_l)
                assert np.array_equal(np.isfinite(LSE), live)
                assert np.max(np.abs(O - want_o)) < 1e-13
                assert np.max(np.abs(LSE[live] - want_l[live])) < 1e-12


def check_merge_properties(seed=20):
    """One part is returned unchanged; order does not matter; all-empty rows
    stay (0, -inf); values far from 1 do not overflow."""
    rng = np.random.default_rng(seed)
    Op = rng.standard_normal((3, 4, 6))
    Lp = rng.standard_normal((3, 4)) * 50.0
    O1, L1 = OS.merge_partials(Op[:1], Lp[:1])
    assert np.max(np.abs(O1 - Op[0])) < 1e-15 and np.max(np.abs(L1 - Lp[0])) < 1e-15
    Oa, La = OS.merge_partials(Op, Lp)
    Ob, Lb = OS.merge_partials(Op[::-1], Lp[::-1])
    assert np.max(np.abs(Oa - Ob)) < 1e-14 and np.max(np.abs(La - Lb)) < 1e-12
    # closed form for two parts with LSE a, b: weights e^a / (e^a + e^b)
    a, b = 700.0, 699.0
    O2, L2 = OS.merge_partials(np.array([[[1.0]], [[0.0]]]), np.array([[a], [b]]))
    assert abs(L2[0] - (a + math.log1p(math.exp(b - a)))) < 1e-12
    assert abs(O2[0, 0] - 1.0 / (1.0 + math.exp(b - a))) < 1e-15
    Oe, Le = OS.merge_partials(np.zeros((2, 1, 3)), np.full((2, 1), -np.inf))
    assert np.all(Oe == 0) and np.all(Le == -np.inf)


# ---------------------------------------------------------------- windows


def check_window_special_cases(seed=21):
    """(-1, 0) is the causal mask and (-1, -1) no mask, forward and backward;
    (0, 0) lets every row see only its own key: O = V, LSE = its own score,
    dV = dO and dQ = dK = 0."""
    rng = np.random.default_rng(seed)
    Q, K, V = _qkv(rng, 2, 4, 2, 10, 10, 6)
    dO = rng.standard_normal(Q.shape)
    for (lw, rw), causal in (((-1, 0), True), ((-1, -1), False)):
        O, L = OW.window_forward(Q, K, V, 0.4, lw, rw)
        Or, Lr = OA.attention_forward(Q, K, V, 0.4, causal)
        assert np.max(np.abs(O - Or)) < 1e-14 and np.max(np.abs(L - Lr)) < 1e-13
        g = OW.window_backward(Q, K, V, dO, 0.4, lw, rw)
        gr = OA.attention_backward(Q, K, V, dO, 0.4, causal)
        for a, b in zip(g, gr):
            assert np.max(np.abs(a - b)) < 1e-12
    O, L = OW.window_forward(Q, K, V, 0.4, 0, 0)
    G = Q.shape[1] // K.shape[1]
    Vr = np.repeat(V, G, axis=1)
    Kr = np.repeat(K, G, axis=1)
    assert np.max(np.abs(O - Vr)) < 1e-15
    assert np.max(np.abs(L - 0.4 * (Q * Kr).sum(axis=3))) < 1e-13
    dQ, dK, dV = OW.window_backward(Q, K, V, dO, 0.4, 0, 0)
    assert np.max(np.abs(dQ)) < 1e-15 and np.max(np.abs(dK)) < 1e-15
    assert np.max(np.abs(dV - dO.reshape(2, 2, G, 10, 6).sum(axis=2))) < 1e-14


def check_window_rows_are_slices(seed=22):
    """Row i of a (left, right) window is plain attention of query i over the
    keys i-left .. i+right (clipped), computed with the square definition on
    that slice."""
    rng = np.random.default_rng(seed)
    n = 17
    Q, K, V = _qkv(rng, 1, 1, 1, n, n, 5)
    for lw, rw in ((3, 0), (0, 2), (4, 5), (-1, 3), (6, -1)):
        O, L = OW.window_forward(Q, K, V, 0.6, lw, rw)
        for i in range(n):
            a = 0 if lw < 0 else max(0, i - lw)
            b = n if rw < 0 else min(n, i + rw + 1)
            o, l = OA.head_forward(Q[0, 0, i:i + 1], K[0, 0, a:b], V[0, 0, a:b], 0.6, False)
            assert np.max(np.abs(O[0, 0, i] - o[0])) < 1e-14 and abs(L[0, 0, i] - l[0]) < 1e-13


def check_window_finite_differences(seed=23):
    """Central differences of <dO, O> for a two-sided window."""
    rng = np.random.default_rng(seed)
    Q, K, V = _qkv(rng, 1, 2, 1, 7, 7, 3)
    dO = rng.standard_normal(Q.shape)
    lw, rw, sc = 2, 1, 0.8
    dQ, dK, dV = OW.window_backward(Q, K, V, dO, sc, lw, rw)
    h = 1e-6

    def loss(q, k, v):
        return float((OW.window_forward(q, k, v, sc, lw, rw)[0] * dO).sum())

    for X, G in ((Q, dQ), (K, dK), (V, dV)):
        idx = [tuple(rng.integers(0, s) for s in X.shape) for _ in range(6)]
        for ix in idx:
            Xp, Xm = X.copy(), X.copy()
            Xp[ix] += h
            Xm[ix] -= h
            args_p = [Xp if Y is X else Y for Y in (Q, K, V)]
            args_m = [Xm if Y is X else Y for Y in (Q, K, V)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - G[ix]) < 1e-7 * max(1.0, abs(fd)), (ix, fd, G[ix])


# ---------------------------------------------------------------- packed variable lengths


def _pack(rng, lens, Hq, Hkv, d):
    total = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    Q = rng.standard_normal((Hq, total, d))
    K = rng.standard_normal((Hkv, total, d))
    V = rng.standard_normal((Hkv, total, d))
    return Q, K, V, cu


def check_varlen_equal_lengths(seed=24):
    """B sequences of one length n, packed [H, B*n, d], give the fixed-length
    batch [B, H, n, d] result, forward and backward, with grouped heads."""
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, n, d = 3, 4, 2, 6, 5
    Q, K, V, cu = _pack(rng, [n] * B, Hq, Hkv, d)
    dO = rng.standard_normal(Q.shape)

    def unpack(X):  # [H, B*n, d] -> [B, H, n, d]
        return X.reshape(X.shape[0], B, n, -1).transpose(1, 0, 2, 3)

    for causal in (False, True):
        O, L = OV.varlen_forward(Q, K, V, cu, 0.45, causal)
        Or, Lr = OA.attention_forward(unpack(Q), unpack(K), unpack(V), 0.45, causal)
        assert np.max(np.abs(unpack(O) - Or)) < 1e-14
        assert np.max(np.abs(L.reshape(Hq, B, n).transpose(1, 0, 2) - Lr)) < 1e-13
        g = OV.varlen_backward(Q, K, V, dO, cu, 0.45, causal)
        gr = OA.attention_backward(unpack(Q), unpack(K), unpack(V), unpack(dO), 0.45, causal)
        for a, b in zip(g, gr):
            assert np.max(np.abs(unpack(a) - b)) < 1e-12


def check_varlen_ragged_slices(seed=25):
    """Ragged lengths (with empty and one-token sequences): every sequence is
    the square definition on its own rows, so no query sees a key of another
    sequence; a one-token sequence has O = its V row and LSE = its own score."""
    rng = np.random.default_rng(seed)
    lens = [5, 0, 1, 9, 3, 1]
    Hq, Hkv, d, sc = 4, 2, 4, 0.7
    Q, K, V, cu = _pack(rng, lens, Hq, Hkv, d)
    G = Hq // Hkv
    for causal in (False, True):
        O, L = OV.varlen_forward(Q, K, V, cu, sc, causal)
        for s, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
            for h in range(Hq):
                o, l = OA.head_forward(Q[h, a:b], K[h // G, a:b], V[h // G, a:b], sc, causal)
                assert np.max(np.abs(O[h, a:b] - o), initial=0.0) < 1e-14
                assert np.max(np.abs(L[h, a:b] - l), initial=0.0) < 1e-13
                if b - a == 1:
                    assert np.max(np.abs(O[h, a] - V[h // G, a])) < 1e-15
                    assert abs(L[h, a] - sc * float(Q[h, a] @ K[h // G, a])) < 1e-13


def check_varlen_finite_differences(seed=26):
    """Central differences of <dO, O> over a ragged, grouped-head pack."""
    rng = np.random.default_rng(seed)
    Q, K, V, cu = _pack(rng, [3, 1, 4], 4, 2, 3)
    dO = rng.standard_normal(Q.shape)
    sc = 0.9
    h = 1e-6
    for causal in (False, True):
        dQ, dK, dV = OV.varlen_backward(Q, K, V, dO, cu, sc, causal)

        def loss(q, k, v):
            return float((OV.varlen_forward(q, k, v, cu, sc, causal)[0] * dO).sum())

        for X, Gr in ((Q, dQ), (K, dK), (V, dV)):
            for _ in range(6):
                ix = tuple(int(rng.integers(0, s)) for s in X.shape)
                Xp, Xm = X.copy(), X.copy()
                Xp[ix] += h
                Xm[ix] -= h
                fd = (loss(*[Xp if Y is X else Y for Y in (Q, K, V)]) -
                      loss(*[Xm if Y is X else Y for Y in (Q, K, V)])) / (2 * h)
                assert abs(fd - Gr[ix]) < 1e-7 * max(1.0, abs(fd)), (ix, fd, Gr[ix])


# ---------------------------------------------------------------- block-sparse masks


def _bs_mask(rng, nb, density):
    return (rng.random((nb, nb)) < density).astype(np.uint8)


def check_blocksparse_full_and_causal_maps(seed=41):
    """An all-ones map is plain attention (causal or not); a lower-triangular
    map with causal is the causal mask; forward and backward.  N = 300 spans
    three 128-blocks with a ragged last one."""
    rng = np.random.default_rng(seed)
    n = 300
    nb = 3
    Q, K, V = _qkv(rng, 1, 2, 1, n, n, 4)
    dO = rng.standard_normal(Q.shape)
    ones = np.ones((nb, nb), dtype=np.uint8)
    tril = np.tril(ones)
    for mask, causal in ((ones, False), (ones, True), (tril, True)):
        O, L = OB.blocksparse_forward(Q, K, V, mask, 0.3, causal)
        Or, Lr = OA.attention_forward(Q, K, V, 0.3, causal)
        assert np.max(np.abs(O - Or)) < 1e-13 and np.max(np.abs(L - Lr)) < 1e-12
        g = OB.blocksparse_backward(Q, K, V, dO, mask, 0.3, causal)
        gr = OA.attention_backward(Q, K, V, dO, 0.3, causal)
        for a, b in zip(g, gr):
            assert np.max(np.abs(a - b)) < 1e-11


def check_blocksparse_block_diagonal(seed=42):
    """A block-diagonal map is independent attention inside every 128-block
    (the square definition on each slice, the last one ragged)."""
    rng = np.random.default_rng(seed)
    n = 290
    Q, K, V = _qkv(rng, 2, 2, 2, n, n, 3)
    mask = np.eye(3, dtype=np.uint8)
    for causal in (False, True):
        O, L = OB.blocksparse_forward(Q, K, V, mask, 0.5, causal)
        for b in range(2):
            for h in range(2):
                for a in range(0, n, OB.BLOCK):
                    e = min(n, a + OB.BLOCK)
                    o, l = OA.head_forward(Q[b, h, a:e], K[b, h, a:e], V[b, h, a:e], 0.5, causal)
                    assert np.max(np.abs(O[b, h, a:e] - o)) < 1e-13
                    assert np.max(np.abs(L[b, h, a:e] - l)) < 1e-12


def check_blocksparse_rows_are_gathers(seed=43):
    """Row i of a random map is the square definition of query i over the
    keys it sees, gathered (not masked) from K and V."""
    rng = np.random.default_rng(seed)
    n = 260
    Q, K, V = _qkv(rng, 1, 1, 1, n, n, 5)
    mask = _bs_mask(rng, 3, 0.6)
    mask[0, 0] = 1  # causal rows of block 0 then see at least their block
    for causal in (False, True):
        O, L = OB.blocksparse_forward(Q, K, V, mask, 0.7, causal)
        for i in range(0, n, 7):
            keys = [j for j in range(n) if mask[i // 128, j // 128] and (not causal or j <= i)]
            if not keys:
                assert np.all(O[0, 0, i] == 0) and L[0, 0, i] == -np.inf
                continue
            o, l = OA.head_forward(Q[0, 0, i:i + 1], K[0, 0, keys], V[0, 0, keys], 0.7, False)
            assert np.max(np.abs(O[0, 0, i] - o[0])) < 1e-13 and abs(L[0, 0, i] - l[0]) < 1e-12


def check_blocksparse_empty_rows(seed=44):
    """Query blocks whose map row is all zero see nothing: O = 0, LSE = -inf,
    dQ = 0 there, and the other rows and every dK / dV equal the same
    problem without those queries (they add no gradient)."""
    rng = np.random.default_rng(seed)
    n = 300
    Q, K, V = _qkv(rng, 1, 2, 1, n, n, 4)
    dO = rng.standard_normal(Q.shape)
    mask = np.array([[1, 0, 1], [0, 0, 0], [1, 1, 1]], dtype=np.uint8)
    O, L = OB.blocksparse_forward(Q, K, V, mask, 0.4, False)
    dQ, dK, dV = OB.blocksparse_backward(Q, K, V, dO, mask, 0.4, False)
    hid = slice(128, 256)
    assert np.all(O[:, :, hid] == 0) and np.all(L[:, :, hid] == -np.inf) and np.all(dQ[:, :, hid] == 0)
    keep = np.r_[0:128, 256:300]
    vis = OB.blocksparse_visible(n, mask, False)[keep]
    dKr, dVr = np.zeros_like(K), np.zeros_like(V)
    for h in range(2):
        s = np.where(vis, 0.4 * Q[0, h, keep] @ K[0, 0].T, -np.inf)
        m = s.max(axis=1)
        p = np.exp(s - m[:, None])
        p /= p.sum(axis=1)[:, None]
        assert np.max(np.abs(O[0, h, keep] - p @ V[0, 0])) < 1e-13
        dp = dO[0, h, keep] @ V[0, 0].T
        ds = p * (dp - (p * dp).sum(axis=1)[:, None])
        dKr[0, 0] += 0.4 * ds.T @ Q[0, h, keep]
        dVr[0, 0] += p.T @ dO[0, h, keep]
    assert np.max(np.abs(dK - dKr)) < 1e-12 and np.max(np.abs(dV - dVr)) < 1e-12


def check_blocksparse_finite_differences(seed=45):
    """Central differences of <dO, O> for a random map with causal, grouped
    heads, a ragged last block and an empty query block."""
    rng = np.random.default_rng(seed)
    n = 140
    Q, K, V = _qkv(rng, 1, 2, 1, n, n, 3)
    dO = rng.standard_normal(Q.shape)
    mask = np.array([[1, 0], [1, 1]], dtype=np.uint8)
    sc, h = 0.9, 1e-6
    for causal in (False, True):
        dQ, dK, dV = OB.blocksparse_backward(Q, K, V, dO, mask, sc, causal)

        def loss(q, k, v):
            return float((OB.blocksparse_forward(q, k, v, mask, sc, causal)[0] * dO).sum())

        for X, G in ((Q, dQ), (K, dK), (V, dV)):
            for _ in range(5):
                ix = tuple(int(rng.integers(0, s)) for s in X.shape)
                Xp, Xm = X.copy(), X.copy()
                Xp[ix] += h
                Xm[ix] -= h
                fd = (loss(*[Xp if Y is X else Y for Y in (Q, K, V)]) -
                      loss(*[Xm if Y is X else Y for Y in (Q, K, V)])) / (2 * h)
                assert abs(fd - G[ix]) < 1e-7 * max(1.0, abs(fd)), (ix, fd, G[ix])


# ---------------------------------------------------------------- dropout (Philox-4x32-10)


def check_philox_known_answers():
    """The generator reproduces the published known-answer values
    (tests/golden/philox4x32_10_kat.txt)."""
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rows.append([int(x, 16) for x in line.split()])
    assert len(rows) == 3
    for r in rows:
        got = ODR.philox4x32_10(*r[:4], *r[4:6])
        assert [int(x) for x in got] == r[6:], (r, [hex(int(x)) for x in got])


def check_dropout_mask_layout(seed=51):
    """Element (i, j) of unit bh is byte j % 4 of word i % 4 of the Philox
    block with counter (j // 4, i // 4, bh, offset): the vectorised mask
    equals that lookup done one element at a time; the keep rule is u >= t8."""
    rng = np.random.default_rng(seed)
    n, bh, sd, off, p = 37, 5, 0x1234567890ABCDEF, 3, 0.3
    keep = ODR.keep_mask(n, n, bh, p, sd, off)
    t8 = ODR.dropout_threshold(p)
    assert t8 == 77
    for _ in range(60):
        i, j = int(rng.integers(n)), int(rng.integers(n))
        w = ODR.philox4x32_10(j // 4, i // 4, bh, off, sd & 0xFFFFFFFF, sd >> 32)[i % 4]
        u = (int(w) >> (8 * (j % 4))) & 0xFF
        assert keep[i, j] == (u >= t8), (i, j)
    # different units, offsets and seeds give different masks
    assert not np.array_equal(keep, ODR.keep_mask(n, n, bh + 1, p, sd, off))
    assert not np.array_equal(keep, ODR.keep_mask(n, n, bh, p, sd, off + 1))
    assert not np.array_equal(keep, ODR.keep_mask(n, n, bh, p, sd + 1, off))


def check_dropout_keep_rate(seed=52):
    """Bytes are uniform: the kept fraction is 1 - t8 / 256 to within five
    standard deviations, and every byte value occurs about equally often."""
    n = 512
    for p in (0.1, 0.5, 0.75):
        keep = ODR.keep_mask(n, n, 2, p, 0xDEADBEEF + seed, 0)
        q = 1.0 - ODR.dropout_threshold(p) / 256.0
        sd = math.sqrt(q * (1 - q) / keep.size)
        assert abs(keep.mean() - q) < 5 * sd, (p, keep.mean(), q)
    i = np.arange(256)[:, None]
    j = np.arange(256)[None, :]
    words = ODR.philox4x32_10(j // 4, i // 4, 0, 0, 7, 9)
    u = (np.choose(i % 4, words) >> (8 * (j % 4)).astype(np.uint32)) & np.uint32(0xFF)
    counts = np.bincount(u.ravel(), minlength=256)
    expect = u.size / 256
    chi2 = float(((counts - expect) ** 2 / expect).sum())
    assert chi2 < 400, chi2  # 255 degrees of freedom


def check_dropout_zero_probability(seed=53):
    """p = 0 keeps everything: plain attention, forward and backward."""
    rng = np.random.default_rng(seed)
    Q, K, V = _qkv(rng, 2, 4, 2, 13, 13, 6)
    dO = rng.standard_normal(Q.shape)
    for causal in (False, True):
        O, L = ODR.dropout_forward(Q, K, V, 0.4, causal, 0.0, 99)
        Or, Lr = OA.attention_forward(Q, K, V, 0.4, causal)
        assert np.max(np.abs(O - Or)) < 1e-14 and np.max(np.abs(L - Lr)) < 1e-13
        g = ODR.dropout_backward(Q, K, V, dO, 0.4, causal, 0.0, 99)
        gr = OA.attention_backward(Q, K, V, dO, 0.4, causal)
        for a, b in zip(g, gr):
            assert np.max(np.abs(a - b)) < 1e-13


def check_dropout_unbiased(seed=54):
    """Inverted dropout keeps the expectation: O averaged over many seeds
    approaches plain attention (standard error about 0.005 here), and the
    LSE never changes."""
    rng = np.random.default_rng(seed)
    Q, K, V = _qkv(rng, 1, 1, 1, 12, 12, 3)
    Or, Lr = OA.attention_forward(Q, K, V, 0.5, False)
    acc = np.zeros_like(Or)
    S = 3000
    for s in range(S):
        O, L = ODR.dropout_forward(Q, K, V, 0.5, False, 0.25, s, 0)
        acc += O
        if s < 3:
            assert np.max(np.abs(L - Lr)) < 1e-13
    assert np.max(np.abs(acc / S - Or)) < 0.05
    # one seed: O is visibly different from plain attention
    O1, _ = ODR.dropout_forward(Q, K, V, 0.5, False, 0.25, 1, 0)
    assert np.max(np.abs(O1 - Or)) > 0.05


def check_dropout_finite_differences(seed=55):
    """Central differences of <dO, O> with the mask fixed by (seed, offset),
    grouped heads, causal and not."""
    rng = np.random.default_rng(seed)
    Q, K, V = _qkv(rng, 1, 2, 1, 9, 9, 3)
    dO = rng.standard_normal(Q.shape)
    sc, h, p, sd = 0.7, 1e-6, 0.3, 12345
    for causal in (False, True):
        dQ, dK, dV = ODR.dropout_backward(Q, K, V, dO, sc, causal, p, sd, 2)

        def loss(q, k, v):
            return float((ODR.dropout_forward(q, k, v, sc, causal, p, sd, 2)[0] * dO).sum())

        for X, G in ((Q, dQ), (K, dK), (V, dV)):
            for _ in range(6):
                ix = tuple(int(rng.integers(0, s)) for s in X.shape)
                Xp, Xm = X.copy(), X.copy()
                Xp[ix] += h
                Xm[ix] -= h
                fd = (loss(*[Xp if Y is X else Y for Y in (Q, K, V)]) -
                      loss(*[Xm if Y is X else Y for Y in (Q, K, V)])) / (2 * h)
                assert abs(fd - G[ix]) < 1e-7 * max(1.0, abs(fd)), (ix, fd, G[ix])


ALL_CHECKS = [
    check_four_token_tiles_consistent,
    check_four_token_recurrence_values,
    check_four_token_oracle,
    check_blocked_recurrence_matches,
    check_rows_sum_to_one,
    check_constant_v,
    check_equal_scores,
    check_single_token,
    check_causal_prefix,
    check_backward_finite_differences,
    check_against_torch_sdpa,
    check_grouped_heads,
    check_forward_rows,
    check_cross_square,
    check_cross_suffix,
    check_merge_four_token,
    check_merge_partition,
    check_merge_properties,
    check_window_special_cases,
    check_window_rows_are_slices,
    check_window_finite_differences,
    check_varlen_equal_lengths,
    check_varlen_ragged_slices,
    check_varlen_finite_differences,
    check_blocksparse_full_and_causal_maps,
    check_blocksparse_block_diagonal,
    check_blocksparse_rows_are_gathers,
    check_blocksparse_empty_rows,
    check_blocksparse_finite_differences,
    check_philox_known_answers,
    check_dropout_mask_layout,
    check_dropout_keep_rate,
    check_dropout_zero_probability,
    check_dropout_unbiased,
    check_dropout_finite_differences,
]
