"""Each plausible mistake planted in a copy of the oracle must fail a pin.

The mistakes are planted on the CPU by patching ``oracle.attention`` for the
duration of one test; the oracle on disk is never changed.
"""

import numpy as np
import pytest

import oracle.attention as OA
import oracle.blocksparse as OB
import oracle.dropout as ODR
import oracle.splitkv as OS
import oracle.varlen as OV
import oracle.window as OW
import oracle_pins


def _scores_no_scale(q, k, scale, causal):
    return OA_orig["_scores"](q, k, 1.0, causal)


def _scores_scale_twice(q, k, scale, causal):
    return OA_orig["_scores"](q, k, scale * scale, causal)


def _mask(q, k, scale, hide):
    s = scale * (q @ k.T)
    i = np.arange(q.shape[0])[:, None]
    j = np.arange(k.shape[0])[None, :]
    return np.where(hide(i, j), -np.inf, s)


def _scores_mask_diagonal(q, k, scale, causal):
    return _mask(q, k, scale, lambda i, j: j >= i) if causal else scale * (q @ k.T)


def _scores_mask_transposed(q, k, scale, causal):
    return _mask(q, k, scale, lambda i, j: j < i) if causal else scale * (q @ k.T)


def _softmax_no_shift(s):
    e = np.exp(s)
    l = e.sum(axis=1)
    return e / l[:, None], np.zeros(s.shape[0]), l


def _softmax_no_norm(s):
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    return e, m, e.sum(axis=1)


def _fwd_lse_no_max(q, k, v, scale, causal):
    p, m, l = OA._row_softmax(OA._scores(np.asarray(q, float), np.asarray(k, float), scale, causal))
    return p @ v, np.log(l)


def _fwd_pt_v(q, k, v, scale, causal):
    p, m, l = OA._row_softmax(OA._scores(np.asarray(q, float), np.asarray(k, float), scale, causal))
    return p.T @ v, m + np.log(l)


def _bwd_factory(change):
    def bwd(q, k, v, do, scale, causal):
        q, k, v, do = (np.asarray(x, float) for x in (q, k, v, do))
        p, _, _ = OA._row_softmax(OA._scores(q, k, scale, causal))
        dv = p.T @ do
        dp = do @ v.T
        d_row = (p * dp).sum(axis=1)
        ds = p * (dp - d_row[:, None])
        dq = scale * (ds @ k)
        dk = scale * (ds.T @ q)
        if change == "dv_no_transpose":
            dv = p @ do
        elif change == "ds_no_rowterm":
            ds = p * dp
            dq, dk = scale * (ds @ k), scale * (ds.T @ q)
        elif change == "dk_no_scale":
            dk = ds.T @ q
        elif change == "dq_transposed":
            dq = scale * (ds.T @ k)
        elif change == "dp_sign":
            ds = p * (d_row[:, None] - dp)
            dq, dk = scale * (ds @ k), scale * (ds.T @ q)
        return dq, dk, dv

    return bwd


def _kv_head_interleaved(h_q, n_heads_q, n_heads_kv):
    return h_q % n_heads_kv


def _rows_off_by_one(Q, K, V, scale, causal, b, h, rows):
    B, Hq, Hkv, N, d = OA._check_shapes(Q, K, V)
    g = OA.kv_head_of(h, Hq, Hkv)
    o = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    for t, i in enumerate(rows):
        s = scale * (K[b, g] @ Q[b, h, i])
        if causal:
            s = s[: max(i, 1)]
        m = s.max()
        e = np.exp(s - m)
        o[t] = (e / e.sum()) @ V[b, g, : s.shape[0]]
        lse[t] = m + np.log(e.sum())
    return o, lse


def _bwd_group_overwrite(Q, K, V, dO, scale, causal):
    B, Hq, Hkv, N, d = OA._check_shapes(Q, K, V)
    dQ, dK, dV = np.zeros(Q.shape), np.zeros(K.shape), np.zeros(V.shape)
    for b in range(B):
        for h in range(Hq):
            g = OA.kv_head_of(h, Hq, Hkv)
            dQ[b, h], dK[b, g], dV[b, g] = OA.head_backward(Q[b, h], K[b, g], V[b, g], dO[b, h], scale, causal)
    return dQ, dK, dV


OA_orig = {name: getattr(OA, name) for name in dir(OA) if not name.startswith("__")}
OS_orig = {name: getattr(OS, name) for name in dir(OS) if not name.startswith("__")}
OW_orig = {name: getattr(OW, name) for name in dir(OW) if not name.startswith("__")}


def _visible_top_left(n_q, n_k, causal, k_begin=0, k_end=None):
    k_end = n_k if k_end is None else k_end
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    vis = np.broadcast_to((j >= k_begin) & (j < k_end), (n_q, n_k))
    return vis & (j <= i) if causal else vis


def _visible_offset_sign(n_q, n_k, causal, k_begin=0, k_end=None):
    k_end = n_k if k_end is None else k_end
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    vis = np.broadcast_to((j >= k_begin) & (j < k_end), (n_q, n_k))
    return vis & (j <= i - (n_k - n_q)) if causal else vis


def _visible_range_short(n_q, n_k, causal, k_begin=0, k_end=None):
    k_end = n_k if k_end is None else k_end
    return OS_orig["_visible"](n_q, n_k, causal, k_begin, max(k_begin, k_end - 1))


def _window_off_by_one(n, left, right):
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    vis = np.ones((n, n), dtype=bool)
    if left >= 0:
        vis &= j > i - left
    if right >= 0:
        vis &= j <= i + right
    return vis


def _window_swapped(n, left, right):
    return OW_orig["window_visible"](n, right, left)


def _window_bwd_no_rowterm(Q, K, V, dO, scale, left, right):
    Q, K, V, dO = (np.asarray(x, float) for x in (Q, K, V, dO))
    B, Hq, Hkv, N, d = OA._check_shapes(Q, K, V)
    vis = OW.window_visible(N, left, right)
    dQ, dK, dV = np.zeros(Q.shape), np.zeros(K.shape), np.zeros(V.shape)
    for b in range(B):
        for h in range(Hq):
            g = OA.kv_head_of(h, Hq, Hkv)
            p, _, _ = OW._head_probs(Q[b, h], K[b, g], scale, vis)
            ds = p * (dO[b, h] @ V[b, g].T)
            dQ[b, h] = scale * (ds @ K[b, g])
            dK[b, g] += scale * (ds.T @ Q[b, h])
            dV[b, g] += p.T @ dO[b, h]
    return dQ, dK, dV


def _merge_unnormalised(O_parts, LSE_parts):
    O_parts, LSE_parts = np.asarray(O_parts, float), np.asarray(LSE_parts, float)
    w = np.where(np.isfinite(LSE_parts), np.exp(LSE_parts), 0.0)
    return (w[..., None] * O_parts).sum(axis=0), np.log(w.sum(axis=0))


def _merge_lse_max(O_parts, LSE_parts):
    O, _ = OS_orig["merge_partials"](O_parts, LSE_parts)
    return O, np.asarray(LSE_parts, float).max(axis=0)


def _merge_plain_mean(O_parts, LSE_parts):
    O, L = OS_orig["merge_partials"](O_parts, LSE_parts)
    return np.asarray(O_parts, float).mean(axis=0), L


def _varlen_fwd_factory(kind):
    def fwd(Q, K, V, cu, scale, causal):
        Q, K, V = (np.asarray(x, float) for x in (Q, K, V))
        Hq, Hkv = Q.shape[0], K.shape[0]
        cu = [int(x) for x in cu]
        O, L = np.zeros((Hq, Q.shape[1], V.shape[2])), np.zeros((Hq, Q.shape[1]))
        for a, b in zip(cu[:-1], cu[1:]):
            if b == a:
                continue
            ka = max(0, a - 1) if kind == "leak_previous" else a
            for h in range(Hq):
                g = OA.kv_head_of(h, Hq, Hkv)
                if kind == "leak_previous":
                    # keys of the previous sequence's last token visible too
                    q, k, v = Q[h, a:b], K[g, ka:b], V[g, ka:b]
                    s = scale * (q @ k.T)
                    if causal:
                        i = np.arange(b - a)[:, None] + (a - ka)
                        j = np.arange(b - ka)[None, :]
                        s = np.where(j > i, -np.inf, s)
                    p, m, l = OA._row_softmax(s)
                    O[h, a:b], L[h, a:b] = p @ v, m + np.log(l)
                else:  # "kv_head_by_query": the query head indexes K/V directly (mod H_kv)
                    O[h, a:b], L[h, a:b] = OA.head_forward(Q[h, a:b], K[h % Hkv, a:b], V[h % Hkv, a:b], scale, causal)
        return O, L

    return fwd


def _varlen_bwd_overwrite(Q, K, V, dO, cu, scale, causal):
    Q, K, V, dO = (np.asarray(x, float) for x in (Q, K, V, dO))
    Hq, Hkv = Q.shape[0], K.shape[0]
    cu = [int(x) for x in cu]
    dQ, dK, dV = np.zeros(Q.shape), np.zeros(K.shape), np.zeros(V.shape)
    for a, b in zip(cu[:-1], cu[1:]):
        if b == a:
            continue
        for h in range(Hq):
            g = OA.kv_head_of(h, Hq, Hkv)
            dq, dk, dv = OA.head_backward(Q[h, a:b], K[g, a:b], V[g, a:b], dO[h, a:b], scale, causal)
            dQ[h, a:b], dK[g, a:b], dV[g, a:b] = dq, dk, dv
    return dQ, dK, dV


def _bs_visible_transposed(n, mask, causal):
    return OB_orig["blocksparse_visible"](n, np.asarray(mask).T, causal)


def _bs_visible_block64(n, mask, causal):
    mask = np.asarray(mask)
    blk = np.minimum(np.arange(n) // 64, mask.shape[0] - 1)
    vis = mask[blk[:, None], blk[None, :]] != 0
    if causal:
        vis &= np.arange(n)[None, :] <= np.arange(n)[:, None]
    return vis


def _bs_probs_empty_rows_see_all(q, k, scale, vis):
    vis = np.where(vis.any(axis=1)[:, None], vis, True)
    return OB_orig["_probs"](q, k, scale, vis)


def _bs_bwd_no_rowterm(Q, K, V, dO, mask, scale, causal):
    Q, K, V, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, dO))
    B, Hq, Hkv, N, d = OA._check_shapes(Q, K, V)
    vis = OB.blocksparse_visible(N, mask, causal)
    dQ, dK, dV = np.zeros(Q.shape), np.zeros(K.shape), np.zeros(V.shape)
    for b in range(B):
        for h in range(Hq):
            g = OA.kv_head_of(h, Hq, Hkv)
            p, _ = OB._probs(Q[b, h], K[b, g], scale, vis)
            ds = p * (dO[b, h] @ V[b, g].T)
            dQ[b, h] = scale * (ds @ K[b, g])
            dK[b, g] += scale * (ds.T @ Q[b, h])
            dV[b, g] += p.T @ dO[b, h]
    return dQ, dK, dV


OB_orig = {"blocksparse_visible": OB.blocksparse_visible, "_probs": OB._probs}


def _philox_words_swapped(c0, c1, c2, c3, k0, k1):
    w = ODR_orig["philox4x32_10"](c0, c1, c2, c3, k0, k1)
    return [w[1], w[0], w[3], w[2]]


def _philox_no_key_bump(c0, c1, c2, c3, k0, k1):
    c = [np.asarray(x, dtype=np.uint64) & np.uint64(0xFFFFFFFF) for x in (c0, c1, c2, c3)]
    c = list(np.broadcast_arrays(*c))
    for _ in range(10):
        p0 = np.uint64(0xD2511F53) * c[0]
        p1 = np.uint64(0xCD9E8D57) * c[2]
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ np.uint64(k0), p1 & np.uint64(0xFFFFFFFF),
             (p0 >> np.uint64(32)) ^ c[3] ^ np.uint64(k1), p0 & np.uint64(0xFFFFFFFF)]
    return [x.astype(np.uint32) for x in c]


def _keep_counter_swapped(n_q, n_k, bh, p, seed, offset):
    t8 = ODR.dropout_threshold(p)
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    words = ODR.philox4x32_10(i // 4, j // 4, bh, offset, seed & 0xFFFFFFFF, seed >> 32)
    u = (np.choose(i % 4, words) >> (8 * (j % 4)).astype(np.uint32)) & np.uint32(0xFF)
    return u >= t8


def _keep_byte_by_query(n_q, n_k, bh, p, seed, offset):
    t8 = ODR.dropout_threshold(p)
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    words = ODR.philox4x32_10(j // 4, i // 4, bh, offset, seed & 0xFFFFFFFF, seed >> 32)
    u = (np.choose(j % 4, words) >> (8 * (i % 4)).astype(np.uint32)) & np.uint32(0xFF)
    return u >= t8


def _dropout_unit_unscaled(q, k, scale, causal, keep, t8):
    p, m, l = OA._row_softmax(OA._scores(q, k, scale, causal))
    return p, np.where(keep, p, 0.0), m + np.log(l)


def _dropout_bwd_dp_unmasked(Q, K, V, dO, scale, causal, p, seed, offset=0):
    Q, K, V, dO = (np.asarray(x, dtype=np.float64) for x in (Q, K, V, dO))
    B, Hq, Hkv, N, d = OA._check_shapes(Q, K, V)
    t8 = ODR.dropout_threshold(p)
    dQ, dK, dV = np.zeros(Q.shape), np.zeros(K.shape), np.zeros(V.shape)
    for b in range(B):
        for h in range(Hq):
            g = OA.kv_head_of(h, Hq, Hkv)
            keep = ODR.keep_mask(N, N, b * Hq + h, p, seed, offset)
            pr, pz, _ = ODR._unit(Q[b, h], K[b, g], scale, causal, keep, t8)
            dp = dO[b, h] @ V[b, g].T
            ds = pr * (dp - (pr * dp).sum(axis=1)[:, None])
            dQ[b, h] = scale * (ds @ K[b, g])
            dK[b, g] += scale * (ds.T @ Q[b, h])
            dV[b, g] += pz.T @ dO[b, h]
    return dQ, dK, dV


ODR_orig = {"philox4x32_10": ODR.philox4x32_10}


MUTANTS = {
    "scale_dropped": ("_scores", _scores_no_scale),
    "scale_twice": ("_scores", _scores_scale_twice),
    "mask_hides_diagonal": ("_scores", _scores_mask_diagonal),
    "mask_transposed": ("_scores", _scores_mask_transposed),
    "softmax_without_max_shift": ("_row_softmax", _softmax_no_shift),
    "softmax_not_normalised": ("_row_softmax", _softmax_no_norm),
    "lse_without_max": ("head_forward", _fwd_lse_no_max),
    "output_uses_p_transposed": ("head_forward", _fwd_pt_v),
    "dv_not_transposed": ("head_backward", _bwd_factory("dv_no_transpose")),
    "ds_missing_row_term": ("head_backward", _bwd_factory("ds_no_rowterm")),
    "dk_missing_scale": ("head_backward", _bwd_factory("dk_no_scale")),
    "dq_transposed": ("head_backward", _bwd_factory("dq_transposed")),
    "ds_sign_flipped": ("head_backward", _bwd_factory("dp_sign")),
    "kv_heads_interleaved": ("kv_head_of", _kv_head_interleaved),
    "rows_causal_off_by_one": ("attention_forward_rows", _rows_off_by_one),
    "group_grads_overwritten": ("attention_backward", _bwd_group_overwrite),
    "split_causal_top_left": (OS, "_visible", _visible_top_left),
    "split_causal_offset_sign": (OS, "_visible", _visible_offset_sign),
    "split_range_drops_last_key": (OS, "_visible", _visible_range_short),
    "merge_not_normalised": (OS, "merge_partials", _merge_unnormalised),
    "merge_lse_is_max": (OS, "merge_partials", _merge_lse_max),
    "merge_ignores_weights": (OS, "merge_partials", _merge_plain_mean),
    "window_left_off_by_one": (OW, "window_visible", _window_off_by_one),
    "window_sides_swapped": (OW, "window_visible", _window_swapped),
    "window_bwd_missing_row_term": (OW, "window_backward", _window_bwd_no_rowterm),
    "varlen_leaks_previous_sequence": (OV, "varlen_forward", _varlen_fwd_factory("leak_previous")),
    "varlen_kv_head_by_query_index": (OV, "varlen_forward", _varlen_fwd_factory("kv_head_by_query")),
    "varlen_group_grads_overwritten": (OV, "varlen_backward", _varlen_bwd_overwrite),
    "blocksparse_map_transposed": (OB, "blocksparse_visible", _bs_visible_transposed),
    "blocksparse_blocks_of_64": (OB, "blocksparse_visible", _bs_visible_block64),
    "blocksparse_empty_rows_see_all": (OB, "_probs", _bs_probs_empty_rows_see_all),
    "blocksparse_bwd_missing_row_term": (OB, "blocksparse_backward", _bs_bwd_no_rowterm),
    "philox_output_words_swapped": (ODR, "philox4x32_10", _philox_words_swapped),
    "philox_key_not_bumped": (ODR, "philox4x32_10", _philox_no_key_bump),
    "dropout_counter_query_key_swapped": (ODR, "keep_mask", _keep_counter_swapped),
    "dropout_byte_chosen_by_query": (ODR, "keep_mask", _keep_byte_by_query),
    "dropout_not_rescaled": (ODR, "_unit", _dropout_unit_unscaled),
    "dropout_bwd_dp_unmasked": (ODR, "dropout_backward", _dropout_bwd_dp_unmasked),
}


def _caught(check):
    try:
        with np.errstate(all="ignore"):
            check()
    except AssertionError:
        return True
    except (ValueError, FloatingPointError, ZeroDivisionError, IndexError):
        return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    spec = MUTANTS[name]
    mod, attr, fn = spec if len(spec) == 3 else (OA, *spec)
    monkeypatch.setattr(mod, attr, fn)
    caught = [c.__name__ for c in oracle_pins.ALL_CHECKS if _caught(c)]
    assert caught, f"no pin catches mutant {name}"
