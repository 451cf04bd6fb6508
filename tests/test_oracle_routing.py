"""Pins for the oracle's router and permutation: brute force on every token,
closed forms, library softmax and invariants (no GPU)."""
import numpy as np
import pytest
import scipy.special

import oracle


def _brute_topk(lrow, k):
    """Rank of e = number of experts with a larger logit, or an equal logit and a lower index."""
    l = np.where(lrow == 0, 0.0, lrow.astype(np.float64))
    E = l.size
    rank = np.array([np.sum((l > l[e]) | ((l == l[e]) & (np.arange(E) < e))) for e in range(E)])
    out = np.full(k, -1)
    for e in range(E):
        if rank[e] < k:
            out[rank[e]] = e
    return out


def _adversarial_logits(E, rng):
    rows = [
        np.zeros(E, np.float32),                                           # all equal
        np.full(E, -3.25, np.float32),
        np.where(np.arange(E) % 2 == 0, 0.0, -0.0).astype(np.float32),    # +0 / -0 mix
        np.repeat(rng.standard_normal(E // 4 + 1), 4)[:E].astype(np.float32),  # ties in groups of 4
        np.concatenate([np.full(3, 5.0), np.full(E - 3, 1.0)]).astype(np.float32),  # ties across boundary
        rng.permutation(np.arange(E, dtype=np.float32)),
        np.round(rng.standard_normal(E) * 2).astype(np.float32),           # many integer ties
    ]
    r = rng.standard_normal(E).astype(np.float32)
    r[E - 1] = r.max() + 1                                                # max at the last index
    r[E - 2] = r[E - 1]                                                   # duplicated maximum
    rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("E,K", [(16, 4), (256, 8), (7, 7), (256, 1), (64, 8)])
def test_route_ids_match_brute_force(E, K):
    rng = np.random.default_rng(E * 100 + K)
    L = np.concatenate([(rng.standard_normal((40, E)) * 1.4).astype(np.float32),
                        _adversarial_logits(E, rng)])
    ids, _ = oracle.route(L, K)
    for t in range(L.shape[0]):
        np.testing.assert_array_equal(ids[t], _brute_topk(L[t], K), err_msg=f"row {t}")


def test_route_all_equal_gives_first_k():
    ids, w = oracle.route(np.zeros((3, 256), np.float32), 8)
    np.testing.assert_array_equal(ids, np.tile(np.arange(8), (3, 1)))
    np.testing.assert_array_equal(w, np.float32(1 / 8))


def test_route_k1_weight_is_one():
    rng = np.random.default_rng(0)
    _, w = oracle.route(rng.standard_normal((50, 256)).astype(np.float32), 1)
    np.testing.assert_array_equal(w, np.float32(1.0))


def test_route_k_equals_e_is_softmax():
    rng = np.random.default_rng(1)
    L = (rng.standard_normal((30, 16)) * 2).astype(np.float32)
    ids, w = oracle.route(L, 16)
    ref = scipy.special.softmax(L.astype(np.float64), axis=1)
    got = np.zeros_like(ref)
    np.put_along_axis(got, ids.astype(np.int64), w.astype(np.float64), axis=1)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-7)


def test_route_weights_closed_form_and_sum():
    rng = np.random.default_rng(2)
    L = (rng.standard_normal((200, 256)) * 1.43).astype(np.float32)
    ids, w = oracle.route(L, 8)
    l = np.take_along_axis(L.astype(np.float64), ids.astype(np.int64), 1)
    ref = np.exp(l - l[:, :1]) / np.exp(l - l[:, :1]).sum(1, keepdims=True)
    np.testing.assert_allclose(w, ref, rtol=0, atol=1e-7)
    np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)  # slots ordered by rank


def test_route_weights_ignore_unselected_logits():
    rng = np.random.default_rng(4)
    L = (rng.standard_normal((100, 256)) * 1.43).astype(np.float32)
    ids, w = oracle.route(L, 8)
    L2 = L.copy()
    kth = np.take_along_axis(L, ids[:, 7:8].astype(np.int64), 1)
    mask = np.ones_like(L, bool)
    np.put_along_axis(mask, ids.astype(np.int64), False, 1)
    L2[mask] = (kth - 5.0 - rng.random(L.shape).astype(np.float32))[mask]  # push the rest further down
    ids2, w2 = oracle.route(L2, 8)
    np.testing.assert_array_equal(ids, ids2)
    np.testing.assert_allclose(w, w2, rtol=0, atol=1e-7)


# --- permutation -------------------------------------------------------------------------

def _check_permutation(ids, e0, e_loc):
    T, K = ids.shape
    off, rt, rs, tr = oracle.permute(ids, e0, e_loc)
    local = (ids >= e0) & (ids < e0 + e_loc)
    M = int(local.sum())
    assert off[0] == 0 and off[-1] == M and np.all(np.diff(off) >= 0)
    assert rt.size == M and rs.size == M
    for el in range(e_loc):  # each expert's block: its pairs in ascending token order
        r0, r1 = off[el], off[el + 1]
        tt, kk = np.nonzero(ids == e0 + el)
        np.testing.assert_array_equal(rt[r0:r1], tt)
        np.testing.assert_array_equal(rs[r0:r1], kk)
    for t in range(T):
        for k in range(K):
            if local[t, k]:
                r = tr[t, k]
                assert rt[r] == t and rs[r] == k
            else:
                assert tr[t, k] == -1
    # permute then unpermute is the identity on token-row payloads
    payload = np.arange(T * 3).reshape(T, 3)
    rows = payload[rt]
    back = np.full((T, K, 3), -1)
    back[local] = rows[tr[local]]
    np.testing.assert_array_equal(back[local], np.broadcast_to(payload[:, None, :], (T, K, 3))[local])
    return off, rt, rs, tr


def test_permute_invariants_random():
    rng = np.random.default_rng(6)
    L = rng.standard_normal((300, 64)).astype(np.float32)
    ids, _ = oracle.route(L, 8)
    _check_permutation(ids, 0, 64)
    _check_permutation(ids, 16, 8)  # a local window, pairs elsewhere are dropped


def test_permute_all_tokens_one_expert():
    T, K = 50, 4
    ids = np.tile(np.array([3, 0, 1, 2]), (T, 1)).astype(np.int32)
    off, rt, rs, tr = _check_permutation(ids, 0, 8)
    np.testing.assert_array_equal(off, [0, 50, 100, 150, 200, 200, 200, 200, 200])
    np.testing.assert_array_equal(rt[150:200], np.arange(T))
    np.testing.assert_array_equal(rs[150:200], 0)


def test_permute_identity_special_case():
    """K=1 and e = t mod E: rows are token t at row (t mod E) * (T/E) + t // E."""
    T, E = 64, 16
    ids = (np.arange(T) % E).reshape(T, 1).astype(np.int32)
    off, rt, rs, tr = _check_permutation(ids, 0, E)
    np.testing.assert_array_equal(off, np.arange(E + 1) * (T // E))
    t = np.arange(T)
    np.testing.assert_array_equal(tr[:, 0], (t % E) * (T // E) + t // E)


def test_permute_no_local_pairs():
    ids = np.full((10, 2), 40, np.int32)
    ids[:, 1] = 41
    off, rt, rs, tr = _check_permutation(ids, 0, 32)
    assert off[-1] == 0 and np.all(tr == -1)


# --------------------------------------------------------------------------- routing variants

def _brute_grouped(lrow, k, n_group, topk_group):
    """Rank the groups by their best logit (ties: lower group), keep topk_group of them, then rank the kept
    experts with the ungrouped rule; every rank counted explicitly."""
    l = np.where(lrow == 0, 0.0, lrow.astype(np.float64))
    E = l.size
    gs = E // n_group
    score = [max(l[g * gs:(g + 1) * gs]) for g in range(n_group)]
    keep = [g for g in range(n_group)
            if sum((score[h] > score[g]) or (score[h] == score[g] and h < g) for h in range(n_group)) < topk_group]
    allowed = [e for e in range(E) if e // gs in keep]
    out = [None] * k
    for e in allowed:
        r = sum((l[f] > l[e]) or (l[f] == l[e] and f < e) for f in allowed)
        if r < k:
            out[r] = e
    return np.array(out)


def test_grouped_route_hand_example():
    # groups {0,1} {2,3} {4,5} {6,7}; best logits 0.9, 0.5, 0.8, 0.3 -> keep groups 0 and 2 -> experts {0,1,4,5}
    L = np.array([[0.1, 0.9, 0.5, 0.4, 0.8, 0.0, 0.3, 0.2]], np.float32)
    ids, w = oracle.route(L, 3, n_group=4, topk_group=2)
    np.testing.assert_array_equal(ids, [[1, 4, 0]])          # ungrouped would be [1, 4, 2]
    e = np.exp(np.array([0.9, 0.8, 0.1], np.float64) - 0.9)
    np.testing.assert_allclose(w[0], e / e.sum(), rtol=1e-7)
    # not renormalised: the plain softmax probabilities of the chosen experts, then scaled
    ids2, w2 = oracle.route(L, 3, n_group=4, topk_group=2, renormalize=False, scaling=2.5)
    p = scipy.special.softmax(L[0].astype(np.float64))
    np.testing.assert_array_equal(ids2, ids)
    np.testing.assert_allclose(w2[0], 2.5 * p[[1, 4, 0]], rtol=1e-7)


@pytest.mark.parametrize("E,K,G,TG", [(8, 3, 4, 2), (16, 4, 4, 1), (12, 5, 3, 2), (64, 8, 8, 4), (256, 8, 8, 4)])
def test_grouped_route_matches_brute_force(E, K, G, TG):
    rng = np.random.default_rng(E * 31 + G)
    L = np.concatenate([_adversarial_logits(E, rng), (rng.standard_normal((40, E)) * 1.43).astype(np.float32)])
    ids, w = oracle.route(L, K, n_group=G, topk_group=TG)
    for t in range(L.shape[0]):
        np.testing.assert_array_equal(ids[t], _brute_grouped(L[t], K, G, TG))
        groups = set(int(e) // (E // G) for e in ids[t])
        assert len(groups) <= TG
    assert np.allclose(w.astype(np.float64).sum(1), 1.0, atol=1e-6)


def test_grouped_route_degenerate_cases_reduce_to_ungrouped():
    rng = np.random.default_rng(3)
    L = (rng.standard_normal((100, 64)) * 1.43).astype(np.float32)
    base = oracle.route(L, 8)
    for G in (1, 2, 8, 64):
        ids, w = oracle.route(L, 8, n_group=G, topk_group=G)   # every group kept
        np.testing.assert_array_equal(ids, base[0])
        np.testing.assert_array_equal(w, base[1])
    # one expert per group: group selection is itself a top-topk_group, then top-k of those
    ids, _ = oracle.route(L, 4, n_group=64, topk_group=6)
    np.testing.assert_array_equal(ids, base[0][:, :4])


def _brute_sigmoid(lrow, bias, k, n_group, topk_group):
    """Every rank counted explicitly: scores in float64 rounded to float32, biased scores for selection, groups
    scored by their two best biased scores."""
    s = np.array([np.float32(1.0 / (1.0 + np.exp(-float(v)))) for v in lrow], np.float32)
    b = np.array([np.float32(s[e] + np.float32(bias[e])) for e in range(lrow.size)], np.float32)
    E = lrow.size
    gs = E // n_group
    if gs == 1:
        score = [float(b[g]) for g in range(n_group)]
    else:
        score = []
        for g in range(n_group):
            top = sorted((float(v) for v in b[g * gs:(g + 1) * gs]), reverse=True)
            score.append(float(np.float32(np.float32(top[0]) + np.float32(top[1]))))
    keep = [g for g in range(n_group)
            if sum((score[h] > score[g]) or (score[h] == score[g] and h < g) for h in range(n_group)) < topk_group]
    allowed = [e for e in range(E) if e // gs in keep]
    out = [None] * k
    for e in allowed:
        r = sum((b[f] > b[e]) or (b[f] == b[e] and f < e) for f in allowed)
        if r < k:
            out[r] = e
    return np.array(out), s


def test_sigmoid_route_hand_example():
    # logits 0 -> s = 0.5 exactly; bias moves expert 3 ahead of expert 1 for selection only
    L = np.array([[2.0, 1.0, 0.0, 0.5]], np.float32)
    bias = np.array([0.0, 0.0, 0.0, 0.2], np.float32)
    ids, w = oracle.route_sigmoid(L, 2, bias=bias)
    s = 1.0 / (1.0 + np.exp(-np.array([2.0, 1.0, 0.0, 0.5])))
    assert s[3] + 0.2 > s[1]
    np.testing.assert_array_equal(ids, [[0, 3]])
    np.testing.assert_allclose(w[0], s[[0, 3]] / s[[0, 3]].sum(), rtol=1e-7)   # unbiased scores, renormalised
    ids2, w2 = oracle.route_sigmoid(L, 2, bias=bias, renormalize=False, scaling=2.0)
    np.testing.assert_allclose(w2[0], 2.0 * s[[0, 3]], rtol=1e-6)


@pytest.mark.parametrize("E,K,G,TG", [(8, 3, 1, 1), (16, 4, 4, 2), (12, 5, 3, 2), (64, 8, 8, 4), (32, 4, 32, 5)])
def test_sigmoid_route_matches_brute_force(E, K, G, TG):
    rng = np.random.default_rng(E * 17 + G)
    L = np.concatenate([_adversarial_logits(E, rng), (rng.standard_normal((30, E)) * 2).astype(np.float32)])
    bias = (rng.standard_normal(E) * 0.05).astype(np.float32)
    bias[: E // 4] = 0.0
    ids, w = oracle.route_sigmoid(L, K, bias=bias, n_group=G, topk_group=TG)
    for t in range(L.shape[0]):
        ref, s = _brute_sigmoid(L[t], bias, K, G, TG)
        np.testing.assert_array_equal(ids[t], ref)
        sel = s[ref].astype(np.float64)
        np.testing.assert_allclose(w[t], sel / sel.sum(), rtol=1e-6)


def test_sigmoid_route_without_bias_is_monotone_in_logits():
    """With no bias and no groups, sigmoid is monotone: the selected set equals the softmax router's."""
    rng = np.random.default_rng(9)
    L = (rng.standard_normal((200, 64)) * 3).astype(np.float32)
    ids_s, _ = oracle.route_sigmoid(L, 8)
    ids_m, _ = oracle.route(L, 8)
    # equal float32 sigmoid values (saturated logits) may break ties differently; compare where distinct
    s = oracle.sigmoid_scores(L)
    distinct = np.array([np.unique(np.sort(s[t])[::-1][:9]).size == 9 for t in range(L.shape[0])])
    np.testing.assert_array_equal(ids_s[distinct], ids_m[distinct])


# --------------------------------------------------------------------------- router logits

def _bf16_values(rng, shape):
    """Random finite BF16 values (as float64): float32 draws with the low 16 bits cleared."""
    v = rng.standard_normal(shape).astype(np.float32)
    return (v.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)


def test_router_logits_brute_force_sum():
    """Every logit is the FP32 rounding of the exact dot product: each BF16 x FP32 product is exact in float64,
    math.fsum adds them with one rounding, and the float32 cast rounds once more."""
    import math
    rng = np.random.default_rng(11)
    T, E, H = 6, 5, 96
    x = _bf16_values(rng, (T, H))
    w = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    got = oracle.router_logits(x, w)
    assert got.dtype == np.float32 and got.shape == (T, E)
    want = np.array([[np.float32(math.fsum(float(x[t, h]) * float(w[e, h]) for h in range(H))) for e in range(E)]
                     for t in range(T)], dtype=np.float32)
    np.testing.assert_array_equal(got, want)


def test_router_logits_special_weights():
    """One-hot router rows pick one hidden column of x exactly (so a transposed operand or a wrong index shows);
    doubling W_r doubles every logit exactly; a negated row gives the negated logit."""
    rng = np.random.default_rng(12)
    T, H = 9, 40
    x = _bf16_values(rng, (T, H))
    cols = np.array([0, 7, 39, 13])
    w = np.zeros((cols.size, H), np.float32)
    w[np.arange(cols.size), cols] = 1.0
    np.testing.assert_array_equal(oracle.router_logits(x, w), x[:, cols].astype(np.float32))
    w2 = (rng.standard_normal((3, H)) * 0.05).astype(np.float32)
    l2 = oracle.router_logits(x, w2)
    np.testing.assert_array_equal(oracle.router_logits(x, 2 * w2), 2 * l2)
    np.testing.assert_array_equal(oracle.router_logits(x, -w2), -l2)
