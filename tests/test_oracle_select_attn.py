"""Pins of the oracle's permutation, top-p selection and block attention.

Independent checks: a library routine (numpy's stable argsort, scipy's
softmax, torch's scaled-dot-product attention in fp64), closed forms
(two-cluster weights, dense equivalence at p = 1), brute force over all
subsets on tiny inputs, and invariants the pages fix (the permutation
cancels; top-p is monotone in p).
"""
import itertools
import math

import numpy as np
import pytest
import torch
from scipy.special import softmax

import oracle


# ---------------------------------------------------------------- permutation
def test_counting_sort_invariants():
    rng = np.random.default_rng(0)
    lab = rng.integers(0, 13, 500)
    lab[lab == 5] = 6                           # one empty cluster
    perm, off, cnt = oracle.counting_sort(lab, 13)
    assert sorted(perm.tolist()) == list(range(500))                # bijection
    s = lab[perm]
    assert np.all(np.diff(s) >= 0)                                  # sorted
    for c in range(13):                                             # stable
        seg = perm[off[c]:off[c + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(lab[seg] == c)
    assert cnt[5] == 0 and off[5] == off[6]
    assert off[0] == 0 and off[-1] == 500
    # the library's own stable sort of the keys gives the same permutation
    np.testing.assert_array_equal(perm, np.array(sorted(range(500), key=lambda t: (lab[t], t))))


def test_unpermute_inverts_permute():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((64, 3))
    perm = rng.permutation(64)
    np.testing.assert_array_equal(oracle.unpermute_rows(oracle.permute_rows(X, perm), perm), X)
    np.testing.assert_array_equal(oracle.permute_rows(X, perm)[3], X[perm[3]])


# ---------------------------------------------------------------- estimation
def test_two_cluster_closed_form():
    cq = np.array([[1.0, 2.0]])
    ck = np.array([[0.5, -1.0], [2.0, 1.0]])
    cnt = np.array([3, 7])
    s = 0.7
    P = oracle.centroid_probs(cq, ck, cnt, s)
    l0, l1 = s * (0.5 - 2.0), s * (2.0 + 2.0)
    p0 = 3 * math.exp(l0) / (3 * math.exp(l0) + 7 * math.exp(l1))
    np.testing.assert_allclose(P[0], [p0, 1 - p0], rtol=1e-14)


def test_identical_centroids_weight_by_key_cluster_size():
    ck = np.tile(np.array([[0.3, -0.2, 1.0]]), (5, 1))
    cnt = np.array([4, 1, 0, 10, 5])
    P = oracle.centroid_probs(np.random.default_rng(2).standard_normal((3, 3)), ck, cnt, 0.5)
    np.testing.assert_allclose(P, np.tile(cnt / cnt.sum(), (3, 1)), rtol=1e-14)


def test_probs_rows_sum_to_one_and_shift_invariance():
    rng = np.random.default_rng(3)
    cq, ck = rng.standard_normal((6, 8)), rng.standard_normal((20, 8))
    cnt = rng.integers(0, 5, 20)
    P = oracle.centroid_probs(cq, ck, cnt, 1 / math.sqrt(8))
    np.testing.assert_allclose(P.sum(1), 1.0, rtol=1e-14)
    assert np.all(P[:, cnt == 0] == 0)
    # adding one vector to every key centroid shifts each row's logits by a
    # constant, which the per-row normalisation removes
    P2 = oracle.centroid_probs(cq, ck + rng.standard_normal(8)[None], cnt, 1 / math.sqrt(8))
    np.testing.assert_allclose(P2, P, rtol=1e-10, atol=1e-15)


def _brute_min_subset(p_row, valid, top_p):
    idx = [j for j in range(len(p_row)) if valid[j]]
    for r in range(1, len(idx) + 1):
        best = None
        for sub in itertools.combinations(idx, r):
            if sum(p_row[j] for j in sub) >= top_p:
                best = sub
                break
        if best is not None:
            return r
    return len(idx)


@pytest.mark.parametrize("seed", range(6))
def test_topp_is_minimal_prefix_brute_force(seed):
    rng = np.random.default_rng(seed)
    n_k = 9
    cnt = rng.integers(0, 6, n_k)
    cnt[0] = max(cnt[0], 1)
    P = oracle.centroid_probs(rng.standard_normal((4, 5)), rng.standard_normal((n_k, 5)), cnt, 1.0)
    for top_p in (0.3, 0.5, 0.8, 0.95):
        sel = oracle.select_topp(P, cnt, top_p)
        for i in range(4):
            chosen = sel.lists[i]
            assert np.all(np.diff(chosen) > 0)                      # ascending
            assert P[i, chosen].sum() >= top_p - 1e-15
            assert len(chosen) == _brute_min_subset(P[i], cnt > 0, top_p)
            # the chosen ones are the largest: nothing outside beats anything inside
            out = [j for j in range(n_k) if cnt[j] > 0 and j not in chosen]
            if out:
                assert P[i, chosen].min() >= P[i, out].max()


def test_topp_special_cases():
    rng = np.random.default_rng(9)
    cnt = np.array([3, 0, 2, 8, 1, 4])
    P = oracle.centroid_probs(rng.standard_normal((5, 4)), rng.standard_normal((6, 4)), cnt, 0.5)
    s_all = oracle.select_topp(P, cnt, 1.0)
    for l in s_all.lists:
        assert l.tolist() == [0, 2, 3, 4, 5]                        # every non-empty cluster
    s_tiny = oracle.select_topp(P, cnt, 1e-9)
    for i, l in enumerate(s_tiny.lists):
        assert l.tolist() == [int(np.argmax(P[i]))]                 # the arg-max only
    prev = None
    for p in (0.1, 0.3, 0.5, 0.7, 0.9, 0.99):                       # monotone in p
        cur = oracle.select_topp(P, cnt, p).lists
        if prev is not None:
            for a, b in zip(prev, cur):
                assert set(a.tolist()) <= set(b.tolist())
        prev = cur


def test_topp_ties_prefer_lower_index():
    ck = np.zeros((4, 2))
    cnt = np.array([1, 1, 1, 1])
    P = oracle.centroid_probs(np.ones((1, 2)), ck, cnt, 1.0)         # all 0.25
    assert oracle.select_topp(P, cnt, 0.5).lists[0].tolist() == [0, 1]
    assert oracle.select_topp(P, cnt, 0.6).lists[0].tolist() == [0, 1, 2]


# ---------------------------------------------------------------- attention
def _mixture(seed, N=300, d=16, comps=6):
    rng = np.random.default_rng(seed)
    mu = rng.standard_normal((comps, d))
    z = rng.integers(0, comps, N)
    q = mu[z] + 0.3 * rng.standard_normal((N, d))
    k = mu[z] + 0.3 * rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    return q, k, v


def test_topp_ambiguous_flag_hand_built():
    """Rows whose cut sits within ``band`` of p, or whose order at the cut is
    within band * P_(1), are flagged; others are not.  Probabilities chosen by
    hand (exact binary fractions where equality matters)."""
    kc = np.ones(3, np.int64)
    P = np.array([[0.5, 0.25, 0.25],       # cumsum 0.5, 0.75, 1: p = 0.75 is reached exactly at the cut
                  [0.625, 0.25, 0.125],    # p = 0.7: cut at 1 (0.875); neighbours 0.625 and 0.875 are far
                  [0.375, 0.375, 0.25],    # p = 0.3: cut at 0, P_(1) = P_(2): a tie at the cut
                  [0.6, 0.3, 0.1]])        # p = 0.7: cut at 1; |0.6 - 0.7| = 0.1
    want = {(0, 0.75, 1e-12): True, (1, 0.7, 1e-12): False, (1, 0.7, 0.2): True,
            (2, 0.3, 1e-12): True, (3, 0.7, 0.05): False, (3, 0.7, 0.11): True}
    for (i, p, band), amb in want.items():
        sel = oracle.select_topp(P[i:i + 1], kc, p, band=band)
        assert bool(sel.ambiguous[0]) == amb, (i, p, band)
    # the lists themselves do not depend on the band
    assert list(oracle.select_topp(P[0:1], kc, 0.75).lists[0]) == [0, 1]
    assert list(oracle.select_topp(P[2:3], kc, 0.3).lists[0]) == [0]
    # p >= 1 keeps everything and is never ambiguous
    assert not oracle.select_topp(P, kc, 1.0, band=0.5).ambiguous.any()


def test_layer_at_p1_equals_dense_attention():
    """With every cluster selected the permutations cancel and the layer is
    plain softmax attention (wiki: Key claims, §4.1; Method, stage (2))."""
    q, k, v = _mixture(0)
    res = oracle.layer(q, k, v, n_q=5, n_k=8, iters=3, top_p=1.0)
    s = 1 / math.sqrt(q.shape[1])
    dense = softmax(s * q @ k.T, axis=1) @ v
    np.testing.assert_allclose(res.out, dense, rtol=0, atol=1e-12)
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])[0].numpy()
    np.testing.assert_allclose(res.out, t, rtol=0, atol=1e-12)
    lse = np.log(np.sum(np.exp(s * q @ k.T), axis=1))
    np.testing.assert_allclose(res.lse, lse, rtol=1e-13)


@pytest.mark.parametrize("top_p", [0.5, 0.8, 0.95])
def test_block_form_equals_masked_dense(top_p):
    """The permuted block computation equals masked attention in the original
    order, for any selection: this pins the permutation bookkeeping."""
    q, k, v = _mixture(1, N=400)
    res = oracle.layer(q, k, v, n_q=7, n_k=11, iters=2, top_p=top_p)
    s = 1 / math.sqrt(q.shape[1])
    o2, l2 = oracle.masked_dense_attention(q, k, v, res.km_q.labels, res.km_k.labels,
                                           res.selection.lists, s)
    np.testing.assert_allclose(res.out, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(res.lse, l2, rtol=1e-13)
    # masked attention written out directly for a few rows
    sel = res.selection.lists
    for t in (0, 17, 399):
        keys = [u for u in range(len(k)) if res.km_k.labels[u] in set(sel[res.km_q.labels[t]])]
        w = softmax(s * k[keys] @ q[t])
        np.testing.assert_allclose(res.out[t], w @ v[keys], rtol=0, atol=1e-12)
    assert res.pairs == sum(int(res.km_q.counts[i]) * int(res.km_k.counts[sel[i]].sum())
                            for i in range(7))


def test_empty_selection_row():
    q = np.ones((2, 4))
    o, l = oracle.block_attention(q, np.zeros((3, 4)), np.zeros((3, 4)),
                                  np.array([0, 2]), np.array([0, 3]), [np.zeros(0, np.int64)], 0.5)
    assert np.all(o == 0) and np.all(l == -np.inf)


def test_density_definition():
    assert oracle.density([25, 50], 10) == pytest.approx(0.375)
