"""Pins of the oracle's identification-accuracy reference (recall of the
softmax mass, position-based blocks).

Independent checks: the block labels in closed form, recall 1 when every
cluster is selected, recall equal to exp(lse over the selected keys - lse over
all keys) computed through the separately pinned block and dense attention,
recall monotone in p (top-p selections are nested), block representatives
equal to numpy's per-block mean, and on shuffled mixture data the pages' claim
that position-based blocks recall less than semantic clusters at the same
density.
"""
import math

import numpy as np
import pytest

import oracle


def _mixture(seed, N=512, d=16, comps=8, shuffle=True):
    rng = np.random.default_rng(seed)
    mu = 2.0 * rng.standard_normal((comps, d))
    z = np.sort(rng.integers(0, comps, N))
    if shuffle:
        z = rng.permutation(z)
    q = mu[z] + 0.3 * rng.standard_normal((N, d))
    k = mu[z] + 0.3 * rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    return q, k, v


def test_position_blocks_closed_form():
    z = oracle.position_blocks(300, 128)
    assert z.tolist() == [0] * 128 + [1] * 128 + [2] * 44


def test_recall_is_one_when_everything_is_selected():
    q, k, v = _mixture(0)
    r = oracle.layer(q, k, v, 6, 8, 3, top_p=1.0)
    rec = oracle.recall_rows(q, k, r.km_q.labels, r.km_k.labels, r.selection.lists, 1 / math.sqrt(16))
    np.testing.assert_allclose(rec, 1.0, rtol=0, atol=1e-14)
    b = oracle.positional_selection(q, k, 64, 1.0)
    rec = oracle.recall_rows(q, k, b.zq, b.zk, b.selection.lists, 1 / math.sqrt(16))
    np.testing.assert_allclose(rec, 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("top_p", [0.3, 0.7, 0.9])
def test_recall_equals_lse_difference(top_p):
    q, k, v = _mixture(1)
    s = 1 / math.sqrt(q.shape[1])
    r = oracle.layer(q, k, v, 6, 8, 3, top_p=top_p)
    rec = oracle.recall_rows(q, k, r.km_q.labels, r.km_k.labels, r.selection.lists, s)
    _, lse_all = oracle.softmax_attention_rows(q, k, v, s)
    np.testing.assert_allclose(rec, np.exp(r.lse - lse_all), rtol=1e-12, atol=0)


def test_recall_monotone_in_p():
    q, k, v = _mixture(2)
    s = 1 / math.sqrt(q.shape[1])
    prev_sem = prev_pos = None
    km_q = oracle.kmeans(q, 6, 3, seed=0)
    km_k = oracle.kmeans(k, 8, 3, seed=1)
    P = oracle.centroid_probs(km_q.centroids, km_k.centroids, km_k.counts, s)
    for p in (0.2, 0.5, 0.8, 0.95, 1.0):
        sel = oracle.select_topp(P, km_k.counts, p)
        sem = oracle.recall_rows(q, k, km_q.labels, km_k.labels, sel.lists, s)
        b = oracle.positional_selection(q, k, 64, p)
        pos = oracle.recall_rows(q, k, b.zq, b.zk, b.selection.lists, s)
        if prev_sem is not None:
            assert np.all(sem >= prev_sem - 1e-15) and np.all(pos >= prev_pos - 1e-15)
        prev_sem, prev_pos = sem, pos


def test_block_representatives_are_block_means():
    q, k, _ = _mixture(3, N=448)
    b = oracle.positional_selection(q, k, 64, 0.9)
    n = 7
    cq, _ = oracle.update(q, b.zq, np.zeros((n, q.shape[1])))
    expect = q.reshape(n, 64, -1).mean(axis=1).astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(cq, expect, rtol=1e-15, atol=0)
    assert b.pairs == sum(64 * 64 * len(l) for l in b.selection.lists)


def test_positional_blocks_recall_less_on_shuffled_tokens():
    """With the token order shuffled, fixed blocks mix semantics: at the same
    density they recall less mass than semantic clusters (wiki: Key claims,
    §3.2, Figs. 3-4)."""
    q, k, v = _mixture(4, N=1024, comps=8)
    s = 1 / math.sqrt(q.shape[1])
    km_q = oracle.kmeans(q, 8, 5, seed=0)
    km_k = oracle.kmeans(k, 8, 5, seed=1)
    P = oracle.centroid_probs(km_q.centroids, km_k.centroids, km_k.counts, s)
    sem = []
    for p in np.linspace(0.05, 1.0, 40):
        sel = oracle.select_topp(P, km_k.counts, p)
        dens = oracle.pair_count(sel.lists, km_q.counts, km_k.counts) / 1024 ** 2
        sem.append((dens, np.mean(oracle.recall_rows(q, k, km_q.labels, km_k.labels, sel.lists, s))))
    pos = []
    for p in np.linspace(0.05, 1.0, 40):
        b = oracle.positional_selection(q, k, 128, p)
        pos.append((b.pairs / 1024 ** 2, np.mean(oracle.recall_rows(q, k, b.zq, b.zk, b.selection.lists, s))))
    sem, pos = np.array(sorted(sem)), np.array(sorted(pos))
    for target in (0.25, 0.5):
        rs = np.interp(target, sem[:, 0], sem[:, 1])
        rp = np.interp(target, pos[:, 0], pos[:, 1])
        assert rs > rp + 0.05, (target, rs, rp)
