"""Pins of the oracle's denoising-run reference (one layer over the steps).

Independent checks: the dense-step counts the reading fixes (5 of 50 steps,
1 of 10), torch's scaled-dot-product attention in fp64 for dense steps and for
a step at p = 1, the Lloyd fixed point (a warm start from converged centroids
on unchanged inputs changes nothing), and the oracle's own pinned assignment
for what a one-round warm start must produce from the cache.
"""
import numpy as np
import pytest
import torch

import oracle


def _mixture(seed, N=240, d=16, comps=5):
    rng = np.random.default_rng(seed)
    mu = 3.0 * rng.standard_normal((comps, d))
    z = rng.integers(0, comps, N)
    q = mu[z] + 0.3 * rng.standard_normal((N, d))
    k = mu[z] + 0.3 * rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    return q, k, v


def _drifting(steps, seed=0, drift=0.05):
    q, k, v = _mixture(seed)
    rng = np.random.default_rng(seed + 100)
    out = []
    for _ in range(steps):
        out.append((q.copy(), k.copy(), v.copy()))
        q = q + drift * rng.standard_normal(q.shape)
        k = k + drift * rng.standard_normal(k.shape)
        v = v + drift * rng.standard_normal(v.shape)
    return out


def _sdpa(q, k, v):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])[0].numpy()


@pytest.mark.parametrize("steps,fraction,n_dense", [
    (50, 0.1, 5), (10, 0.1, 1), (30, 0.1, 3), (12, 0.1, 2), (7, 0.0, 0), (4, 1.0, 4), (20, 0.25, 5)])
def test_dense_step_count(steps, fraction, n_dense):
    flags = [oracle.is_dense_step(s, steps, fraction) for s in range(steps)]
    assert sum(flags) == n_dense
    assert flags == [True] * n_dense + [False] * (steps - n_dense)      # the leading steps


def test_dense_steps_are_softmax_attention():
    seq = _drifting(3)
    r = oracle.denoise_layer(seq, 4, 6, 0.9, fraction=1.0, cold_iters=3, warm_iters=1)
    assert r.modes == ["dense"] * 3
    for (q, k, v), o in zip(seq, r.outs):
        np.testing.assert_allclose(o, _sdpa(q, k, v), rtol=0, atol=1e-12)


def test_modes_and_first_sparse_step_is_cold():
    """Dense steps leave the cache empty: the first sparse step is a cold
    start whatever came before it."""
    seq = _drifting(5)
    r = oracle.denoise_layer(seq, 4, 6, 0.9, fraction=0.4, cold_iters=3, warm_iters=2)
    assert r.modes == ["dense", "dense", "cold", "warm", "warm"]
    fresh = oracle.denoise_layer(seq[2:], 4, 6, 0.9, fraction=0.0, cold_iters=3, warm_iters=2)
    assert fresh.modes == ["cold", "warm", "warm"]
    for a, b in zip(r.outs[2:], fresh.outs):
        np.testing.assert_array_equal(a, b)


def test_warm_start_from_converged_centroids_is_a_fixed_point():
    q, k, v = _mixture(3)
    seq = [(q, k, v)] * 3
    r = oracle.denoise_layer(seq, 5, 5, 0.8, fraction=0.0, cold_iters=60, warm_iters=2)
    assert r.modes == ["cold", "warm", "warm"]
    for s in (1, 2):
        np.testing.assert_array_equal(r.layers[s].km_q.labels, r.layers[0].km_q.labels)
        np.testing.assert_array_equal(r.layers[s].km_k.labels, r.layers[0].km_k.labels)
        np.testing.assert_allclose(r.outs[s], r.outs[0], rtol=0, atol=1e-12)


def test_one_round_warm_start_assigns_to_the_cached_centroids():
    """With one warm round, step s's labels are this step's tokens assigned to
    the centroids step s-1 ended with (fp32, as cached)."""
    seq = _drifting(4, seed=5, drift=0.2)
    r = oracle.denoise_layer(seq, 4, 6, 0.9, fraction=0.0, cold_iters=3, warm_iters=1)
    for s in (1, 2, 3):
        q, k, _ = seq[s]
        cq = r.layers[s - 1].km_q.centroids.astype(np.float32).astype(np.float64)
        ck = r.layers[s - 1].km_k.centroids.astype(np.float32).astype(np.float64)
        np.testing.assert_array_equal(r.layers[s].km_q.labels, oracle.assign(q, cq).labels)
        np.testing.assert_array_equal(r.layers[s].km_k.labels, oracle.assign(k, ck).labels)


def test_top_p_schedule_step_at_one_is_dense_attention():
    seq = _drifting(3, seed=7)
    sched = lambda s: 1.0 if s == 1 else 0.5
    r = oracle.denoise_layer(seq, 4, 6, sched, fraction=0.0, cold_iters=3, warm_iters=2)
    q, k, v = seq[1]
    np.testing.assert_allclose(r.outs[1], _sdpa(q, k, v), rtol=0, atol=1e-12)
    assert r.layers[0].pairs < q.shape[0] ** 2                           # p = 0.5 is sparse here
