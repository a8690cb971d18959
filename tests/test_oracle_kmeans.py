"""Pins of the oracle's random numbers, k-means++ seeding and Lloyd iterations.

Each check is independent of the oracle's own code: a published test vector,
a library routine (scikit-learn's Lloyd k-means, scipy's chi-square test),
brute force on tiny inputs, or an invariant the method fixes (every centroid
is the mean of its members; the objective never increases).
"""
import os

import numpy as np
import pytest
from scipy import stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_ints(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [int(l, 16) for l in f if l.strip() and not l.startswith("#")]


# ---------------------------------------------------------------- generator
def test_splitmix64_published_vector():
    want = _golden_ints("splitmix64_state0.txt")
    gamma = 0x9E3779B97F4A7C15
    got = [oracle.splitmix64((i * gamma) & ((1 << 64) - 1)) for i in range(len(want))]
    assert got == want


def test_seeding_uniform_range_and_uniformity():
    u = np.array([oracle.seeding_uniform(1234, p, k) for p in range(4) for k in range(5000)])
    assert u.min() >= 0.0 and u.max() < 1.0
    hist, _ = np.histogram(u, bins=20, range=(0, 1))
    assert stats.chisquare(hist).pvalue > 1e-4
    # distinct problems and picks give distinct streams
    assert oracle.seeding_uniform(7, 0, 1) != oracle.seeding_uniform(7, 1, 1)
    assert oracle.seeding_uniform(7, 0, 1) != oracle.seeding_uniform(7, 0, 2)


@pytest.mark.parametrize("problem,pick", [(0, 0), (0, 7), (3, 0), (5, 999), ((1 << 20) + 1, 12345)])
def test_seeding_uniform_published_vector(problem, pick):
    """u(seed, problem, pick) is the top 53 bits of splitmix64 of
    seed XOR (problem * 2^32 + pick), times 2^-53.  With the seed chosen so that
    this state is i * gamma, the generator's output is output i of the
    published vector: a '+' for the XOR, a dropped or shifted problem term, or
    a wrong bit count in the conversion fails it."""
    want = _golden_ints("splitmix64_state0.txt")
    gamma = 0x9E3779B97F4A7C15
    for i, w in enumerate(want):
        state = (i * gamma) & ((1 << 64) - 1)
        seed = state ^ ((problem << 32) + pick)
        u = oracle.seeding_uniform(seed, problem, pick)
        assert u == (w >> 11) / 2.0 ** 53
        assert u == float(np.ldexp(float(w >> 11), -53))


# ---------------------------------------------------------------- k-means++
def _kmeanspp_with_uniforms(monkeypatch, X, n, us):
    """kmeanspp with the draws u_k replaced by the given values."""
    from oracle import svg2_oracle as so
    monkeypatch.setattr(so, "seeding_uniform", lambda seed, problem, k: us[k])
    return so.kmeanspp(X, n, seed=0)


def test_kmeanspp_margin_hand_built(monkeypatch):
    """Points 0, 1, 3 on a line, pick 0 = token 0 (u_0 = 0): D2 = (0, 1, 9),
    cumulative sums (0, 1, 10).  u_1 = 0.3 puts the target at 3, inside token
    2's interval (1, 10]: margin = min(3 - 1, 10 - 3) / 10 = 0.2.  u_1 = 0.05
    puts it at 0.5 in token 1's interval (0, 1]: margin = 0.05."""
    X = np.array([[0.0], [1.0], [3.0]])
    r = _kmeanspp_with_uniforms(monkeypatch, X, 2, [0.0, 0.3])
    assert list(r.index) == [0, 2]
    assert r.margin[0] == np.inf
    assert abs(r.margin[1] - 0.2) < 1e-15
    r = _kmeanspp_with_uniforms(monkeypatch, X, 2, [0.0, 0.05])
    assert list(r.index) == [0, 1]
    assert abs(r.margin[1] - 0.05) < 1e-15


def test_kmeanspp_margin_is_the_pick_preserving_radius(monkeypatch):
    """The margin of pick k is how far u_k may move with the pick unchanged:
    moving u_k by 0.999 margin keeps it, moving it by 1.001 margin one way or
    the other changes it."""
    X = np.random.default_rng(3).standard_normal((40, 4))
    for u1 in (0.137, 0.5, 0.861):
        base = _kmeanspp_with_uniforms(monkeypatch, X, 2, [0.25, u1])
        m = base.margin[1]
        assert 0 < m < 0.5
        for f in (0.999, -0.999):
            assert _kmeanspp_with_uniforms(monkeypatch, X, 2, [0.25, u1 + f * m]).index[1] == base.index[1]
        moved = [_kmeanspp_with_uniforms(monkeypatch, X, 2, [0.25, u1 + f * m]).index[1] for f in (1.001, -1.001)]
        assert any(t != base.index[1] for t in moved)


def test_kmeanspp_first_pick_and_rows():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((97, 5))
    r = oracle.kmeanspp(X, 10, seed=42, problem=3)
    assert r.index[0] == int(np.floor(oracle.seeding_uniform(42, 3, 0) * 97))
    np.testing.assert_array_equal(r.centroids, X[r.index])
    assert len(set(r.index.tolist())) == 10          # no repeats while sum D2 > 0


def test_kmeanspp_picks_every_row_when_n_equals_N():
    X = np.random.default_rng(1).standard_normal((12, 3))
    r = oracle.kmeanspp(X, 12, seed=5)
    assert sorted(r.index.tolist()) == list(range(12))


def test_kmeanspp_duplicate_rows_fallback():
    # three distinct rows, five picks: after three picks every D2 is zero and
    # the uniform fallback floor(u N) takes over
    X = np.repeat(np.eye(3), 2, axis=0)
    r = oracle.kmeanspp(X, 5, seed=9)
    assert len({tuple(X[i]) for i in r.index[:3]}) == 3
    for k in (3, 4):
        assert r.index[k] == int(np.floor(oracle.seeding_uniform(9, 0, k) * 6))


@pytest.mark.parametrize("pick", [1, 2])
def test_kmeanspp_d2_distribution_chi_square(pick):
    """Pick k is distributed as D^2 / sum D^2 given the earlier picks
    (Arthur & Vassilvitskii 2007).  Sampling with D instead of D^2, or with the
    distance to the last centre instead of the nearest one, fails this."""
    X = np.array([[0.0, 0.0], [1.0, 0.0], [0.0, 2.0], [3.0, 3.0], [-1.5, 0.5]])
    N = len(X)
    counts = {}
    for s in range(30000):
        idx = oracle.kmeanspp(X, pick + 1, seed=s).index
        key = tuple(idx[:pick])
        counts.setdefault(key, np.zeros(N))
        counts[key][idx[pick]] += 1
    tested = 0
    for key, c in counts.items():
        if c.sum() < 400:
            continue
        D2 = np.min([np.sum((X - X[j]) ** 2, axis=1) for j in key], axis=0)
        p = D2 / D2.sum()
        pos = p > 0
        assert np.all(c[~pos] == 0)
        res = stats.chisquare(c[pos], c.sum() * p[pos])
        assert res.pvalue > 1e-5, (key, c, p)
        tested += 1
    assert tested >= 3


# ---------------------------------------------------------------- Lloyd
def _blobs(seed, N=600, d=6, k=5, sigma=0.4):
    rng = np.random.default_rng(seed)
    mu = 3.0 * rng.standard_normal((k, d))
    z = rng.integers(0, k, N)
    return mu[z] + sigma * rng.standard_normal((N, d))


def test_assign_brute_force():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((10, 4))
    C = rng.standard_normal((6, 4))
    a = oracle.assign(X, C)
    for t in range(10):
        d = [sum((X[t, i] - C[c, i]) ** 2 for i in range(4)) for c in range(6)]
        best = min(range(6), key=lambda c: (d[c], c))
        assert a.labels[t] == best
        assert abs(a.min_dist[t] - d[best]) < 1e-12
        srt = sorted(d)
        m = (srt[1] - srt[0]) / (np.sum(X[t] ** 2) + np.sum(C[best] ** 2))
        assert abs(a.margin[t] - m) < 1e-12


def test_assign_exact_tie_goes_to_lowest_index():
    X = np.array([[0.0, 0.0]])
    C = np.array([[1.0, 0.0], [0.0, 1.0], [-1.0, 0.0]])
    a = oracle.assign(X, C)
    assert a.labels[0] == 0 and a.margin[0] == 0.0


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_lloyd_matches_sklearn(seed):
    """scikit-learn's Lloyd k-means from the same initial centres gives the
    same centres whenever no cluster empties (sklearn relocates empty ones)."""
    from sklearn.cluster import KMeans
    X = _blobs(seed)
    C0 = X[[0, 50, 100, 150, 200, 250, 300]]
    T = 4
    ours = oracle.kmeans(X, 7, T, init=C0, round_fp32=False)
    assert np.all(ours.counts > 0)
    km = KMeans(n_clusters=7, init=C0, n_init=1, max_iter=T, tol=0.0, algorithm="lloyd").fit(X)
    np.testing.assert_allclose(ours.centroids, km.cluster_centers_, rtol=0, atol=1e-10)


def test_lloyd_invariants():
    X = _blobs(7, N=800)
    r = oracle.kmeans(X, 9, 6, seed=3)
    # centroid = mean of members (up to fp32 rounding of the stored centroid)
    for c in range(9):
        mem = X[r.labels == c]
        if len(mem):
            np.testing.assert_allclose(r.centroids[c], mem.mean(0), rtol=1e-6, atol=1e-6)
            assert np.all(r.centroids[c] == r.centroids[c].astype(np.float32))
    np.testing.assert_array_equal(r.counts, np.bincount(r.labels, minlength=9))
    # the objective never increases, neither in assign nor in update steps
    seq = []
    for a, u in zip(r.J_assign, r.J_update):
        seq += [a, u]
    assert all(seq[i + 1] <= seq[i] * (1 + 1e-9) for i in range(len(seq) - 1))
    # labels are the argmin over the centroids they were assigned against
    r1 = oracle.kmeans(X, 9, 1, seed=3)
    brute = np.argmin(((X[:, None, :] - r1.seed.centroids[None]) ** 2).sum(-1), axis=1)
    np.testing.assert_array_equal(r1.labels, brute)


def test_empty_cluster_keeps_previous_centroid():
    X = np.array([[0.0], [0.1], [5.0], [5.1]])
    C0 = np.array([[0.0], [5.0], [100.0]])
    r = oracle.kmeans(X, 3, 2, init=C0)
    assert r.counts.tolist() == [2, 2, 0]
    assert r.centroids[2, 0] == 100.0
    np.testing.assert_allclose(r.centroids[:2, 0], [0.05, 5.05], rtol=1e-7)


def test_warm_start_fixed_point():
    """Warm-starting from converged centroids of the same data changes nothing."""
    X = _blobs(11, N=500)
    conv = oracle.kmeans(X, 6, 60, seed=1)
    warm = oracle.kmeans(X, 6, 1, init=conv.centroids)
    np.testing.assert_array_equal(warm.labels, conv.labels)
    np.testing.assert_array_equal(warm.centroids, conv.centroids)
