"""fp64 CPU oracle of SVG2 semantic-aware-permutation sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
executes this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg do.  It shares no code with the HIP library (no headers,
helpers, tables or generated constants) and is written to be checked against
the pages by eye: plain numpy in float64, library primitives (matmul, exp,
stable sort, cumsum) as single steps, no blocking or fusion.

Sources.  "wiki" below is the page "Sparse VideoGen2: Accelerate Video
Generation with Sparse Attention via Semantic-Aware Permutation" (the
bud-325 paper-wiki summary), cited by its section and by the paper section,
equation or figure that the section names in brackets; "abstract" is the
arXiv abstract of the same paper.  The method, per head and layer:

  1. k-means over the Q tokens and, separately, the K tokens, seeded by
     k-means++ (cold) or by the previous step's centroids (warm)
     [wiki: Method, stage (1); Key claims, §4.1 and §4.3 / Fig. 7(a)];
  2. a permutation P_Q of the Q rows and a permutation P_K of the K rows and
     the V rows into contiguous cluster blocks [wiki: Method, stage (2)];
  3. centroid dot products as estimates of pre-softmax attention, weighted
     by cluster size, then top-p selection of K-clusters
     [wiki: Method, stage (3); Key claims, §4.2, Eq. 1, Eq. 2];
  4. block-sparse attention over the variable-sized blocks
     [wiki: Method, stage (4); Key claims, §4.3 / Fig. 7(b)];
  5. the inverse permutation of the output rows [wiki: Method, stage (2)].

Where the pages leave a step open the plainest reading is taken; each such
reading is named where it is used ("reading: ...").

Parity pins.  Every function here is pinned in tests/test_oracle_*.py to a
closed form, a library routine, an invariant, brute force on tiny inputs or a
published test vector.  The k-means++ sampler is pinned by distributional
(chi-square) and special-case checks only: for a random sampler no exact
expected value exists without running it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

# --------------------------------------------------------------------------
# Counter-based random numbers for k-means++ seeding.
# reading: the pages name k-means++ but no generator.  splitmix64 (Steele,
# Lea & Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014)
# is used as a counter-based generator: one output of a fresh state.
# --------------------------------------------------------------------------
_M64 = (1 << 64) - 1
_GOLDEN_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(state: int) -> int:
    """First output of a splitmix64 generator whose state is ``state``."""
    z = (state + _GOLDEN_GAMMA) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def seeding_uniform(seed: int, problem: int, pick: int) -> float:
    """u in [0, 1) for pick ``pick`` of problem ``problem``: the top 53 bits of
    splitmix64(seed XOR (problem * 2**32 + pick)), times 2**-53."""
    x = (seed ^ ((problem << 32) + pick)) & _M64
    return (splitmix64(x) >> 11) * (2.0 ** -53)


# --------------------------------------------------------------------------
# Step 1a: k-means++ seeding  [wiki: Method, stage (1)]
# Arthur & Vassilvitskii (2007): the first centre is a uniform data point,
# each further centre is a data point drawn with probability proportional to
# D^2(x), the squared distance to the nearest centre chosen so far.
# --------------------------------------------------------------------------
def sqdist_to(X: np.ndarray, c: np.ndarray) -> np.ndarray:
    """||x - c||^2 for every row x of X, as a sum of squared differences."""
    diff = X - c[None, :]
    return np.sum(diff * diff, axis=1)


@dataclass
class SeedResult:
    index: np.ndarray            # int64 [n]: token chosen by pick k
    centroids: np.ndarray        # fp64 [n, d]: X[index]
    margin: np.ndarray           # fp64 [n]: distance of the sampling target to the
                                 # nearest cumulative-sum boundary / total (inf for pick 0)


def kmeanspp(X: np.ndarray, n: int, seed: int, problem: int = 0) -> SeedResult:
    """k-means++ seeding of ``n`` centres from the rows of X (fp64 [N, d]).

    Pick 0 is token floor(u_0 N).  Pick k >= 1 is the smallest token t with
    sum_{s <= t} D2_s > u_k * sum_s D2_s, i.e. inverse-CDF sampling of the
    D^2 distribution (if rounding leaves no such t, the last token with
    D2 > 0); if every D2 is zero (fewer distinct rows than n) the pick falls
    back to floor(u_k N).
    """
    X = np.asarray(X, dtype=np.float64)
    N = X.shape[0]
    index = np.zeros(n, dtype=np.int64)
    margin = np.full(n, np.inf)
    index[0] = min(int(math.floor(seeding_uniform(seed, problem, 0) * N)), N - 1)
    D2 = sqdist_to(X, X[index[0]])
    for k in range(1, n):
        u = seeding_uniform(seed, problem, k)
        cs = np.cumsum(D2)
        total = cs[-1]
        if total <= 0.0:
            t = min(int(math.floor(u * N)), N - 1)
        else:
            target = u * total
            t = int(np.searchsorted(cs, target, side="right"))
            if t >= N:
                # u * total rounded up to the total: take the last token that
                # still has positive mass
                t = int(np.nonzero(D2 > 0)[0][-1])
            lo = cs[t - 1] if t > 0 else 0.0
            margin[k] = min(target - lo, cs[t] - target) / total
        index[k] = t
        D2 = np.minimum(D2, sqdist_to(X, X[t]))
    return SeedResult(index=index, centroids=X[index].copy(), margin=margin)


# --------------------------------------------------------------------------
# Steps 1b-1c: Lloyd iterations  [wiki: Method, stage (1); Key claims, §4.3]
# reading: squared Euclidean distance on the raw vectors; a fixed number T of
# (assign, update) rounds; labels are those of the T-th assignment and the
# centroids are the means of those labels; an empty cluster keeps its
# previous centroid; centroids are stored in fp32 (rounded after each update);
# exact ties go to the lowest centroid index.
# --------------------------------------------------------------------------
@dataclass
class AssignResult:
    labels: np.ndarray           # int64 [N]
    min_dist: np.ndarray         # fp64 [N]: ||x - c_label||^2
    margin: np.ndarray           # fp64 [N]: (d2 - d1) / (||x||^2 + ||c_label||^2)


def assign(X: np.ndarray, C: np.ndarray, chunk: int = 8192) -> AssignResult:
    """Nearest centroid of every row of X under ||x - c||^2 (ties: lowest c).

    Distances come from the expansion ||x||^2 - 2 x.c + ||c||^2 in fp64, whose
    rounding (~1e-16 of ||x||^2 + ||c||^2) is far below any tie band used.
    """
    X = np.asarray(X, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    N = X.shape[0]
    cn = np.sum(C * C, axis=1)
    labels = np.zeros(N, dtype=np.int64)
    best = np.zeros(N)
    margin = np.zeros(N)
    for s in range(0, N, chunk):
        x = X[s:s + chunk]
        xn = np.sum(x * x, axis=1)
        dist = xn[:, None] - 2.0 * (x @ C.T) + cn[None, :]
        lab = np.argmin(dist, axis=1)            # first minimum = lowest index
        d1 = dist[np.arange(len(x)), lab]
        if C.shape[0] > 1:
            part = np.partition(dist, 1, axis=1)
            d2 = part[:, 1]
        else:
            d2 = np.full(len(x), np.inf)
        labels[s:s + chunk] = lab
        best[s:s + chunk] = np.maximum(d1, 0.0)
        margin[s:s + chunk] = (d2 - d1) / (xn + cn[lab])
    return AssignResult(labels=labels, min_dist=best, margin=margin)


def update(X: np.ndarray, labels: np.ndarray, C_prev: np.ndarray,
           round_fp32: bool = True):
    """New centroids = mean of members; empty clusters keep C_prev.
    Returns (C_new fp64 [n, d], counts int64 [n])."""
    X = np.asarray(X, dtype=np.float64)
    n = C_prev.shape[0]
    counts = np.bincount(labels, minlength=n).astype(np.int64)
    sums = np.zeros((n, X.shape[1]))
    np.add.at(sums, labels, X)
    C = np.array(C_prev, dtype=np.float64, copy=True)
    nz = counts > 0
    C[nz] = sums[nz] / counts[nz, None]
    if round_fp32:
        C = C.astype(np.float32).astype(np.float64)
    return C, counts


def objective(X: np.ndarray, C: np.ndarray, labels: np.ndarray) -> float:
    """k-means objective J = sum_x ||x - c_label(x)||^2 (difference form)."""
    diff = np.asarray(X, dtype=np.float64) - np.asarray(C, dtype=np.float64)[labels]
    return float(np.sum(diff * diff))


@dataclass
class KMeansResult:
    centroids: np.ndarray        # fp64 [n, d] (fp32-valued when round_fp32)
    labels: np.ndarray           # int64 [N], from the last assignment
    counts: np.ndarray           # int64 [n]
    min_dist: np.ndarray         # fp64 [N] at the last assignment
    margins: List[np.ndarray] = field(default_factory=list)   # per iteration
    J_assign: List[float] = field(default_factory=list)       # J after assign t
    J_update: List[float] = field(default_factory=list)       # J after update t
    seed: Optional[SeedResult] = None


def kmeans(X: np.ndarray, n: int, iters: int, init: Optional[np.ndarray] = None,
           seed: int = 0, problem: int = 0, round_fp32: bool = True) -> KMeansResult:
    """k-means of the rows of X: k-means++ (``init`` None) or warm start from
    ``init`` [wiki: Method, stage (1)], then ``iters`` Lloyd rounds."""
    X = np.asarray(X, dtype=np.float64)
    sr = None
    if init is None:
        sr = kmeanspp(X, n, seed, problem)
        C = sr.centroids
    else:
        C = np.asarray(init, dtype=np.float64)
    if round_fp32:
        C = C.astype(np.float32).astype(np.float64)
    res = KMeansResult(centroids=C, labels=np.zeros(X.shape[0], np.int64),
                       counts=np.zeros(n, np.int64), min_dist=np.zeros(X.shape[0]), seed=sr)
    for _ in range(iters):
        a = assign(X, C)
        res.J_assign.append(objective(X, C, a.labels))
        C, counts = update(X, a.labels, C, round_fp32)
        res.J_update.append(objective(X, C, a.labels))
        res.margins.append(a.margin)
        res.labels, res.counts, res.min_dist = a.labels, counts, a.min_dist
    res.centroids = C
    return res


# --------------------------------------------------------------------------
# Step 2: semantic-aware permutation  [wiki: Method, stage (2); Key claims, §4.1]
# reading: clusters in ascending label order, tokens inside a cluster in
# ascending original index (a stable sort); P_Q from the Q labels permutes Q,
# P_K from the K labels permutes both K and V.
# --------------------------------------------------------------------------
def counting_sort(labels: np.ndarray, n: int):
    """Returns (perm, offsets, counts): perm[i] is the original token placed at
    sorted slot i; cluster c occupies slots [offsets[c], offsets[c+1])."""
    labels = np.asarray(labels, dtype=np.int64)
    perm = np.argsort(labels, kind="stable")
    counts = np.bincount(labels, minlength=n).astype(np.int64)
    offsets = np.zeros(n + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return perm, offsets, counts


def permute_rows(X: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """Row i of the result is row perm[i] of X."""
    return np.asarray(X)[np.asarray(perm)]


def unpermute_rows(Xp: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """Inverse of permute_rows: out[perm[i]] = Xp[i]."""
    out = np.empty_like(np.asarray(Xp))
    out[np.asarray(perm)] = Xp
    return out


# --------------------------------------------------------------------------
# Step 3: centroid-based estimation and top-p  [wiki: Method, stage (3);
# Key claims, §4.2, Eq. 1, Eq. 2].  The equations themselves are not printed
# on the pages.  reading: logit l_ij = s * cQ_i . cK_j with s = 1/sqrt(d);
# weight w_ij = |K_j| exp(l_ij - max_l l_il) over non-empty K-clusters;
# P_ij = w_ij / sum_l w_il (a per-Q-cluster distribution); sort descending
# (ties: lower j first), keep the shortest prefix whose cumulative sum
# reaches p; p >= 1 keeps every non-empty cluster; the list is emitted in
# ascending j.
# --------------------------------------------------------------------------
def centroid_probs(cq: np.ndarray, ck: np.ndarray, k_counts: np.ndarray,
                   scale: float) -> np.ndarray:
    """P [n_q, n_k] in fp64; zero for empty K-clusters."""
    cq = np.asarray(cq, dtype=np.float64)
    ck = np.asarray(ck, dtype=np.float64)
    k_counts = np.asarray(k_counts)
    logits = scale * (cq @ ck.T)
    nonempty = k_counts > 0
    P = np.zeros_like(logits)
    if not nonempty.any():
        return P
    m = np.max(logits[:, nonempty], axis=1, keepdims=True)
    w = np.where(nonempty[None, :], k_counts[None, :] * np.exp(logits - m), 0.0)
    return w / np.sum(w, axis=1, keepdims=True)


@dataclass
class Selection:
    lists: List[np.ndarray]      # per Q-cluster: selected K-clusters, ascending
    probs: np.ndarray            # fp64 [n_q, n_k]
    ambiguous: np.ndarray        # bool [n_q]: the cut lies within `band` of p,
                                 # or the order at the cut is within `band`


def select_topp(P: np.ndarray, k_counts: np.ndarray, top_p: float,
                band: float = 1e-12) -> Selection:
    P = np.asarray(P, dtype=np.float64)
    nonempty = np.asarray(k_counts) > 0
    n_q, n_k = P.shape
    lists, amb = [], np.zeros(n_q, dtype=bool)
    j = np.arange(n_k)
    for i in range(n_q):
        cand = j[nonempty]
        if len(cand) == 0:
            lists.append(np.zeros(0, np.int64))
            continue
        order = cand[np.lexsort((cand, -P[i, cand]))]     # -P first, then j
        if top_p >= 1.0:
            keep = len(order)
        else:
            cs = np.cumsum(P[i, order])
            reach = np.nonzero(cs >= top_p)[0]
            keep = int(reach[0]) + 1 if len(reach) else len(order)
            cut = keep - 1
            pv = P[i, order]
            near = abs(cs[cut] - top_p) < band
            if cut > 0:
                near |= abs(cs[cut - 1] - top_p) < band
            if cut + 1 < len(order):
                near |= abs(pv[cut] - pv[cut + 1]) < band * pv[0]
            amb[i] = near
        lists.append(np.sort(order[:keep]))
    return Selection(lists=lists, probs=P, ambiguous=amb)


def pair_count(lists, q_counts, k_counts) -> int:
    """sum_i sum_{j in S_i} |Q_i| |K_j|: (query, key) pairs the selection computes."""
    return int(sum(int(q_counts[i]) * int(np.sum(np.asarray(k_counts)[l]))
                   for i, l in enumerate(lists)))


# --------------------------------------------------------------------------
# Step 4: block-sparse attention  [wiki: Method, stage (4); Key claims, §4.1]
# reading: each query row of Q-cluster i attends to the union of the rows of
# its selected K-clusters with softmax(s q.k) renormalised over those keys
# only; a row with no selected key gives O = 0, LSE = -inf.
# --------------------------------------------------------------------------
def softmax_attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                           scale: float):
    """Plain softmax attention of the rows of q over (k, v).  Returns (O, lse)."""
    q = np.asarray(q, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros((q.shape[0], v.shape[1])), np.full(q.shape[0], -np.inf)
    s = scale * (q @ np.asarray(k, dtype=np.float64).T)
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    z = np.sum(e, axis=1, keepdims=True)
    out = (e @ np.asarray(v, dtype=np.float64)) / z
    return out, (m + np.log(z))[:, 0]


def block_attention(qp, kp, vp, q_offsets, k_offsets, lists, scale: float,
                    q_clusters=None):
    """Attention in permuted order: Q-cluster i (rows q_offsets[i]:q_offsets[i+1]
    of qp) over the concatenated key rows of its selected K-clusters.
    Returns (O' fp64 [N, d], lse fp64 [N]); ``q_clusters`` limits the work to
    those clusters (other rows are NaN)."""
    N, d = qp.shape[0], vp.shape[1]
    out = np.full((N, d), np.nan)
    lse = np.full(N, np.nan)
    ids = range(len(lists)) if q_clusters is None else q_clusters
    for i in ids:
        a, b = int(q_offsets[i]), int(q_offsets[i + 1])
        if a == b:
            continue
        rows = np.concatenate([np.arange(k_offsets[j], k_offsets[j + 1]) for j in lists[i]]) \
            if len(lists[i]) else np.zeros(0, np.int64)
        o, l = softmax_attention_rows(qp[a:b], kp[rows], vp[rows], scale)
        out[a:b], lse[a:b] = o, l
    return out, lse


def masked_dense_attention(q, k, v, zq, zk, lists, scale: float, rows=None):
    """The same attention written in the original token order: query t attends
    to the keys u whose K-label is selected by the Q-cluster of t.  Returns
    (O, lse) for ``rows`` (default: all tokens)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    zq, zk = np.asarray(zq), np.asarray(zk)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    n_k = int(max(zk.max() + 1, max((int(l.max()) + 1 for l in lists if len(l)), default=0)))
    selected = np.zeros((len(lists), n_k), dtype=bool)
    for i, l in enumerate(lists):
        selected[i, np.asarray(l, dtype=np.int64)] = True
    out = np.zeros((len(rows), v.shape[1]))
    lse = np.zeros(len(rows))
    for i in np.unique(zq[rows]):
        r = np.nonzero(zq[rows] == i)[0]
        mask = selected[int(i)][zk]
        o, l = softmax_attention_rows(q[rows[r]], k[mask], v[mask], scale)
        out[r], lse[r] = o, l
    return out, lse


# --------------------------------------------------------------------------
# Whole layer for one head: steps 1-5.
# --------------------------------------------------------------------------
@dataclass
class LayerResult:
    out: np.ndarray
    lse: np.ndarray
    km_q: KMeansResult
    km_k: KMeansResult
    perm_q: np.ndarray
    perm_k: np.ndarray
    q_offsets: np.ndarray
    k_offsets: np.ndarray
    selection: Selection
    pairs: int


def layer(q, k, v, n_q: int, n_k: int, iters: int, top_p: float,
          seed_q: int = 0, seed_k: int = 1, problem: int = 0,
          init_q=None, init_k=None, q_clusters=None) -> LayerResult:
    """One head of the layer: k-means on Q and K, permute, select, attend,
    un-permute.  ``q_clusters`` limits the attention to those Q-clusters
    (output rows of the others are NaN)."""
    d = np.asarray(q).shape[1]
    scale = 1.0 / math.sqrt(d)
    kq = kmeans(q, n_q, iters, init_q, seed_q, problem)
    kk = kmeans(k, n_k, iters, init_k, seed_k, problem)
    pq, qoff, _ = counting_sort(kq.labels, n_q)
    pk, koff, _ = counting_sort(kk.labels, n_k)
    P = centroid_probs(kq.centroids, kk.centroids, kk.counts, scale)
    sel = select_topp(P, kk.counts, top_p)
    op, lp = block_attention(permute_rows(q, pq), permute_rows(k, pk), permute_rows(v, pk),
                             qoff, koff, sel.lists, scale, q_clusters)
    return LayerResult(out=unpermute_rows(op, pq), lse=unpermute_rows(lp, pq), km_q=kq, km_k=kk,
                       perm_q=pq, perm_k=pk, q_offsets=qoff, k_offsets=koff, selection=sel,
                       pairs=pair_count(sel.lists, kq.counts, kk.counts))


def density(pairs_per_head, n_tokens: int) -> float:
    """Share of the N^2 (query, key) pairs per head that the selection computes."""
    return float(np.sum(pairs_per_head)) / (len(pairs_per_head) * float(n_tokens) ** 2)


# --------------------------------------------------------------------------
# Around the layer: one layer along a denoising run  [wiki: Method, stage (1)
# and its dense warm-up paragraph; Key claims, §4.3 / Fig. 7(a)]
# reading: "the first ~10% of steps run dense" = step s (0-based) is dense
# when s < fraction * steps, less a 1e-9 guard so that float rounding of the
# product never adds a step (5 of 50 steps, 1 of 10).  The first sparse step
# of a layer seeds with k-means++ and runs the cold rounds; every later step
# starts from the centroids the layer ended the previous step with (the
# centroid cache) and runs the warm rounds.  Dense steps leave the cache
# untouched.
# --------------------------------------------------------------------------
def is_dense_step(step: int, steps: int, fraction: float) -> bool:
    return step < fraction * steps - 1e-9


@dataclass
class DenoiseResult:
    outs: list        # per step: [N, d] output in the input's token order
    modes: list       # per step: "dense", "cold" or "warm"
    layers: list      # per step: LayerResult, or None on dense steps


def denoise_layer(steps_qkv, n_q: int, n_k: int, top_p, fraction: float, cold_iters: int, warm_iters: int,
                  seed_q: int = 0, seed_k: int = 1, problem: int = 0) -> DenoiseResult:
    """One head of one layer over the steps of a run; ``steps_qkv`` lists the
    (q, k, v) of every step and ``top_p`` is a number or a function of the step."""
    steps = len(steps_qkv)
    res = DenoiseResult(outs=[], modes=[], layers=[])
    cache = None
    for s, (q, k, v) in enumerate(steps_qkv):
        if is_dense_step(s, steps, fraction):
            d = np.asarray(q).shape[1]
            out, _ = softmax_attention_rows(q, k, v, 1.0 / math.sqrt(d))
            res.outs.append(out)
            res.modes.append("dense")
            res.layers.append(None)
            continue
        p = top_p(s) if callable(top_p) else top_p
        if cache is None:
            r = layer(q, k, v, n_q, n_k, cold_iters, p, seed_q, seed_k, problem)
            res.modes.append("cold")
        else:
            r = layer(q, k, v, n_q, n_k, warm_iters, p, seed_q, seed_k, problem,
                      init_q=cache[0], init_k=cache[1])
            res.modes.append("warm")
        cache = (r.km_q.centroids, r.km_k.centroids)
        res.outs.append(r.out)
        res.layers.append(r)
    return res


# --------------------------------------------------------------------------
# Identification accuracy, beside the path  [wiki: Key claims, §3.1 / Fig. 3;
# §3.2, Figs. 3-4; §5.3]
# reading: the recall of query row r under a selection is the share of r's
# exact softmax mass that falls on the keys the selection gives r,
#   sum_{u selected} exp(s_ru) / sum_u exp(s_ru),  s_ru = scale q_r . k_u.
# Position-based blocks: fixed blocks of `block` consecutive tokens of the
# original order (the last one may be shorter), each represented by the mean
# of its rows and scored and selected exactly as the semantic clusters are
# (the same size-weighted estimate and top-p).
# --------------------------------------------------------------------------
def position_blocks(n_tokens: int, block: int) -> np.ndarray:
    """Label of every token: its fixed block, t // block."""
    return np.arange(n_tokens) // block


def recall_rows(q, k, zq, zk, lists, scale: float) -> np.ndarray:
    """Per query row, the share of its softmax mass on its selected keys."""
    s = scale * (np.asarray(q, dtype=np.float64) @ np.asarray(k, dtype=np.float64).T)
    e = np.exp(s - np.max(s, axis=1, keepdims=True))
    total = np.sum(e, axis=1)
    rec = np.zeros(s.shape[0])
    for i, sel in enumerate(lists):
        rows = np.nonzero(zq == i)[0]
        if len(rows) == 0:
            continue
        keys = np.isin(zk, sel)
        rec[rows] = np.sum(e[np.ix_(rows, keys)], axis=1) / total[rows]
    return rec


@dataclass
class BlockSelection:
    zq: np.ndarray
    zk: np.ndarray
    selection: Selection
    pairs: int


def positional_selection(q, k, block: int, top_p: float) -> BlockSelection:
    """Fixed position-based blocks with mean-pooled representatives, scored
    and selected like the semantic clusters (fp32 means, as the GPU keeps)."""
    N, d = np.asarray(q).shape
    z = position_blocks(N, block)
    n = int(z[-1]) + 1
    cq, nq = update(q, z, np.zeros((n, d)))
    ck, nk = update(k, z, np.zeros((n, d)))
    sel = select_topp(centroid_probs(cq, ck, nk, 1.0 / math.sqrt(d)), nk, top_p)
    return BlockSelection(zq=z, zk=z, selection=sel, pairs=pair_count(sel.lists, nq, nk))


# --------------------------------------------------------------------------
# FP8 attention (the open-source plan's "Support FP8 attention" [README]).
# reading: the pages name FP8 but no format or scaling.  OCP FP8 E4M3 (1 sign,
# 4 exponent bits with bias 7, 3 mantissa bits, subnormals, largest finite
# value 448, no infinities) with one scale per problem and tensor:
# scale = max|x| / 448 for the dequantization, r = 448 / max|x| (both
# correctly rounded to fp32) and x8 = round-to-nearest-even(x * r) on the E4M3
# grid, the product taken in fp32 and clamped to +-448.
# --------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_grid() -> np.ndarray:
    """Every non-negative finite E4M3 value, ascending (code order)."""
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:          # the NaN code
                continue
            vals.append(m / 8.0 * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals)


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """x (|x| <= 448) to the nearest E4M3 value; ties go to the even code."""
    g = e4m3_grid()
    a = np.abs(np.asarray(x, dtype=np.float64))
    i = np.clip(np.searchsorted(g, a), 1, len(g) - 1)
    lo, hi = g[i - 1], g[i]
    pick_hi = (a - lo > hi - a) | ((a - lo == hi - a) & (i % 2 == 0))
    r = np.where(pick_hi, hi, lo)
    r = np.where(a <= 0.0, 0.0, r)
    return np.copysign(r, x)


def fp8_scale(x) -> float:
    """Per-tensor scale of one problem: max|x| / 448 in fp32 (1 if x is all zero)."""
    amax = float(np.max(np.abs(np.asarray(x, dtype=np.float64))))
    return float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0


def fp8_ratio(x) -> float:
    """Quantization factor of one problem: 448 / max|x| in fp32 (1 if all zero)."""
    amax = float(np.max(np.abs(np.asarray(x, dtype=np.float64))))
    return float(np.float32(E4M3_MAX / amax)) if amax > 0 else 1.0


def fp8_quantize(x) -> np.ndarray:
    """The E4M3 values of x * fp8_ratio(x) (the product taken in fp32)."""
    q = (np.asarray(x, dtype=np.float32) * np.float32(fp8_ratio(x))).astype(np.float64)
    return e4m3_round(np.clip(q, -E4M3_MAX, E4M3_MAX))
