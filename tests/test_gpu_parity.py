"""GPU parity: every HIP entry point against the fp64 oracle on the same
seeded inputs.  Inputs come from the generator and, for later stages, from
the oracle's own earlier stages, except where a stage is teacher-forced: the
centroid update is checked against the oracle's update of the GPU's own
labels, so that one near-tie token cannot skip the check.

Bars (the tolerances are fixed by the method's statement of the path):
  * integer / index outputs (labels, offsets, permutation, selections,
    k-means++ picks): bit-exact, except tokens / rows inside the stated
    tie bands, which must be rare;
  * bf16 attention: max-abs 2e-2 and relative-L2 1e-2; fp32: 1e-4 / 1e-4;
  * centroids: within 1e-5 * max(1, |c|).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from parity_checks import check_labels_in_tie_band
from sparse_attention_video_head_amd import binding as B
from sparse_attention_video_head_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype != torch.float64 else t.cpu().numpy()


def dtype_of(name):
    return torch.float32 if name == "f32" else torch.bfloat16


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def mixture(bh, N, d, comps, seed, dtype):
    """Clustered [bh, N, d] Q, K and N(0,1) V (seeded, numpy -> rounded)."""
    rng = np.random.default_rng(seed)
    qs, ks, vs = [], [], []
    for _ in range(bh):
        mu = rng.standard_normal((comps, d))
        z = rng.integers(0, comps, N)
        qs.append(mu[z] + 0.3 * rng.standard_normal((N, d)))
        ks.append(mu[z] + 0.3 * rng.standard_normal((N, d)))
        vs.append(rng.standard_normal((N, d)))
    f = lambda a: torch.from_numpy(np.stack(a)).to(dtype)
    return f(qs), f(ks), f(vs)


# ====================================================================== permute
@pytest.mark.parametrize("dt,d,N,n,skew,nt", [
    ("bf16", 128, 5000, 37, 0.0, 1), ("bf16", 128, 4097, 300, 1.2, 2), ("f32", 64, 2048, 5, 0.0, 2),
    ("bf16", 64, 1, 1, 0.0, 1), ("f32", 128, 777, 777, 0.0, 1), ("bf16", 128, 20000, 4096, 0.8, 2),
])
def test_permute_bit_exact(dt, d, N, n, skew, nt):
    bh = 3
    dtype = dtype_of(dt)
    labels = np.stack([synth.random_labels(N, n, seed=10 + h, skew=skew) for h in range(bh)])
    xs = [synth.uniform_rows(bh * N, d, seed=20 + t, dtype=dtype).reshape(bh, N, d) for t in range(nt)]
    outs, perm, off = B.permute(torch.from_numpy(labels).to(DEV), n, *[x.to(DEV) for x in xs])
    torch.cuda.synchronize()
    for h in range(bh):
        p_ref, o_ref, _ = oracle.counting_sort(labels[h], n)
        np.testing.assert_array_equal(perm[h].cpu().numpy(), p_ref)
        np.testing.assert_array_equal(off[h].cpu().numpy(), o_ref)
        for t in range(nt):
            assert torch.equal(outs[t][h].cpu(), xs[t][h][torch.from_numpy(p_ref)])


def test_permute_strided_bnhd_layout_and_unpermute():
    """A [B, N, H, d] source (model layout) gathered through strides; the
    un-permute scatters back into the same strided layout exactly."""
    Bsz, H, N, d, n = 2, 3, 1500, 128, 20
    x = synth.uniform_rows(Bsz * N * H, d, seed=5, dtype=torch.bfloat16).reshape(Bsz, N, H, d)
    labels = np.stack([synth.random_labels(N, n, seed=30 + p) for p in range(Bsz * H)])
    xv = x.to(DEV).transpose(1, 2)                      # [B, H, N, d] view, strided
    (xp,), perm, off = B.permute(torch.from_numpy(labels).to(DEV), n, xv)
    back = torch.zeros_like(x, device=DEV)
    B.unpermute(xp, perm, out=back.transpose(1, 2))
    torch.cuda.synchronize()
    xh = x.transpose(1, 2).reshape(Bsz * H, N, d)
    for p in range(Bsz * H):
        pr, _, _ = oracle.counting_sort(labels[p], n)
        assert torch.equal(xp[p].cpu(), xh[p][torch.from_numpy(pr)])
    assert torch.equal(back.cpu(), x)


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f32", 64), ("bf16", 64)])
def test_unpermute_bit_exact(dt, d):
    bh, N = 2, 3001
    src = synth.uniform_rows(bh * N, d, seed=7, dtype=dtype_of(dt)).reshape(bh, N, d)
    rng = np.random.default_rng(3)
    perm = np.stack([rng.permutation(N) for _ in range(bh)]).astype(np.int32)
    out = B.unpermute(src.to(DEV), torch.from_numpy(perm).to(DEV))
    torch.cuda.synchronize()
    for h in range(bh):
        ref = oracle.unpermute_rows(np64(src[h]), perm[h])
        np.testing.assert_array_equal(np64(out[h]), ref)


# ====================================================================== select
@pytest.mark.parametrize("n_q,n_k,d,top_p,spread", [
    (40, 250, 128, 0.9, 1.0), (17, 1000, 128, 0.8, 0.5), (8, 64, 64, 0.95, 1.5), (5, 1, 64, 0.5, 1.0),
    (12, 4096, 128, 0.9, 0.7), (9, 300, 128, 1.0, 1.0), (9, 300, 128, 1e-6, 1.0),
    # sort sizes: 128 entries (one thread each, a cross-wave stage) and 2048 (the shared-memory network)
    (6, 100, 64, 0.9, 1.0), (7, 1500, 128, 0.95, 0.8),
])
def test_select_topp_exact(n_q, n_k, d, top_p, spread):
    bh = 2
    cq = np.stack([synth.gaussian_centroids(n_q, d, seed=40 + h, spread=spread) for h in range(bh)])
    ck = np.stack([synth.gaussian_centroids(n_k, d, seed=50 + h, spread=spread) for h in range(bh)])
    rng = np.random.default_rng(6)
    kc = rng.integers(0, 200, (bh, n_k)).astype(np.int32)
    kc[:, 0] = np.maximum(kc[:, 0], 1)
    if n_k > 3:
        kc[:, 1] = 0                                       # an empty cluster
    qc = rng.integers(0, 300, (bh, n_q)).astype(np.int32)
    scale = 1.0 / math.sqrt(d)
    r = B.select_topp(torch.from_numpy(cq).to(DEV), torch.from_numpy(qc).to(DEV), torch.from_numpy(ck).to(DEV),
                      torch.from_numpy(kc).to(DEV), top_p, scale=scale, probs=True)
    torch.cuda.synchronize()
    p32 = float(np.float32(top_p))
    s32 = float(np.float32(scale))
    n_amb = 0
    for h in range(bh):
        P = oracle.centroid_probs(cq[h].astype(np.float64), ck[h].astype(np.float64), kc[h], s32)
        sel = oracle.select_topp(P, kc[h], p32, band=1e-10)
        np.testing.assert_allclose(r["probs"][h].cpu().numpy(), P, rtol=1e-6, atol=1e-30)
        cnt = r["sel_count"][h].cpu().numpy()
        idx = r["sel_idx"][h].cpu().numpy()
        pairs = 0
        for i in range(n_q):
            got = idx[i, :cnt[i]]
            pairs += int(qc[h, i]) * int(kc[h, got].sum())
            if sel.ambiguous[i]:
                n_amb += 1
                continue
            np.testing.assert_array_equal(got, sel.lists[i], err_msg=f"head {h} row {i}")
        assert int(r["pair_count"][h]) == pairs
    assert n_amb <= max(1, bh * n_q // 1000)


# ====================================================================== attention
def _attn_case(dt, d, bh, N, n_q, n_k, top_p, seed, empty_rows=False):
    dtype = dtype_of(dt)
    q, k, v = mixture(bh, N, d, comps=max(4, n_k // 3), seed=seed, dtype=dtype)
    qo, ko, cnt, idx, lists = [], [], [], [], []
    for h in range(bh):
        lq = synth.random_labels(N, n_q, seed=seed * 7 + h, skew=0.7)
        lk = synth.random_labels(N, n_k, seed=seed * 11 + h, skew=0.9)
        _, oq, cq_ = oracle.counting_sort(lq, n_q)
        _, okk, ck_ = oracle.counting_sort(lk, n_k)
        P = oracle.centroid_probs(synth.gaussian_centroids(n_q, d, seed + h), synth.gaussian_centroids(n_k, d, seed + 99 + h),
                                  ck_, 1 / math.sqrt(d))
        sel = oracle.select_topp(P, ck_, top_p)
        ls = [l.copy() for l in sel.lists]
        if empty_rows:
            ls[0] = np.zeros(0, np.int64)
        row_idx = np.zeros((n_q, n_k), np.int32)
        for i, l in enumerate(ls):
            row_idx[i, :len(l)] = l
        qo.append(oq); ko.append(okk); idx.append(row_idx); lists.append(ls)
        cnt.append([len(l) for l in ls])
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).to(DEV)
    return q, k, v, t(qo), t(ko), t(cnt), t(idx), lists, np.array(qo), np.array(ko)


@pytest.mark.parametrize("dt,d,N,n_q,n_k,top_p", [
    ("bf16", 128, 3000, 20, 50, 0.9), ("bf16", 128, 4099, 7, 130, 0.6), ("bf16", 64, 2500, 30, 40, 0.95),
    ("f32", 64, 2000, 16, 32, 0.9), ("f32", 128, 1500, 9, 25, 0.7), ("bf16", 128, 700, 1, 1, 1.0),
    # many Q-clusters: the plan's longest-first sort over more than 1024 clusters, and at the limit
    ("bf16", 64, 6000, 1500, 200, 0.8), ("bf16", 128, 8192, 4096, 300, 0.9),
])
def test_varblock_attn_vs_oracle(dt, d, N, n_q, n_k, top_p):
    bh = 2
    q, k, v, qo, ko, cnt, idx, lists, qo_np, ko_np = _attn_case(dt, d, bh, N, n_q, n_k, top_p, seed=N + n_q,
                                                               empty_rows=(dt == "bf16" and n_q > 1))
    out, lse = B.varblock_attn(q.to(DEV), k.to(DEV), v.to(DEV), qo, ko, cnt, idx, lse=True)
    torch.cuda.synchronize()
    tol = (2e-2, 1e-2) if dt == "bf16" else (1e-4, 1e-4)
    s = 1 / math.sqrt(d)
    for h in range(bh):
        ref, ref_lse = oracle.block_attention(np64(q[h]), np64(k[h]), np64(v[h]), qo_np[h], ko_np[h], lists[h], s)
        got = np64(out[h])
        assert np.max(np.abs(got - ref)) <= tol[0]
        assert rel_l2(got, ref) <= tol[1]
        gl = lse[h].cpu().numpy().astype(np.float64)
        fin = np.isfinite(ref_lse)
        # bf16: the kernel's normaliser is the sum of the bf16-rounded
        # probabilities that weight V (each within 2^-9 relative of the exact
        # one), so log(sum) may move by up to 2^-9 = 1.95e-3 from the oracle's,
        # plus fp32 rounding of the scores and the sum
        np.testing.assert_allclose(gl[fin], ref_lse[fin], rtol=0, atol=2.5e-3 if dt == "bf16" else 1e-4)
        assert np.all(gl[~fin] == -np.inf) and np.all(got[~fin] == 0)


@pytest.mark.parametrize("boost", [1.0, 4.0, 12.0])
def test_varblock_attn_reference_modes_vs_oracle(boost):
    """The bf16 kernel fixes a query's softmax reference at the Cauchy-Schwarz
    bound of its scores when that bound is small for its whole wave (32 rows),
    and tracks the running maximum otherwise.  In every Q-cluster the rows of
    every other 32-row block are multiplied by `boost` (the products, rounded
    to bf16, are the inputs of both sides), so that with boost > 1 the waves of
    one work-group run both modes, and with 12 the large scores also meet the
    lazy rescale; each must match the oracle."""
    bh, N, d, n_q, n_k = 2, 3000, 128, 24, 60
    q, k, v, qo, ko, cnt, idx, lists, qo_np, ko_np = _attn_case("bf16", d, bh, N, n_q, n_k, 0.9, seed=404)
    qf = q.float()
    for h in range(bh):
        for i in range(n_q):
            a, b = int(qo_np[h][i]), int(qo_np[h][i + 1])
            for r0 in range(a + 32, b, 64):
                qf[h, r0:min(r0 + 32, b)] *= boost
    q = qf.to(torch.bfloat16)
    out, lse = B.varblock_attn(q.to(DEV), k.to(DEV), v.to(DEV), qo, ko, cnt, idx, lse=True)
    torch.cuda.synchronize()
    s = 1 / math.sqrt(d)
    for h in range(bh):
        ref, ref_lse = oracle.block_attention(np64(q[h]), np64(k[h]), np64(v[h]), qo_np[h], ko_np[h], lists[h], s)
        got = np64(out[h])
        assert np.max(np.abs(got - ref)) <= 2e-2
        assert rel_l2(got, ref) <= 1e-2
        gl = lse[h].cpu().numpy().astype(np.float64)
        fin = np.isfinite(ref_lse)
        # the bf16 normaliser bound of test_varblock_attn_vs_oracle, plus the
        # fp32 rounding of the scores, which grows with their size (scores of
        # ~200 here at boost 12): 3e-5 relative
        np.testing.assert_allclose(gl[fin], ref_lse[fin], rtol=3e-5, atol=2.5e-3)


@pytest.mark.parametrize("dt,d,layout", [("bf16", 128, "contiguous"), ("bf16", 128, "bnhd"), ("f32", 64, "bnhd"),
                                         ("bf16", 64, "contiguous")])
def test_varblock_attn_unpermute_vs_oracle(dt, d, layout):
    """The fused call writes row i of the attention to token perm[i] (and its
    lse there): against the oracle's block attention scattered the same way,
    and bit-identical to the attention followed by the separate un-permute."""
    Bsz, H, N, n_q, n_k = 2, 2, 2100, 15, 40
    bh = Bsz * H
    q, k, v, qo, ko, cnt, idx, lists, qo_np, ko_np = _attn_case(dt, d, bh, N, n_q, n_k, 0.85, seed=404,
                                                               empty_rows=True)
    rng = np.random.default_rng(9)
    perm_np = np.stack([rng.permutation(N) for _ in range(bh)]).astype(np.int32)
    perm = torch.from_numpy(perm_np).to(DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    if layout == "bnhd":
        buf = torch.full((Bsz, N, H, d), 7.0, dtype=qd.dtype, device=DEV)
        out, lse = B.varblock_attn_unpermute(qd, kd, vd, qo, ko, cnt, idx, perm, lse=True, out=buf.transpose(1, 2))
        got_all = buf.transpose(1, 2).reshape(bh, N, d)
    else:
        out, lse = B.varblock_attn_unpermute(qd, kd, vd, qo, ko, cnt, idx, perm, lse=True)
        got_all = out
    sep, sep_lse = B.varblock_attn(qd, kd, vd, qo, ko, cnt, idx, lse=True)
    back = B.unpermute(sep, perm)
    torch.cuda.synchronize()
    assert torch.equal(got_all.contiguous(), back)
    tol = (2e-2, 1e-2) if dt == "bf16" else (1e-4, 1e-4)
    s = 1 / math.sqrt(d)
    for h in range(bh):
        ref, ref_lse = oracle.block_attention(np64(q[h]), np64(k[h]), np64(v[h]), qo_np[h], ko_np[h], lists[h], s)
        exp = np.empty_like(ref)
        exp[perm_np[h]] = ref
        exp_lse = np.empty_like(ref_lse)
        exp_lse[perm_np[h]] = ref_lse
        got = np64(got_all[h])
        assert np.max(np.abs(got - exp)) <= tol[0]
        assert rel_l2(got, exp) <= tol[1]
        gl = lse[h].cpu().numpy().astype(np.float64)
        fin = np.isfinite(exp_lse)
        np.testing.assert_allclose(gl[fin], exp_lse[fin], rtol=0, atol=2.5e-3 if dt == "bf16" else 1e-4)
        assert np.all(gl[~fin] == -np.inf)
        np.testing.assert_array_equal(gl, sep_lse[h].cpu().numpy()[np.argsort(perm_np[h])])


def test_varblock_attn_dense_equals_softmax_attention():
    """n_q = n_k = 1 with every key selected is plain softmax attention."""
    bh, N, d = 2, 1100, 128
    q, k, v = mixture(bh, N, d, 10, seed=3, dtype=torch.bfloat16)
    off = torch.tensor([[0, N]] * bh, dtype=torch.int32, device=DEV)
    out, _ = B.varblock_attn(q.to(DEV), k.to(DEV), v.to(DEV), off, off,
                             torch.ones(bh, 1, dtype=torch.int32, device=DEV),
                             torch.zeros(bh, 1, 1, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    for h in range(bh):
        ref, _ = oracle.softmax_attention_rows(np64(q[h]), np64(k[h]), np64(v[h]), 1 / math.sqrt(d))
        assert np.max(np.abs(np64(out[h]) - ref)) <= 2e-2
        assert rel_l2(np64(out[h]), ref) <= 1e-2


def test_varblock_attn_deterministic():
    q, k, v, qo, ko, cnt, idx, *_ = _attn_case("bf16", 128, 2, 3000, 20, 50, 0.9, seed=77)
    a, _ = B.varblock_attn(q.to(DEV), k.to(DEV), v.to(DEV), qo, ko, cnt, idx)
    b, _ = B.varblock_attn(q.to(DEV), k.to(DEV), v.to(DEV), qo, ko, cnt, idx)
    assert torch.equal(a, b)


# ====================================================================== k-means
@pytest.mark.parametrize("dt,d,N,n", [("bf16", 128, 6000, 50), ("bf16", 64, 3000, 17), ("f32", 64, 4096, 64),
                                      ("bf16", 128, 2000, 1)])
def test_kmeans_one_round_vs_oracle(dt, d, N, n):
    """One Lloyd round from the same initial centroids: labels outside the
    tie band, counts and centroids."""
    bh = 2
    q, _, _ = mixture(bh, N, d, comps=max(2, n // 2), seed=N + n, dtype=dtype_of(dt))
    init = np.stack([np64(q[h])[np.random.default_rng(h).choice(N, n, replace=False)] for h in range(bh)])
    init = init + 0.01 * np.random.default_rng(9).standard_normal(init.shape)
    init32 = init.astype(np.float32)
    r = B.kmeans(q.to(DEV), n, 1, init=torch.from_numpy(init32).to(DEV), min_dist=True)
    torch.cuda.synchronize()
    for h in range(bh):
        X = np64(q[h])
        C0 = init32[h].astype(np.float64)
        a = oracle.assign(X, C0)
        lab = r["labels"][h].cpu().numpy()
        check_labels_in_tie_band(X, C0, lab, a, max_share=1e-3 + 1.0 / N)
        np.testing.assert_array_equal(r["counts"][h].cpu().numpy(), np.bincount(lab, minlength=n))
        np.testing.assert_allclose(r["min_dist"][h].cpu().numpy(), a.min_dist, rtol=1e-4, atol=1e-3)
        # the update teacher-forced with the GPU's labels: every centroid
        C, _ = oracle.update(X, lab.astype(np.int64), C0)
        got = r["centroids"][h].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - C) <= 1e-5 * np.maximum(1.0, np.abs(C)))


@pytest.mark.parametrize("d", [128, 64])
def test_assign_near_ties_decided_exactly(d):
    """Centroids built to put many tokens at near ties: an exact duplicate
    (ties go to the lower index), a copy moved by ~1e-6 relative (margins far
    inside the matrix-core error bound, decided again in fp64), and a group of
    20 copies moved by ~1e-7 (more near candidates than the per-token list
    holds: every centroid is then evaluated in fp64).  Labels must equal the
    oracle's for every token outside a 1e-12 relative band, min-distances
    within fp32 rounding of the oracle's."""
    bh, N, n = 2, 4000, 64
    q, _, _ = mixture(bh, N, d, comps=24, seed=17 + d, dtype=torch.bfloat16)
    rng = np.random.default_rng(d)
    init = np.stack([np64(q[h])[rng.choice(N, n, replace=False)] for h in range(bh)])
    init = init + 0.05 * rng.standard_normal(init.shape)
    init[:, 1] = init[:, 0]
    init[:, 2] = init[:, 3] * (1 + 1e-6 * rng.standard_normal((bh, d)))
    init[:, 10:30] = init[:, 9:10] * (1 + 1e-7 * rng.standard_normal((bh, 20, d)))
    init32 = init.astype(np.float32)
    r = B.kmeans(q.to(DEV), n, 1, init=torch.from_numpy(init32).to(DEV), min_dist=True)
    torch.cuda.synchronize()
    for h in range(bh):
        X = np64(q[h])
        C0 = init32[h].astype(np.float64)
        a = oracle.assign(X, C0)
        lab = r["labels"][h].cpu().numpy()
        near = a.margin < 1e-5
        print(f"head {h}: {int(near.sum())} tokens with margin < 1e-5", flush=True)
        assert near.sum() >= 50                          # the case exercises the near-tie pass
        check_labels_in_tie_band(X, C0, lab, a, max_share=0.5)
        assert not np.any(lab == 1)                      # the duplicate of centroid 0 never wins
        np.testing.assert_array_equal(r["counts"][h].cpu().numpy(), np.bincount(lab, minlength=n))
        np.testing.assert_allclose(r["min_dist"][h].cpu().numpy(), a.min_dist, rtol=1e-4, atol=1e-3)


def test_kmeans_chained_rounds_equal_one_call():
    """T chained one-round calls equal one T-round call, bit for bit."""
    bh, N, d, n = 2, 5000, 128, 40
    q, _, _ = mixture(bh, N, d, comps=30, seed=5, dtype=torch.bfloat16)
    qd = q.to(DEV)
    one = B.kmeans(qd, n, 3, seed=11)
    c = B.kmeans(qd, n, 0, seed=11)["centroids"].clone()
    for _ in range(3):
        step = B.kmeans(qd, n, 1, init=c)
        c = step["centroids"].clone()
    torch.cuda.synchronize()
    assert torch.equal(one["centroids"], c)
    assert torch.equal(one["labels"], step["labels"])
    assert torch.equal(one["counts"], step["counts"])


@pytest.mark.parametrize("dt,d,N,n,iters,warm,with_y", [
    ("bf16", 128, 5000, 40, 3, False, True), ("bf16", 128, 3001, 37, 1, True, True),
    ("bf16", 128, 3001, 37, 1, False, True),
    ("bf16", 64, 2000, 17, 2, False, False), ("f32", 64, 4097, 64, 2, True, True),
    ("bf16", 128, 700, 700, 1, False, True), ("bf16", 128, 1000, 1, 2, True, False),
])
def test_kmeans_permute_equals_kmeans_then_permute(dt, d, N, n, iters, warm, with_y):
    """The permutation fused into the last Lloyd round gives, bit for bit, what
    k-means followed by the stand-alone permutation gives; perm / offsets are the
    oracle's counting sort of the returned labels and the rows follow them."""
    bh = 3
    q, k, v = mixture(bh, N, d, comps=max(2, n // 2), seed=N + n, dtype=dtype_of(dt))
    xd, yd = k.to(DEV), v.to(DEV)
    init = B.kmeans(xd, n, 0, seed=5)["centroids"].clone() if warm else None
    ref = B.kmeans(xd, n, iters, init=init, seed=3)
    (rx, *ry), rperm, roff = B.permute(ref["labels"], n, xd, *([yd] if with_y else []))
    got = B.kmeans_permute(xd, n, iters, y=yd if with_y else None, init=init, seed=3)
    torch.cuda.synchronize()
    for key in ("centroids", "labels", "counts"):
        assert torch.equal(got[key], ref[key]), key
    assert torch.equal(got["perm"], rperm) and torch.equal(got["offsets"], roff)
    assert torch.equal(got["x_perm"], rx)
    if with_y:
        assert torch.equal(got["y_perm"], ry[0])
    else:
        assert got["y_perm"] is None
    lab = got["labels"].cpu().numpy()
    for h in range(bh):
        p_ref, o_ref, _ = oracle.counting_sort(lab[h], n)
        np.testing.assert_array_equal(got["perm"][h].cpu().numpy(), p_ref)
        np.testing.assert_array_equal(got["offsets"][h].cpu().numpy(), o_ref)
        idx = torch.from_numpy(p_ref)
        assert torch.equal(got["x_perm"][h].cpu(), k[h][idx])
        if with_y:
            assert torch.equal(got["y_perm"][h].cpu(), v[h][idx])


@pytest.mark.parametrize("d,N,n,iters,with_y", [(128, 5000, 40, 2, True), (128, 3001, 37, 1, False),
                                               (64, 2000, 17, 2, True)])
def test_kmeans_permute_fp8_equals_quantized_rows(d, N, n, iters, with_y):
    """E4M3 rows stored by the last Lloyd round equal, byte for byte, the
    quantization of the bf16 rows the same call gives without fp8, and the
    scales are the quantization's; clusters, perm and offsets are unchanged."""
    bh = 3
    q, k, v = mixture(bh, N, d, comps=max(2, n // 2), seed=7 * N + n, dtype=torch.bfloat16)
    # one all-zero problem of V: scale 1, zero bytes
    v[1] = 0
    xd, yd = k.to(DEV), v.to(DEV)
    ref = B.kmeans_permute(xd, n, iters, y=yd if with_y else None, seed=9)
    got = B.kmeans_permute(xd, n, iters, y=yd if with_y else None, seed=9, fp8=True)
    torch.cuda.synchronize()
    for key in ("centroids", "labels", "counts", "perm", "offsets"):
        assert torch.equal(got[key], ref[key]), key
    pairs = [("x_perm", "x_scale")] + ([("y_perm", "y_scale")] if with_y else [])
    for rows, sc in pairs:
        x8, s8 = B.quantize_fp8(ref[rows])
        torch.cuda.synchronize()
        assert got[rows].dtype == torch.uint8 and torch.equal(got[rows], x8), rows
        assert torch.equal(got[sc], s8), sc
    if with_y:
        assert float(got["y_scale"][1]) == 1.0 and int(got["y_perm"][1].abs().sum()) == 0
    else:
        assert got["y_perm"] is None and got["y_scale"] is None


@pytest.mark.parametrize("dt,d,N,n", [("bf16", 128, 6000, 50), ("f32", 64, 4096, 64), ("bf16", 64, 3001, 37),
                                      ("bf16", 128, 2000, 1)])
def test_first_round_after_seeding_vs_oracle(dt, d, N, n):
    """After k-means++ the first round's labels are the seeding's nearest picks
    (no assignment runs); asked for min_dist, the same round runs the
    assignment.  Both must equal the oracle's assignment of the tokens to the
    picked rows outside the tie band, and equal each other bit for bit."""
    bh = 2
    q, _, _ = mixture(bh, N, d, comps=max(4, n // 2), seed=3 * N + n, dtype=dtype_of(dt))
    seed = 0x5EED + n
    qd = q.to(DEV)
    fast = B.kmeans(qd, n, 1, seed=seed, seed_index=True)
    full = B.kmeans(qd, n, 1, seed=seed, seed_index=True, min_dist=True)
    torch.cuda.synchronize()
    assert torch.equal(fast["seed_index"], full["seed_index"])
    for h in range(bh):
        X = np64(q[h])
        C0 = X[fast["seed_index"][h].cpu().numpy()]
        a = oracle.assign(X, C0)
        for r in (fast, full):
            lab = r["labels"][h].cpu().numpy()
            check_labels_in_tie_band(X, C0, lab, a, max_share=1e-3 + 1.0 / N)
            np.testing.assert_array_equal(r["counts"][h].cpu().numpy(), np.bincount(lab, minlength=n))
        np.testing.assert_allclose(full["min_dist"][h].cpu().numpy(), a.min_dist, rtol=1e-4, atol=1e-3)
    assert torch.equal(fast["labels"], full["labels"])
    assert torch.equal(fast["counts"], full["counts"])
    assert torch.equal(fast["centroids"], full["centroids"])


@pytest.mark.parametrize("dt,d,N,n,heads", [("f32", 64, 4096, 64, 1), ("bf16", 128, 16384, 250, 2),
                                           ("bf16", 128, 3000, 100, 2), ("bf16", 64, 700, 700, 1)])
def test_kmeanspp_picks_match_oracle(dt, d, N, n, heads):
    q, _, _ = mixture(heads, N, d, comps=max(8, n // 2), seed=n, dtype=dtype_of(dt))
    seed = 0xABCDEF12345 + n
    r = B.kmeans(q.to(DEV), n, 0, seed=seed, seed_index=True)
    torch.cuda.synchronize()
    for h in range(heads):
        X = np64(q[h])
        ref = oracle.kmeanspp(X, n, seed, problem=h)
        got = r["seed_index"][h].cpu().numpy()
        amb = np.nonzero(ref.margin < 1e-10)[0]
        upto = int(amb[0]) if len(amb) else n
        np.testing.assert_array_equal(got[:upto], ref.index[:upto])
        assert upto >= n // 2
        np.testing.assert_array_equal(r["centroids"][h].cpu().numpy()[:upto].astype(np.float64), X[got[:upto]])


# ====================================================================== whole layer
def test_layer_tiny_config_end_to_end():
    """The tiny fp32 config: the whole GPU layer (cold k-means++, 5 rounds,
    permute, top-p 0.9, attention, un-permute) against the oracle layer."""
    from sparse_attention_video_head_amd.pipeline import SVG2Layer
    cfg = synth.CONFIGS["tiny"]
    data = synth.make_layer(cfg)
    layer = SVG2Layer(cfg.bh, cfg.n_tokens, cfg.head_dim, cfg.torch_dtype, cfg.n_q, cfg.n_k)
    top_p = cfg.top_p[0]
    out = layer.run(data["q"].to(DEV), data["k"].to(DEV), data["v"].to(DEV), top_p, iters=cfg.iters,
                    seed_q=100, seed_k=200)
    torch.cuda.synchronize()
    q, k, v = (np64(data[x][0]) for x in "qkv")
    ref = oracle.layer(q, k, v, cfg.n_q, cfg.n_k, cfg.iters, float(np.float32(top_p)), seed_q=100, seed_k=200)
    agree_q = np.mean(layer.labels_q[0].cpu().numpy() == ref.km_q.labels)
    agree_k = np.mean(layer.labels_k[0].cpu().numpy() == ref.km_k.labels)
    assert agree_q >= 0.999 and agree_k >= 0.999
    got = np64(out[0])
    assert rel_l2(got, ref.out) <= 1e-4
    assert np.max(np.abs(got - ref.out)) <= 1e-3
    assert int(layer.pairs[0]) == ref.pairs


def test_layer_small_bf16_untethered_vs_oracle():
    """The small bf16 config (4 heads x 16,384 tokens, d = 128, 100 / 250
    clusters, 5 rounds, top-p 0.9), whole layer on the GPU from the same seeds
    as the oracle's layer, with nothing passed between them.  Reports the label
    agreement of both sides and the output's error against the oracle per head;
    the bars allow the few tokens a near tie sends elsewhere."""
    from sparse_attention_video_head_amd.pipeline import SVG2Layer
    cfg = synth.CONFIGS["small"]
    data = synth.make_layer(cfg)
    layer = SVG2Layer(cfg.bh, cfg.n_tokens, cfg.head_dim, torch.bfloat16, cfg.n_q, cfg.n_k)
    top_p = cfg.top_p[0]
    out = layer.run(data["q"].to(DEV), data["k"].to(DEV), data["v"].to(DEV), top_p, iters=cfg.iters,
                    seed_q=100, seed_k=200)
    torch.cuda.synchronize()
    for h in range(cfg.bh):
        q, k, v = (np64(data[x][h]) for x in "qkv")
        ref = oracle.layer(q, k, v, cfg.n_q, cfg.n_k, cfg.iters, float(np.float32(top_p)), seed_q=100,
                           seed_k=200, problem=h)
        agree_q = float(np.mean(layer.labels_q[h].cpu().numpy() == ref.km_q.labels))
        agree_k = float(np.mean(layer.labels_k[h].cpu().numpy() == ref.km_k.labels))
        got = np64(out[h])
        err = rel_l2(got, ref.out)
        mx = float(np.max(np.abs(got - ref.out)))
        print(f"head {h}: label agreement Q {agree_q:.5f} K {agree_k:.5f}; output rel-L2 {err:.3e} "
              f"max-abs {mx:.3e}; pairs {int(layer.pairs[h])} vs {ref.pairs}", flush=True)
        assert agree_q >= 0.99 and agree_k >= 0.99
        assert err <= 2e-2


# ====================================================================== denoising run
def test_denoise_driver_vs_oracle():
    """The driver along a drifting tiny-config sequence (fp32): one dense step,
    then a cold step and warm steps from the centroid cache, each step against
    the oracle's reference run of the same layer."""
    from sparse_attention_video_head_amd.driver import DenoiseDriver
    cfg = synth.CONFIGS["tiny"]
    steps, frac, top_p = 5, 0.2, 0.9
    seq = list(synth.denoise_sequence(cfg, heads=[0], steps=steps))
    drv = DenoiseDriver(1, cfg.n_tokens, cfg.head_dim, torch.float32, cfg.n_q, cfg.n_k, steps, top_p=top_p,
                        dense_fraction=frac, cold_iters=cfg.iters, warm_iters=2, seed=3, device=DEV)
    seed_q, seed_k = drv.seeds(0)
    ref = oracle.denoise_layer([tuple(np64(x[c][0]) for c in "qkv") for x in seq], cfg.n_q, cfg.n_k,
                               float(np.float32(top_p)), frac, cfg.iters, 2, seed_q, seed_k, problem=0)
    assert ref.modes == ["dense", "cold", "warm", "warm", "warm"]
    for s, x in enumerate(seq):
        out = drv(0, s, *(x[c].to(DEV) for c in "qkv")).clone()
        torch.cuda.synchronize()
        assert drv.last_mode == ref.modes[s], f"step {s}"
        got = np64(out[0])
        assert rel_l2(got, ref.outs[s]) <= 1e-4, f"step {s}"
        assert np.max(np.abs(got - ref.outs[s])) <= 1e-3, f"step {s}"
        if ref.layers[s] is not None:
            assert np.mean(drv.engine.labels_q[0].cpu().numpy() == ref.layers[s].km_q.labels) >= 0.999
            assert np.mean(drv.engine.labels_k[0].cpu().numpy() == ref.layers[s].km_k.labels) >= 0.999


def test_denoise_driver_layers_keep_separate_caches():
    """Two layers interleaved step by step give the same outputs as two
    drivers that each see one layer."""
    from sparse_attention_video_head_amd.driver import DenoiseDriver
    cfg = synth.CONFIGS["tiny"]
    steps = 4
    seqs = [list(synth.denoise_sequence(cfg, heads=[h], steps=steps)) for h in (0, 1)]
    mk = lambda: DenoiseDriver(1, cfg.n_tokens, cfg.head_dim, torch.float32, cfg.n_q, cfg.n_k, steps,
                               top_p=0.9, dense_fraction=0.25, cold_iters=3, warm_iters=2, seed=1, device=DEV)
    both, single = mk(), [mk(), mk()]
    for s in range(steps):
        for layer in (0, 1):
            x = [seqs[layer][s][c].to(DEV) for c in "qkv"]
            a = both(layer, s, *x).clone()
            b = single[layer](layer, s, *x).clone()
            torch.cuda.synchronize()
            assert torch.equal(a, b), f"layer {layer} step {s}"
    assert sorted(both.cache) == [0, 1]


# ====================================================================== identification study
@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f32", 64)])
def test_cluster_means_vs_oracle(dt, d):
    bh, N, n = 2, 3000, 37
    x, _, _ = mixture(bh, N, d, comps=10, seed=21, dtype=dtype_of(dt))
    rng = np.random.default_rng(4)
    lab = rng.integers(0, n, (bh, N)).astype(np.int32)
    lab[lab == 5] = 6                                   # label 5 has no row
    prev = torch.full((bh, n, d), 7.0, dtype=torch.float32, device=DEV)
    means, counts = B.cluster_means(x.to(DEV), torch.from_numpy(lab).to(DEV), n, means=prev)
    torch.cuda.synchronize()
    for h in range(bh):
        C, cnt = oracle.update(np64(x[h]), lab[h].astype(np.int64), np.full((n, d), 7.0))
        np.testing.assert_array_equal(counts[h].cpu().numpy(), cnt)
        got = means[h].cpu().numpy().astype(np.float64)
        assert np.all(np.abs(got - C) <= 1e-6 * np.maximum(1.0, np.abs(C)))
        assert np.all(got[5] == 7.0)


def test_recall_mass_vs_definition():
    rng = np.random.default_rng(8)
    bh, N = 3, 5000
    a = rng.standard_normal((bh, N))
    b = a + np.abs(rng.standard_normal((bh, N)))        # lse over all keys >= over the selected ones
    a[0, :10] = -np.inf                                  # rows that keep nothing
    b[1, :7] = -np.inf                                   # rows with no key: skipped
    a[1, :7] = -np.inf
    a32, b32 = a.astype(np.float32), b.astype(np.float32)
    got = B.recall_mass(torch.from_numpy(a32).to(DEV), torch.from_numpy(b32).to(DEV)).cpu().numpy()
    for h in range(bh):
        ok = np.isfinite(b32[h])
        expect = np.mean(np.exp(a32[h][ok].astype(np.float64) - b32[h][ok].astype(np.float64)))
        assert abs(got[h] - expect) <= 1e-12 * max(1.0, expect)


def test_identification_study_vs_oracle():
    """Tiny fp32 config: mean recall of the semantic path and of fixed
    128-token blocks at p = 0.9 against the oracle's definitions."""
    from sparse_attention_video_head_amd.study import IdentificationStudy
    cfg = synth.CONFIGS["tiny"]
    data = synth.make_layer(cfg)
    q, k, v = (data[c].to(DEV) for c in "qkv")
    st = IdentificationStudy(cfg.bh, cfg.n_tokens, cfg.head_dim, torch.float32, cfg.n_q, cfg.n_k, block=128)
    p = 0.9
    sem = st.semantic(q, k, v, [p], iters=cfg.iters, seed_q=100, seed_k=200)[0]
    pos = st.positional(q, k, v, [p])[0]
    torch.cuda.synchronize()
    qn, kn, vn = (np64(data[c][0]) for c in "qkv")
    s = 1 / math.sqrt(cfg.head_dim)
    pf = float(np.float32(p))
    ref = oracle.layer(qn, kn, vn, cfg.n_q, cfg.n_k, cfg.iters, pf, seed_q=100, seed_k=200)
    assert np.mean(st.layer.labels_q[0].cpu().numpy() == ref.km_q.labels) >= 0.999
    rec = np.mean(oracle.recall_rows(qn, kn, ref.km_q.labels, ref.km_k.labels, ref.selection.lists, s))
    assert abs(float(sem["recall"][0]) - rec) <= 1e-3
    assert int(sem["pairs"][0]) == ref.pairs
    b = oracle.positional_selection(qn, kn, 128, pf)
    rec_b = np.mean(oracle.recall_rows(qn, kn, b.zq, b.zk, b.selection.lists, s))
    assert abs(float(pos["recall"][0]) - rec_b) <= 1e-5
    assert int(pos["pairs"][0]) == b.pairs


# ====================================================================== fp8 attention
def _decode_e4m3(b):
    g = oracle.e4m3_grid()
    mag = b & 0x7F
    assert np.all(mag < 127), "NaN code"
    return np.where(b & 0x80, -1.0, 1.0) * g[mag]


@pytest.mark.parametrize("d", [128, 64])
def test_quantize_fp8_bit_exact(d):
    """E4M3 bytes and scales against the oracle's quantizer, over magnitudes
    that reach the subnormal codes, with one all-zero problem."""
    bh, N = 3, 1000
    rng = np.random.default_rng(d)
    x = rng.standard_normal((bh, N, d)) * 2.0 ** rng.integers(-14, 4, (bh, N, 1))
    x[2] = 0.0
    xb = torch.from_numpy(x).to(torch.bfloat16)
    x8, sc = B.quantize_fp8(xb.to(DEV))
    torch.cuda.synchronize()
    for h in range(bh):
        xs = np64(xb[h])
        s = oracle.fp8_scale(xs)
        assert float(sc[h]) == s
        np.testing.assert_array_equal(_decode_e4m3(x8[h].cpu().numpy()), oracle.fp8_quantize(xs))


# Tolerances of the FP8 path.  Against the oracle on the dequantized inputs the
# error is the E4M3 rounding of P (half a code step is 2^-4 relative, about
# 3.6% RMS per probability), which a fp64 model of exactly that rounding puts
# at 2.6% rel-L2 on this mixture (measured on the GPU: 2.6%, max-abs 1.1e-2);
# against the bf16 inputs the E4M3 rounding of Q, K and V adds to it (6%).
FP8_TOL_DEQ = (5e-2, 4e-2)        # max-abs, rel-L2 against the oracle on the dequantized inputs
FP8_TOL_RAW = 1e-1                # rel-L2 against the oracle on the bf16 inputs


@pytest.mark.parametrize("N,n_q,n_k", [(3000, 20, 50), (6000, 1500, 200), (4099, 7, 130)])
def test_varblock_attn_fp8_vs_oracle(N, n_q, n_k):
    """Including many Q-clusters (the per-XCD plan over more than 1024 clusters)
    and a ragged token count."""
    bh = 2
    q, k, v, qo, ko, cnt, idx, lists, qo_np, ko_np = _attn_case("bf16", 128, bh, N, n_q, n_k, 0.9, seed=91 + n_q,
                                                               empty_rows=True)
    q8, sq = B.quantize_fp8(q.to(DEV))
    k8, sk = B.quantize_fp8(k.to(DEV))
    v8, sv = B.quantize_fp8(v.to(DEV))
    out, lse = B.varblock_attn_fp8(q8, k8, v8, sq, sk, sv, qo, ko, cnt, idx, lse=True)
    torch.cuda.synchronize()
    s = 1 / math.sqrt(128)
    for h in range(bh):
        deq = []
        for x in (q, k, v):
            xs = np64(x[h])
            deq.append(oracle.fp8_quantize(xs) * oracle.fp8_scale(xs))
        ref, ref_lse = oracle.block_attention(*deq, qo_np[h], ko_np[h], lists[h], s)
        raw, _ = oracle.block_attention(np64(q[h]), np64(k[h]), np64(v[h]), qo_np[h], ko_np[h], lists[h], s)
        got = np64(out[h])
        fin = np.isfinite(ref_lse)
        err_deq = (np.max(np.abs(got - ref)), rel_l2(got, ref))
        err_raw = rel_l2(got, raw)
        print(f"head {h}: vs dequantized max-abs {err_deq[0]:.3e} rel-L2 {err_deq[1]:.3e}; vs bf16 rel-L2 {err_raw:.3e}; "
              f"lse max-abs {np.max(np.abs(lse[h].cpu().numpy()[fin] - ref_lse[fin])):.3e}")
        assert err_deq[0] <= FP8_TOL_DEQ[0] and err_deq[1] <= FP8_TOL_DEQ[1]
        assert err_raw <= FP8_TOL_RAW
        np.testing.assert_allclose(lse[h].cpu().numpy()[fin], ref_lse[fin], rtol=0, atol=1e-3)
        assert np.all(lse[h].cpu().numpy()[~fin] == -np.inf) and np.all(got[~fin] == 0)


@pytest.mark.parametrize("layout", ["contiguous", "bnhd"])
def test_varblock_attn_fp8_unpermute_equals_attn_then_unpermute(layout):
    """The FP8 attention with the inverse permutation in its stores writes, bit
    for bit, what the FP8 attention followed by the stand-alone un-permute
    writes (outputs and lse); the permutation is the oracle's of random labels."""
    bh, N, n_q, n_k, heads = 4, 2500, 16, 40, 2
    q, k, v, qo, ko, cnt, idx, lists, qo_np, ko_np = _attn_case("bf16", 128, bh, N, n_q, n_k, 0.9, seed=93,
                                                               empty_rows=True)
    q8, sq = B.quantize_fp8(q.to(DEV))
    k8, sk = B.quantize_fp8(k.to(DEV))
    v8, sv = B.quantize_fp8(v.to(DEV))
    perm = np.stack([oracle.counting_sort(synth.random_labels(N, 23, seed=40 + p), 23)[0] for p in range(bh)])
    pd = torch.from_numpy(perm.astype(np.int32)).to(DEV)
    o_ref, l_ref = B.varblock_attn_fp8(q8, k8, v8, sq, sk, sv, qo, ko, cnt, idx, lse=True)
    if layout == "contiguous":
        dst = torch.full((bh, N, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
        view = dst
        want = torch.empty_like(dst)
        B.unpermute(o_ref, pd, out=want)
    else:
        dst = torch.full((bh // heads, N, heads, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
        view = dst.transpose(1, 2)
        want_full = torch.empty_like(dst)
        B.unpermute(o_ref, pd, out=want_full.transpose(1, 2))
        want = want_full
    _, lse = B.varblock_attn_fp8_unpermute(q8, k8, v8, sq, sk, sv, qo, ko, cnt, idx, pd, lse=True, out=view)
    torch.cuda.synchronize()
    assert torch.equal(dst.view(torch.int16), want.view(torch.int16))
    lr = l_ref.cpu().numpy()
    for p in range(bh):
        np.testing.assert_array_equal(lse[p].cpu().numpy()[perm[p]], lr[p])


def test_layer_fp8_attention_vs_oracle():
    """One head of the small bf16 config: the whole layer with FP8 attention
    against the oracle layer (fp64 on the bf16 inputs), at the FP8 tolerance."""
    from sparse_attention_video_head_amd.pipeline import SVG2Layer
    cfg = synth.CONFIGS["small"]
    data = synth.make_layer(cfg, heads=[0])
    layer = SVG2Layer(1, cfg.n_tokens, cfg.head_dim, torch.bfloat16, cfg.n_q, cfg.n_k, fp8_attention=True)
    top_p = cfg.top_p[0]
    out = layer.run(data["q"].to(DEV), data["k"].to(DEV), data["v"].to(DEV), top_p, iters=cfg.iters,
                    seed_q=100, seed_k=200)
    torch.cuda.synchronize()
    q, k, v = (np64(data[x][0]) for x in "qkv")
    ref = oracle.layer(q, k, v, cfg.n_q, cfg.n_k, cfg.iters, float(np.float32(top_p)), seed_q=100, seed_k=200)
    assert np.mean(layer.labels_k[0].cpu().numpy() == ref.km_k.labels) >= 0.999
    got = np64(out[0])
    print(f"fp8 layer vs oracle rel-L2 {rel_l2(got, ref.out):.4f}")
    assert rel_l2(got, ref.out) <= FP8_TOL_RAW
