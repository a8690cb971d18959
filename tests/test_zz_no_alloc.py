"""svg2_varblock_attn_noalloc: the attention with the library's fixed scratch
array instead of a caller workspace, called through the C ABI, against
svg2_varblock_attn on the same inputs (same kernels, so bit-identical), on two
calls in a row, the second smaller; and the size limit refused on the host."""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_video_head_amd import binding as B
from sparse_attention_video_head_amd import synth

DEV = "cuda"


def _case(bh, N, d, n_q, n_k, top_p, seed, dtype):
    rng = np.random.default_rng(seed)
    q, k, v = (torch.from_numpy(rng.standard_normal((bh, N, d))).to(dtype) for _ in range(3))
    qo, ko, cnt, idx, lists = [], [], [], [], []
    for h in range(bh):
        _, oq, _ = oracle.counting_sort(synth.random_labels(N, n_q, seed=seed + h, skew=0.7), n_q)
        _, okk, ck = oracle.counting_sort(synth.random_labels(N, n_k, seed=seed + 50 + h, skew=0.9), n_k)
        P = oracle.centroid_probs(synth.gaussian_centroids(n_q, d, seed + h),
                                  synth.gaussian_centroids(n_k, d, seed + 99 + h), ck, 1 / math.sqrt(d))
        ls = oracle.select_topp(P, ck, top_p).lists
        row = np.zeros((n_q, n_k), np.int32)
        for i, l in enumerate(ls):
            row[i, :len(l)] = l
        qo.append(oq); ko.append(okk); idx.append(row); cnt.append([len(l) for l in ls]); lists.append(ls)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int32)).to(DEV)
    return (q.to(DEV), k.to(DEV), v.to(DEV), t(qo), t(ko), t(cnt), t(idx)), lists, np.array(qo), np.array(ko)


@pytest.mark.gpu
def test_noalloc_attention_equals_workspace_call_twice():
    """Two calls in a row (the second on a smaller problem, so stale scratch
    from the first would show) give bit for bit what svg2_varblock_attn with a
    caller workspace gives, and the oracle's block attention within the bf16
    bars."""
    cases = [(4, 3000, 128, 40, 90, 0.9, 11, torch.bfloat16), (2, 1100, 64, 9, 20, 0.8, 12, torch.bfloat16),
             (1, 700, 64, 5, 7, 0.95, 13, torch.float32)]
    for bh, N, d, n_q, n_k, p, seed, dt in cases:
        print(f"noalloc case bh={bh} N={N} d={d} n_q={n_q} n_k={n_k} {dt}", flush=True)
        args, lists, qo_np, ko_np = _case(bh, N, d, n_q, n_k, p, seed, dt)
        q = args[0]
        out = torch.full_like(q, float("nan"))
        lse = torch.full((bh, N), float("nan"), dtype=torch.float32, device=DEV)
        B.varblock_attn_noalloc(*args, out=out, lse=lse)
        ref, ref_lse = B.varblock_attn(*args, lse=True)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if dt == torch.bfloat16 else out.view(torch.int32),
                           ref.view(torch.int16) if dt == torch.bfloat16 else ref.view(torch.int32))
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
        tol = (2e-2, 1e-2) if dt == torch.bfloat16 else (1e-4, 1e-4)
        s = 1 / math.sqrt(d)
        for h in range(bh):
            o_ref, _ = oracle.block_attention(*(x[h].double().cpu().numpy() for x in args[:3]), qo_np[h], ko_np[h],
                                              lists[h], s)
            got = out[h].double().cpu().numpy()
            assert np.max(np.abs(got - o_ref)) <= tol[0]
            assert np.linalg.norm(got - o_ref) <= tol[1] * np.linalg.norm(o_ref)


def test_noalloc_refuses_problems_beyond_the_scratch_on_the_host():
    """Sizes whose workspace exceeds the fixed array are refused with
    SVG2_ERR_WORKSPACE before any HIP call (so this runs without a GPU);
    argument errors are svg2_varblock_attn's."""
    L = B.lib()
    cap = L.svg2_varblock_attn_noalloc_max_scratch()
    assert cap == 16 << 20
    FAKE = 0x10000

    def call(bh, N, n_q, n_k, d=128, q=FAKE):
        return L.svg2_varblock_attn_noalloc(q, FAKE, FAKE, 1, bh, N, d, FAKE, n_q, FAKE, n_k, FAKE, FAKE,
                                            ctypes.c_float(0.088), FAKE, None, None)
    big = (512, 118800, 400, 1000)
    assert L.svg2_varblock_attn_workspace_size(*big, 128) > cap
    assert call(*big) == 3                       # SVG2_ERR_WORKSPACE
    assert call(24, 118800, 400, 1000, q=None) == 1  # SVG2_ERR_INVALID_ARG
    assert call(24, 118800, 400, 1000, d=96) == 2    # SVG2_ERR_UNSUPPORTED
