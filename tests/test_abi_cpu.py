"""The C ABI without a GPU: the library loads, exports every function that
include/svg2.h declares, and rejects bad arguments on the host before any
HIP call (so these calls never touch a device)."""
import ctypes
import os
import re

import pytest

from sparse_attention_video_head_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "svg2.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x10000        # 16-byte aligned non-null address; never dereferenced
MISALIGNED = 0x10004


def _declared():
    src = open(HDR).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(svg2_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_five_calls():
    names = _declared()
    for call in ("svg2_kmeans", "svg2_permute", "svg2_select_topp", "svg2_varblock_attn", "svg2_unpermute"):
        assert call in names


def test_library_exports_every_declared_symbol():
    L = B.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert sorted(_declared()) == sorted(B.EXPORTED)
    assert "gfx950" in B.version()


def test_status_strings():
    L = B.lib()
    for s in range(5):
        assert L.svg2_status_string(s)
    assert L.svg2_status_string(99) == b"unknown status"


def _km(**kw):
    a = dict(x=FAKE, dtype=1, bh=2, N=1000, d=128, n=16, iters=3, init=None, seed=0, cent=FAKE, lab=FAKE,
             cnt=FAKE, md=None, si=None, ws=FAKE, wsn=1 << 40)
    a.update(kw)
    return B.lib().svg2_kmeans(a["x"], a["dtype"], a["bh"], a["N"], a["d"], a["n"], a["iters"], a["init"],
                               a["seed"], a["cent"], a["lab"], a["cnt"], a["md"], a["si"], a["ws"], a["wsn"],
                               None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), INVALID), (dict(x=MISALIGNED), INVALID), (dict(dtype=7), INVALID),
    (dict(bh=0), INVALID), (dict(N=0), INVALID), (dict(n=0), INVALID), (dict(n=1001), INVALID),
    (dict(n=4097, N=10000), INVALID), (dict(d=96), UNSUPPORTED), (dict(iters=-1), INVALID),
    (dict(iters=101), INVALID), (dict(cent=None), INVALID), (dict(lab=None), INVALID),
    (dict(cnt=None), INVALID), (dict(N=1 << 25), INVALID), (dict(wsn=10), WORKSPACE),
    (dict(ws=None), WORKSPACE), (dict(init=MISALIGNED), INVALID), (dict(lab=FAKE + 2), INVALID),
])
def test_kmeans_validation(kw, code):
    assert _km(**kw) == code


def test_kmeans_size_queries():
    L = B.lib()
    assert L.svg2_kmeans_workspace_size(1, 10, 96, 4) == 0
    assert L.svg2_kmeans_workspace_size(1, 10, 128, 11) == 0
    assert L.svg2_kmeans_workspace_size(24, 118800, 128, 1000) > 24 * 118800 * 8


def test_token_limit_below_2_pow_24():
    """n_tokens < 2^24: one head's rows at d = 128 then stay under the 4 GiB a
    buffer resource addresses."""
    L = B.lib()
    assert L.svg2_kmeans_workspace_size(1, (1 << 24) - 1, 128, 8) > 0
    assert L.svg2_kmeans_workspace_size(1, 1 << 24, 128, 8) == 0
    assert L.svg2_varblock_attn_workspace_size(1, (1 << 24) - 1, 8, 8, 128) > 0
    assert L.svg2_varblock_attn_workspace_size(1, 1 << 24, 8, 8, 128) == 0


def _perm(**kw):
    a = dict(lab=FAKE, bh=4, N=500, n=8, nt=1, src=[FAKE], heads=1, sb=500 * 128, sh=0, st=128, dst=[FAKE],
             dtype=1, d=128, perm=FAKE, off=FAKE, ws=FAKE, wsn=1 << 30)
    a.update(kw)
    src = (ctypes.c_void_p * 2)(*a["src"], *([0] * (2 - len(a["src"]))))
    dst = (ctypes.c_void_p * 2)(*a["dst"], *([0] * (2 - len(a["dst"]))))
    return B.lib().svg2_permute(a["lab"], a["bh"], a["N"], a["n"], a["nt"], src, a["heads"], a["sb"], a["sh"],
                                a["st"], dst, a["dtype"], a["d"], a["perm"], a["off"], a["ws"], a["wsn"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(nt=0), INVALID), (dict(nt=3), INVALID), (dict(src=[0]), INVALID), (dict(dst=[MISALIGNED]), INVALID),
    (dict(nt=2, src=[FAKE]), INVALID), (dict(heads=3), INVALID), (dict(st=12), INVALID), (dict(sb=-128), INVALID),
    (dict(lab=None), INVALID), (dict(perm=None), INVALID), (dict(off=None), INVALID), (dict(d=32), UNSUPPORTED),
    (dict(wsn=4), WORKSPACE), (dict(n=501), INVALID),
])
def test_permute_validation(kw, code):
    assert _perm(**kw) == code


def _sel(**kw):
    a = dict(cq=FAKE, qc=FAKE, nq=10, ck=FAKE, kc=FAKE, nk=20, bh=2, d=128, scale=0.088, p=0.9, sc=FAKE,
             si=FAKE, pr=None, pc=None, ws=FAKE, wsn=1 << 20)
    a.update(kw)
    return B.lib().svg2_select_topp(a["cq"], a["qc"], a["nq"], a["ck"], a["kc"], a["nk"], a["bh"], a["d"],
                                    ctypes.c_float(a["scale"]), ctypes.c_float(a["p"]), a["sc"], a["si"],
                                    a["pr"], a["pc"], a["ws"], a["wsn"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(p=0.0), INVALID), (dict(p=1.5), INVALID), (dict(p=float("nan")), INVALID),
    (dict(scale=0.0), INVALID), (dict(scale=float("inf")), INVALID), (dict(nk=4097), INVALID),
    (dict(nq=0), INVALID), (dict(cq=None), INVALID), (dict(si=None), INVALID), (dict(d=80), UNSUPPORTED),
    (dict(pc=FAKE + 4), INVALID), (dict(wsn=0), WORKSPACE),
])
def test_select_validation(kw, code):
    assert _sel(**kw) == code


def _attn(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, bh=2, N=1000, d=128, qo=FAKE, nq=8, ko=FAKE, nk=9, sc=FAKE,
             si=FAKE, scale=0.088, out=FAKE, lse=None, ws=FAKE, wsn=1 << 30)
    a.update(kw)
    return B.lib().svg2_varblock_attn(a["q"], a["k"], a["v"], a["dtype"], a["bh"], a["N"], a["d"], a["qo"],
                                      a["nq"], a["ko"], a["nk"], a["sc"], a["si"], ctypes.c_float(a["scale"]),
                                      a["out"], a["lse"], a["ws"], a["wsn"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(v=MISALIGNED), INVALID), (dict(out=None), INVALID), (dict(dtype=2), INVALID),
    (dict(N=1 << 25), INVALID), (dict(nq=5000), INVALID), (dict(scale=-1.0), INVALID), (dict(d=256), UNSUPPORTED),
    (dict(si=None), INVALID), (dict(lse=FAKE + 2), INVALID), (dict(wsn=16), WORKSPACE),
])
def test_attn_validation(kw, code):
    assert _attn(**kw) == code


def _attn_unperm(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, bh=2, N=1000, d=128, qo=FAKE, nq=8, ko=FAKE, nk=9, sc=FAKE,
             si=FAKE, scale=0.088, perm=FAKE, out=FAKE, heads=1, sb=128000, sh=0, st=128, lse=None, ws=FAKE,
             wsn=1 << 30)
    a.update(kw)
    return B.lib().svg2_varblock_attn_unpermute(
        a["q"], a["k"], a["v"], a["dtype"], a["bh"], a["N"], a["d"], a["qo"], a["nq"], a["ko"], a["nk"], a["sc"],
        a["si"], ctypes.c_float(a["scale"]), a["perm"], a["out"], a["heads"], a["sb"], a["sh"], a["st"], a["lse"],
        a["ws"], a["wsn"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(perm=None), INVALID), (dict(perm=FAKE + 2), INVALID), (dict(out=None), INVALID),
    (dict(heads=3), INVALID), (dict(st=130), INVALID), (dict(sb=-8), INVALID), (dict(dtype=2), INVALID),
    (dict(N=1 << 25), INVALID), (dict(nk=5000), INVALID), (dict(scale=0.0), INVALID), (dict(d=96), UNSUPPORTED),
    (dict(lse=FAKE + 2), INVALID), (dict(wsn=16), WORKSPACE),
])
def test_attn_unpermute_validation(kw, code):
    """The fused call validates like the attention and unpermute calls, before any HIP call."""
    assert _attn_unperm(**kw) == code


def _kmeans_perm(**kw):
    a = dict(x=FAKE, y=FAKE + 4096, dtype=1, bh=2, N=1000, d=128, n=8, it=3, init=None, cent=FAKE + 8192,
             lab=FAKE + 12288, cnt=FAKE + 16384, xp=FAKE + 20480, yp=FAKE + 24576, perm=FAKE + 28672,
             off=FAKE + 32768, ws=FAKE + 36864, wsn=1 << 30)
    a.update(kw)
    return B.lib().svg2_kmeans_permute(
        a["x"], a["y"], a["dtype"], a["bh"], a["N"], a["d"], a["n"], a["it"], a["init"], ctypes.c_uint64(7),
        a["cent"], a["lab"], a["cnt"], None, None, a["xp"], a["yp"], a["perm"], a["off"], a["ws"], a["wsn"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(it=0), INVALID), (dict(xp=None), INVALID), (dict(xp=FAKE + 20482), INVALID), (dict(perm=None), INVALID),
    (dict(off=None), INVALID), (dict(y=None), INVALID), (dict(yp=None), INVALID), (dict(yp=FAKE + 24578), INVALID),
    (dict(xp=FAKE), INVALID), (dict(yp=FAKE + 4096), INVALID), (dict(yp=FAKE + 20480), INVALID),
    (dict(lab=None), INVALID), (dict(dtype=2), INVALID), (dict(d=96), UNSUPPORTED), (dict(n=1001), INVALID),
    (dict(it=101), INVALID), (dict(wsn=16), WORKSPACE),
])
def test_kmeans_permute_validation(kw, code):
    """The fused k-means + permutation validates every argument before any HIP call:
    n_iters >= 1, outputs present, aligned and not aliasing the inputs, y and y_perm given together."""
    assert _kmeans_perm(**kw) == code


def _kmeans_perm8(**kw):
    a = dict(x=FAKE, y=FAKE + 4096, bh=2, N=1000, d=128, n=8, it=3, init=None, cent=FAKE + 8192, lab=FAKE + 12288,
             cnt=FAKE + 16384, xp=FAKE + 20480, xs=FAKE + 40960, yp=FAKE + 24576, ys=FAKE + 45056,
             perm=FAKE + 28672, off=FAKE + 32768, ws=FAKE + 36864, wsn=1 << 30)
    a.update(kw)
    return B.lib().svg2_kmeans_permute_fp8(
        a["x"], a["y"], a["bh"], a["N"], a["d"], a["n"], a["it"], a["init"], ctypes.c_uint64(7), a["cent"], a["lab"],
        a["cnt"], a["xp"], a["xs"], a["yp"], a["ys"], a["perm"], a["off"], a["ws"], a["wsn"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(it=0), INVALID), (dict(xp=None), INVALID), (dict(xs=None), INVALID), (dict(xs=FAKE + 40962), INVALID),
    (dict(y=None), INVALID), (dict(ys=None), INVALID), (dict(yp=None), INVALID),
    (dict(y=None, yp=None), INVALID), (dict(y=None, ys=None), INVALID), (dict(xp=FAKE), INVALID),
    (dict(yp=FAKE + 20480), INVALID), (dict(d=96), UNSUPPORTED), (dict(n=2000), INVALID), (dict(wsn=16), WORKSPACE),
])
def test_kmeans_permute_fp8_validation(kw, code):
    """The E4M3 variant adds the scale outputs; y, y8_perm and y_scale go together."""
    assert _kmeans_perm8(**kw) == code


def test_unpermute_validation():
    L = B.lib()
    assert L.svg2_unpermute(None, 1, 1, 10, 128, FAKE, FAKE, 1, 1280, 0, 128, None) == INVALID
    assert L.svg2_unpermute(FAKE, 1, 1, 10, 100, FAKE, FAKE, 1, 1280, 0, 128, None) == UNSUPPORTED
    assert L.svg2_unpermute(FAKE, 1, 2, 10, 128, FAKE, FAKE, 3, 1280, 0, 128, None) == INVALID
    assert L.svg2_unpermute(FAKE, 0, 1, 10, 128, FAKE, FAKE, 1, 1280, 0, 130, None) == INVALID
    assert L.svg2_unpermute(FAKE, 1, 1, 10, 128, None, FAKE, 1, 1280, 0, 128, None) == INVALID


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(B.Svg2Error):
        B.kmeans(torch.zeros(1, 8, 64), 2, 1)
    with pytest.raises(B.Svg2Error):
        B.unpermute(torch.zeros(1, 8, 64), torch.zeros(1, 8, dtype=torch.int32))
    with pytest.raises(B.Svg2Error):
        B.kmeans_permute(torch.zeros(1, 8, 64), 2, 1, y=torch.zeros(1, 8, 64))
    with pytest.raises(B.Svg2Error):
        z8 = torch.zeros(1, 8, 128, dtype=torch.uint8)
        s1 = torch.ones(1)
        i1 = torch.zeros(1, 2, dtype=torch.int32)
        B.varblock_attn_fp8_unpermute(z8, z8, z8, s1, s1, s1, i1, i1, torch.ones(1, 1, dtype=torch.int32),
                                      torch.zeros(1, 1, 1, dtype=torch.int32), torch.zeros(1, 8, dtype=torch.int32))


def _means(**kw):
    a = dict(x=FAKE, dtype=1, bh=2, N=500, d=128, lab=FAKE, n=8, means=FAKE, cnt=FAKE, ws=FAKE, wsn=1 << 30)
    a.update(kw)
    return B.lib().svg2_cluster_means(a["x"], a["dtype"], a["bh"], a["N"], a["d"], a["lab"], a["n"], a["means"],
                                      a["cnt"], a["ws"], a["wsn"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), INVALID), (dict(bh=0), INVALID), (dict(n=0), INVALID), (dict(n=501), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(x=None), INVALID), (dict(x=MISALIGNED), INVALID), (dict(lab=None), INVALID),
    (dict(means=None), INVALID), (dict(cnt=None), INVALID), (dict(cnt=FAKE + 2), INVALID), (dict(wsn=16), WORKSPACE),
    (dict(ws=None), WORKSPACE),
])
def test_cluster_means_validation(kw, code):
    assert _means(**kw) == code


def test_cluster_means_size_query():
    L = B.lib()
    assert L.svg2_cluster_means_workspace_size(1, 10, 96, 4) == 0
    assert L.svg2_cluster_means_workspace_size(1, 10, 128, 11) == 0
    # the per-chunk partial sums dominate: bh (n + ceil(N / 512)) d doubles
    assert L.svg2_cluster_means_workspace_size(24, 118800, 128, 929) >= 24 * (929 + 233) * 128 * 8


def test_recall_mass_validation():
    L = B.lib()
    assert L.svg2_recall_mass(FAKE, FAKE, 0, 10, FAKE, None) == INVALID
    assert L.svg2_recall_mass(FAKE, FAKE, 1, 0, FAKE, None) == INVALID
    assert L.svg2_recall_mass(FAKE, FAKE, 1, 1 << 25, FAKE, None) == INVALID
    assert L.svg2_recall_mass(None, FAKE, 1, 10, FAKE, None) == INVALID
    assert L.svg2_recall_mass(FAKE, FAKE + 2, 1, 10, FAKE, None) == INVALID
    assert L.svg2_recall_mass(FAKE, FAKE, 1, 10, FAKE + 4, None) == INVALID


def test_fp8_validation():
    L = B.lib()
    ws = FAKE
    assert L.svg2_quantize_fp8_workspace_size(0) == 0
    assert L.svg2_quantize_fp8(FAKE, 0, 10, 128, FAKE, FAKE, ws, 1 << 20, None) == INVALID
    assert L.svg2_quantize_fp8(FAKE, 1, 10, 96, FAKE, FAKE, ws, 1 << 20, None) == UNSUPPORTED
    assert L.svg2_quantize_fp8(None, 1, 10, 128, FAKE, FAKE, ws, 1 << 20, None) == INVALID
    assert L.svg2_quantize_fp8(FAKE, 1, 10, 128, FAKE + 8, FAKE, ws, 1 << 20, None) == INVALID
    assert L.svg2_quantize_fp8(FAKE, 4, 10, 128, FAKE, FAKE, ws, 4, None) == WORKSPACE

    def attn(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, sq=FAKE, sk=FAKE, sv=FAKE, bh=2, N=300, d=128, qo=FAKE, nq=5, ko=FAKE, nk=7,
                 sc=FAKE, si=FAKE, scale=0.088, out=FAKE, lse=None, ws=FAKE, wsn=1 << 30)
        a.update(kw)
        return L.svg2_varblock_attn_fp8(a["q"], a["k"], a["v"], a["sq"], a["sk"], a["sv"], a["bh"], a["N"], a["d"],
                                        a["qo"], a["nq"], a["ko"], a["nk"], a["sc"], a["si"], ctypes.c_float(a["scale"]),
                                        a["out"], a["lse"], a["ws"], a["wsn"], None)
    assert attn(d=64) == UNSUPPORTED
    assert attn(bh=0) == INVALID
    assert attn(nq=0) == INVALID
    assert attn(sv=None) == INVALID
    assert attn(k=MISALIGNED) == INVALID
    assert attn(scale=-1.0) == INVALID
    assert attn(wsn=8) == WORKSPACE

    def attn_unperm(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, sq=FAKE, sk=FAKE, sv=FAKE, bh=2, N=300, d=128, qo=FAKE, nq=5, ko=FAKE, nk=7,
                 sc=FAKE, si=FAKE, scale=0.088, perm=FAKE, out=FAKE, heads=1, sb=38400, sh=0, st=128, lse=None,
                 ws=FAKE, wsn=1 << 30)
        a.update(kw)
        return L.svg2_varblock_attn_fp8_unpermute(
            a["q"], a["k"], a["v"], a["sq"], a["sk"], a["sv"], a["bh"], a["N"], a["d"], a["qo"], a["nq"], a["ko"],
            a["nk"], a["sc"], a["si"], ctypes.c_float(a["scale"]), a["perm"], a["out"], a["heads"], a["sb"], a["sh"],
            a["st"], a["lse"], a["ws"], a["wsn"], None)
    # the fused inverse permutation adds perm and the destination strides to the checks
    assert attn_unperm(d=64) == UNSUPPORTED
    assert attn_unperm(perm=None) == INVALID
    assert attn_unperm(perm=FAKE + 2) == INVALID
    assert attn_unperm(heads=3) == INVALID
    assert attn_unperm(st=130) == INVALID
    assert attn_unperm(out=None) == INVALID
    assert attn_unperm(sv=None) == INVALID
    assert attn_unperm(lse=FAKE + 2) == INVALID
    assert attn_unperm(wsn=8) == WORKSPACE


def test_binding_checks_caller_buffers(monkeypatch):
    """Outputs, in/out buffers and workspaces handed in by the caller are
    checked for device, dtype, exact shape and contiguity before any library
    call: the kernels write through their raw pointers.  Without a GPU the
    inputs are host tensors with the GPU check switched off; a buffer on the
    "meta" device stands for one on another device."""
    import torch
    monkeypatch.setattr(B, "_need_cuda", lambda *ts: None)
    real = B.lib()

    class SizeQueriesOnly:
        """The library with only its workspace-size queries: a check that lets
        a bad buffer through reaches a compute call and fails the test."""
        def __getattr__(self, name):
            if name.endswith("_workspace_size"):
                return getattr(real, name)
            raise AssertionError(f"{name} reached with a bad buffer")

    monkeypatch.setattr(B, "lib", lambda: SizeQueriesOnly())
    bf, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    bh, N, d, n = 2, 100, 64, 5
    meta = lambda *s, dt=i32: torch.empty(*s, dtype=dt, device="meta")
    z = lambda *s, dt=i32: torch.zeros(*s, dtype=dt)
    x = z(bh, N, d, dt=bf)

    def bad(fn, *a, **kw):
        with pytest.raises(B.Svg2Error):
            fn(*a, **kw)

    # k-means
    bad(B.kmeans, x, n, 1, centroids=z(bh, n + 1, d, dt=f32))
    bad(B.kmeans, x, n, 1, labels=meta(bh, N))
    bad(B.kmeans, x, n, 1, counts=z(bh, n, dt=torch.int64))
    bad(B.kmeans, x, n, 1, init=z(bh, n, d + 1, dt=f32))
    bad(B.kmeans, x, n, 1, workspace=meta(1 << 20, dt=torch.uint8))
    bad(B.kmeans, x, n, 1, workspace=z(4, dt=torch.uint8))
    # k-means with the permutation
    bad(B.kmeans_permute, x, n, 1, perm=z(bh, N + 1))
    bad(B.kmeans_permute, x, n, 1, offsets=meta(bh, n + 1))
    bad(B.kmeans_permute, x, n, 1, x_out=z(bh, N, d, dt=f32))
    bad(B.kmeans_permute, x, n, 1, y=x, y_out=z(bh, d, N, dt=bf).transpose(1, 2))
    bad(B.kmeans_permute, x, n, 1, y=meta(bh, N, d, dt=bf))
    bad(B.kmeans_permute, x, n, 1, fp8=True, x_scale=z(bh + 1, dt=f32))
    # permute
    lab = z(bh, N)
    bad(B.permute, lab, n, x, outs=[z(bh, N, d + 1, dt=bf)])
    bad(B.permute, lab, n, x, perm=meta(bh, N))
    bad(B.permute, lab, n, x, offsets=z(bh, n))
    bad(B.permute, lab, n, meta(bh, N, d, dt=bf))
    # select
    cq, ck = z(bh, 3, d, dt=f32), z(bh, n, d, dt=f32)
    qc, kc = z(bh, 3), z(bh, n)
    bad(B.select_topp, cq, z(bh, 4), ck, kc, 0.9)
    bad(B.select_topp, cq, qc, ck, z(bh, n + 1), 0.9)
    bad(B.select_topp, cq, qc, z(bh, n, d + 1, dt=f32), kc, 0.9)
    bad(B.select_topp, cq, qc, ck, kc, 0.9, sel_idx=meta(bh, 3, n))
    bad(B.select_topp, cq, qc, ck, kc, 0.9, pair_count=z(bh, dt=i32))
    # attention
    qo, ko = z(bh, 4), z(bh, n + 1)
    sc, si = z(bh, 3), z(bh, 3, n)
    bad(B.varblock_attn, x, x, x, z(bh + 1, 4), ko, sc, si)
    bad(B.varblock_attn, x, x, x, qo, ko, z(bh, 4), si)
    bad(B.varblock_attn, x, x, x, qo, ko, sc, si, out=meta(bh, N, d, dt=bf))
    bad(B.varblock_attn, x, x, x, qo, ko, sc, si, out=z(bh, N, d, dt=f32))
    bad(B.varblock_attn, x, x, x, qo, ko, sc, si, lse=z(bh, N + 1, dt=f32))
    bad(B.varblock_attn, x, x, x, qo, ko, sc, si, workspace=z(8, dt=torch.uint8))
    bad(B.varblock_attn_unpermute, x, x, x, qo, ko, sc, si, z(bh, N - 1))
    bad(B.varblock_attn_unpermute, x, x, x, qo, ko, sc, si, z(bh, N), out=meta(bh, N, d, dt=bf))
    bad(B.varblock_attn_unpermute, x, x, x, qo, ko, z(bh, 3, n + 1), si, z(bh, N))
    # un-permute
    bad(B.unpermute, x, z(bh, N), out=meta(bh, N, d, dt=bf))
    bad(B.unpermute, x, meta(bh, N))
    # identification study
    bad(B.cluster_means, x, lab, n, means=z(bh, n, d + 1, dt=f32))
    bad(B.cluster_means, x, lab, n, counts=meta(bh, n))
    bad(B.recall_mass, z(bh, N, dt=f32), z(bh, N, dt=f32), out=z(bh, dt=f32))
    # FP8
    bad(B.quantize_fp8, x, x8=meta(bh, N, d, dt=torch.uint8))
    bad(B.quantize_fp8, x, scale=z(bh, 1, dt=f32))
    q8, s1 = z(bh, N, 128, dt=torch.uint8), z(bh, dt=f32)
    bad(B.varblock_attn_fp8, q8, q8, q8, s1, s1, s1, qo, ko, sc, si, out=z(bh, N, 128, dt=f32))
    bad(B.varblock_attn_fp8, q8, q8, q8, s1, s1, s1, qo, ko, sc, si, lse=z(bh, N + 3, dt=f32))
    bad(B.varblock_attn_fp8, q8, q8, q8, z(bh + 1, dt=f32), s1, s1, qo, ko, sc, si)
    bad(B.varblock_attn_fp8_unpermute, q8, q8, q8, s1, s1, s1, qo, ko, z(bh, 2), si, z(bh, N))
    bad(B.varblock_attn_fp8_unpermute, q8, q8, q8, s1, s1, s1, qo, ko, sc, si, z(bh, N),
        out=meta(bh, N, 128, dt=bf))

    # well-formed buffers pass every check and reach the library's compute call
    def good(fn, *a, **kw):
        with pytest.raises(AssertionError, match="reached"):
            fn(*a, **kw)

    good(B.kmeans, x, n, 1, centroids=z(bh, n, d, dt=f32), labels=z(bh, N), counts=z(bh, n))
    good(B.kmeans_permute, x, n, 1, y=x, perm=z(bh, N), offsets=z(bh, n + 1))
    good(B.permute, lab, n, x, outs=[z(bh, N, d, dt=bf)])
    good(B.select_topp, cq, qc, ck, kc, 0.9, pair_count=z(bh, dt=torch.int64))
    good(B.varblock_attn, x, x, x, qo, ko, sc, si, lse=z(bh, N, dt=f32))
    good(B.varblock_attn_unpermute, x, x, x, qo, ko, sc, si, z(bh, N), out=z(bh, N, d, dt=bf))
    good(B.varblock_attn_fp8, q8, q8, q8, s1, s1, s1, qo, ko, sc, si, lse=True)
