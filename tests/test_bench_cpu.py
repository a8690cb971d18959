"""bench.py host logic that needs no GPU: the roofline traffic lookup."""
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _profile(path, sha, value):
    path.write_text("# counters\n\n"
                    f"- attn.hip sha256[:16]: {sha}\n"
                    f"- calibrated HBM bytes per launch: {value}\n"
                    "- algorithmic bytes per launch (Q, K, V read once, O written once): 2.9e+09\n")


def test_traffic_read_when_the_hash_matches(tmp_path, monkeypatch):
    src = tmp_path / "attn.hip"
    src.write_bytes(b"kernel source")
    sha = hashlib.sha256(b"kernel source").hexdigest()[:16]
    prof = tmp_path / "prof.md"
    _profile(prof, sha, "3.5e+11")
    monkeypatch.setattr(bench, "ATTN_SOURCE", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    assert bench.attn_traffic_per_launch() == 3.5e11


def test_traffic_null_once_the_kernel_changed(tmp_path, monkeypatch):
    src = tmp_path / "attn.hip"
    src.write_bytes(b"kernel source, edited")
    prof = tmp_path / "prof.md"
    _profile(prof, hashlib.sha256(b"kernel source").hexdigest()[:16], "3.5e+11")
    monkeypatch.setattr(bench, "ATTN_SOURCE", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    assert bench.attn_traffic_per_launch() is None


def test_committed_profile_parses():
    """The committed counter summary has both fields in the form the lookup reads."""
    fields = {}
    for line in open(bench.TRAFFIC_PROFILE):
        if ": " in line and line.startswith("- "):
            k, v = line[2:].split(": ", 1)
            fields[k.strip()] = v.strip()
    assert len(fields["attn.hip sha256[:16]"]) == 16
    assert float(fields["calibrated HBM bytes per launch"]) > 0


def test_cpu_baseline_sample_on_the_tiny_config():
    """The oracle leg on a small layer: every stage timed, the sample named."""
    from sparse_attention_video_head_amd import synth
    cfg = synth.CONFIGS["tiny"]
    host = synth.make_layer(cfg)
    r = bench.cpu_baseline(host, cfg, 0.9, budget_s=5.0)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
    assert set(r["stage_s_per_head"]) == {"kmeanspp", "lloyd", "permute_select", "attention", "unpermute"}
    assert f"all {cfg.iters} Lloyd rounds" in r["sample"] and "32 picks per side" in r["sample"]
    assert f"on {cfg.n_q} of {cfg.n_q} Q-clusters" in r["sample"]
