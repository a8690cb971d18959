"""The seeded input generator (host only): the incremental denoising sequence
equals regenerating each step from scratch, the drift has the stated size,
and the label field has the configured structure."""
import dataclasses

import numpy as np
import torch

from sparse_attention_video_head_amd import synth


def _small_denoise():
    # the denoising generator on a small grid: same recipe, fewer tokens
    base = synth.CONFIGS["denoise"]
    return dataclasses.replace(base, name="denoise-small", heads=2, n_tokens=4 * 8 * 16, grid=(4, 8, 16),
                               n_centers=40, n_q=8, n_k=16, steps=4)


def test_denoise_sequence_matches_make_layer():
    cfg = _small_denoise()
    serial = list(synth.denoise_sequence(cfg))
    pooled = list(synth.denoise_sequence(cfg, workers=2))
    for s in range(cfg.steps):
        ref = synth.make_layer(cfg, step=s)
        assert serial[s]["step"] == pooled[s]["step"] == s
        for x in "qkv":
            assert torch.equal(serial[s][x], ref[x]), (s, x)
            assert torch.equal(pooled[s][x], ref[x]), (s, x)


def test_drift_is_relative_rms_noise():
    cfg = _small_denoise()
    q0, _, _, _ = synth.head_master(cfg, 0)
    q1 = synth.drift_step(cfg, 0, 1, q0, 0)
    rms = np.sqrt(np.mean(q0 * q0))
    step_rms = np.sqrt(np.mean((q1 - q0) ** 2))
    assert abs(step_rms / (cfg.drift * rms) - 1.0) < 0.05


def test_voronoi_labels_are_spatially_coherent():
    cfg = synth.CONFIGS["small"]
    lab = synth.make_layer(cfg, heads=[0])["labels"][0].numpy().reshape(cfg.grid)
    same_x = np.mean(lab[:, :, 1:] == lab[:, :, :-1])
    # neighbours share a label far more often than 1/C (0.005); the 20% of
    # relabelled tokens cap it near 0.8^2 times the chance of sharing a cell
    assert 0.25 < same_x < 0.7
