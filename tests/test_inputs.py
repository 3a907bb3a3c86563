"""Stream-shape bookkeeping and the synthetic input recipe (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

from linear_attention_sequence_modality_amd.inputs import (
    WORKLOADS, WORKLOAD, PATCHIFY, VAE_COMPRESSION, StreamConfig, latent_grid, make_inputs, token_index)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "stream_shapes.json")


def test_grid_arithmetic_matches_pages():
    g = json.load(open(GOLDEN))
    assert list(VAE_COMPRESSION) == g["vae_compression"]
    assert list(PATCHIFY) == g["patchify"]
    assert VAE_COMPRESSION[1] * PATCHIFY[1] == g["effective_spatial_patch"]
    for case in g["cases"]:
        grid = latent_grid(case["frames"], case["height"], case["width"])
        assert list(grid) == case["grid"]
        assert int(np.prod(grid)) == case["visual_tokens"]
    # "about 65K tokens" for a 4096^2 image at 16x16
    n = int(np.prod(latent_grid(1, 4096, 4096)))
    assert abs(n - g["image_4096_tokens_about"]) / g["image_4096_tokens_about"] < 0.01


def test_config_table():
    assert [c.T for c in WORKLOADS] == [512, 4608, 33272, 66048, 189272]
    assert [c.B * c.T for c in WORKLOADS] == [512, 36864, 33272, 66048, 189272]
    assert WORKLOAD["tiny_fp32"].dtype == "f32" and all(c.dtype == "bf16" for c in WORKLOADS[1:])


def test_raster_order():
    cfg = WORKLOAD["tiny_fp32"]
    t, h, w = cfg.grid
    idx = [token_index(cfg, a, b, c) for a in range(t) for b in range(h) for c in range(w)]
    assert idx == list(range(cfg.n_text, cfg.T))


def test_inputs_are_seeded_and_follow_the_recipe():
    cfg = StreamConfig("t", B=2, H=3, dk=64, dv=32, n_text=5, grid=(2, 3, 4), dtype="bf16", seed=5)
    a, b = make_inputs(cfg), make_inputs(cfg)
    for key in a:
        assert torch.equal(a[key], b[key])
        assert a[key].dtype == torch.bfloat16
    assert a["q"].shape == (2, cfg.T, 3, 64) and a["v"].shape == (2, cfg.T, 3, 32)
    assert a["beta"].shape == (2, cfg.T, 3)
    assert a["w_text_v"].shape == (3 * 32, 4) and a["w_vis_k"].shape == (3 * 64, 27)
    nq = a["q"].float().norm(dim=-1)
    assert torch.allclose(nq, torch.ones_like(nq), atol=2e-2)
    al = a["alpha"].float()
    assert float(al.min()) > 0.0 and float(al.max()) <= 1.0
    bt = a["beta"].float()
    assert float(bt.min()) > 0.0 and float(bt.max()) < 1.0
    c = make_inputs(cfg, seed=6)
    assert not torch.equal(a["q"], c["q"])


def test_fp32_config_keeps_fp32():
    x = make_inputs(WORKLOAD["tiny_fp32"])
    assert x["q"].dtype == torch.float32


def test_bad_grid_rejected():
    with pytest.raises(ValueError):
        latent_grid(80, 480, 832)
    with pytest.raises(ValueError):
        latent_grid(81, 481, 832)
