"""bench.py's host-side contract and models (CPU only).

* --gpus above 1 is refused with a message before anything touches a GPU;
* the segment plan bench.py models (for the state pass's matrix-core work)
  is the library's: the workspace the library asks for holds one segment
  record per (head, segment) of exactly that plan;
* the matrix-core model equals the counters recorded for the 5 s video
  stream, operation for operation;
* the algorithmic bytes follow their stated per-token-head figures.
"""
import os
import subprocess
import sys

import pytest

import bench
from linear_attention_sequence_modality_amd import kda
from linear_attention_sequence_modality_amd.inputs import WORKLOAD, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "single-GPU" in r.stderr and r.stdout.strip() == ""


@pytest.fixture(scope="module")
def lib():
    try:
        return kda.load_library()
    except RuntimeError as e:
        pytest.skip(str(e))


@pytest.mark.parametrize("cfg", [c for c in WORKLOADS], ids=[c.name for c in WORKLOADS])
def test_segment_plan_matches_the_library(lib, cfg):
    import torch
    d = kda.make_desc(cfg.n_text, cfg.grid, causal_t=cfg.causal_t)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    ws = kda.kda_forward_workspace_size(d, cfg.B, cfg.H, cfg.dk, cfg.dv, dt)
    nseg, _ = bench.seg_plan(cfg)
    nch = (cfg.T + 63) // 64
    per_chunk = int(lib.kda_forward_workspace_size(kda.make_desc(64, (0, 0, 0)), 1, 1, cfg.dk, cfg.dv,
                                                   kda._dtype_code(dt)))
    records = (per_chunk * cfg.H * cfg.B * nch + 255) // 256 * 256
    seg_bytes = (2 * cfg.dk * cfg.dv + cfg.dk * cfg.dk) * 4
    want = records + (cfg.B * nseg * cfg.H * seg_bytes if nseg > 1 else 0)
    assert ws == want, (cfg.name, ws, want, nseg)


def test_mfma_model_equals_the_recorded_counters():
    cfg = WORKLOAD["video_5s_480x832"]
    fl = bench.mfma_flops(cfg)
    rec = bench.MEASURED_MFMA_MOPS
    assert fl["chunks"] == (rec[(cfg.name, "chunks")][1] + rec[(cfg.name, "chunks")][2]) * 512
    assert fl["scan"] == rec[(cfg.name, "scan")][1] * 512
    assert fl["scan_f32"] == rec[(cfg.name, "scan")][2] * 512


def test_algorithmic_bytes_per_token_head():
    """The measurement plan's figures at d = 128 in bf16: conv 1536, chunk transform 2306,
    state pass 1536, path minimum 2818 bytes per token-head."""
    cfg = WORKLOAD["video_5s_480x832"]
    th = cfg.B * cfg.T * cfg.H
    rb = bench.roofline_bytes(cfg)
    taps = 31 * cfg.H * (2 * cfg.dk + cfg.dv) * 2
    assert rb["conv"] == th * 1536 + taps                 # q, k, v in and out
    assert rb["chunks"] == th * 2306                      # q', k', v', alpha, beta in; 5 d workspace out
    assert rb["scan"] == th * 1536                        # 5 d workspace in; o out
    assert rb["path_min"] == th * 2818                    # conv in/out + KDA in/out
    nch = (cfg.T + 63) // 64
    ws = th * (3 * 128 + 64 + 128) * 2 + cfg.B * cfg.H * nch * 128 * 4
    assert rb["scan_interface"] == ws + th * 128 * 2      # this design's workspace once, o once
    assert rb["chunks_interface"] == th * (4 * 128 + 1) * 2 + ws
