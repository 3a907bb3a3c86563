"""Shared helpers for the GPU parity tests (HIP path vs the fp64 oracle)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from linear_attention_sequence_modality_amd import kda
from linear_attention_sequence_modality_amd.inputs import StreamConfig, make_inputs

# Max relative error (per (batch, head): max |x - ref| over max |ref|) allowed
# for each input dtype: fp32 in and out, or bf16 in and out with fp32 accumulation.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(inp: dict) -> dict:
    return {k: v.cuda() for k, v in inp.items()}


def desc_of(cfg: StreamConfig):
    return kda.make_desc(cfg.n_text, cfg.grid, causal_t=cfg.causal_t)


def run_path(cfg: StreamConfig, dev: dict, S0=None, want_state=False):
    """HIP conv then HIP KDA on the current stream; returns host fp64 numpy arrays."""
    d = desc_of(cfg)
    sT = None
    if want_state:
        sT = torch.empty(cfg.B, cfg.H, cfg.dk, cfg.dv, dtype=torch.float32, device="cuda")
    s0 = None if S0 is None else torch.as_tensor(S0, dtype=torch.float32).cuda().contiguous()
    qc, kc, vc, o = kda.conv_kda_forward(d, dev, initial_state=s0, final_state=sT)
    torch.cuda.synchronize()
    return qc, kc, vc, o, sT


def heads_slice(x: torch.Tensor, heads) -> np.ndarray:
    """[B, T, H, d] -> fp64 numpy [B, T, len(heads), d] of the chosen heads."""
    return x[:, :, list(heads)].double().cpu().numpy()


def weight_slice(w: torch.Tensor, heads, d: int) -> np.ndarray:
    """[H*d, taps] -> fp64 numpy [len(heads)*d, taps]."""
    return torch.cat([w[h * d:(h + 1) * d] for h in heads]).double().cpu().numpy()


def oracle_conv_heads(cfg, inp_cpu: dict, stream: str, heads) -> np.ndarray:
    d = cfg.dv if stream == "v" else cfg.dk
    x = heads_slice(inp_cpu[stream], heads)
    return oracle.short_conv_heads(x, weight_slice(inp_cpu["w_text_" + stream], heads, d),
                                   weight_slice(inp_cpu["w_vis_" + stream], heads, d),
                                   cfg.n_text, cfg.grid, cfg.causal_t)


def oracle_end_to_end_heads(cfg, inp_cpu: dict, heads, S0=None):
    qc = oracle_conv_heads(cfg, inp_cpu, "q", heads)
    kc = oracle_conv_heads(cfg, inp_cpu, "k", heads)
    vc = oracle_conv_heads(cfg, inp_cpu, "v", heads)
    s0 = None if S0 is None else np.asarray(S0)[:, list(heads)]
    o, st = oracle.kda_recurrence(qc, kc, vc, heads_slice(inp_cpu["alpha"], heads),
                                  heads_slice(inp_cpu["beta"][..., None], heads)[..., 0], s0)
    return qc, kc, vc, o, st


def rel(x: np.ndarray, ref: np.ndarray) -> float:
    return oracle.rel_err(x, ref)
