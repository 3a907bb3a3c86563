"""Seeded synthetic token streams for the conv + KDA token mixer.

This module is shared by the oracle tests and the HIP path; it holds shapes,
stream layout bookkeeping and value distributions only, none of the method's
arithmetic (no convolution, no decay, no state update).

Stream layout (Chimera paper, core method and method step (2)): text tokens
first, then the visual tokens of the (t, h, w) latent-patch grid flattened in
time-major raster order (w fastest).  The grid of a clip follows from the
frozen causal 3D VAE with (4, 8, 8) compression followed by a (1, 2, 2)
patchify (method step (1)): ``(1 + (frames - 1) // 4, height // 16, width // 16)``.

Value distributions (the workload descriptions of the five stream configs):
q, k ~ N(0, 1) then L2-normalised over the key dimension per (b, t, h);
v ~ N(0, 1); alpha = sigmoid(N(3, 1)) per key channel; beta = sigmoid(N(0, 1))
per (b, t, h); conv weights ~ N(0, 1/taps) (variance = 1/fan-in, taps = 4 for
the text conv and 27 for the 3x3x3 visual conv).  bf16 streams are generated in
fp32 and rounded to bf16 (round-to-nearest-even) before anything consumes them,
so every consumer sees identical values.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional, Tuple

import numpy as np
import torch

VAE_COMPRESSION = (4, 8, 8)   # (t, h, w) factors of the frozen causal 3D VAE
PATCHIFY = (1, 2, 2)          # (t, h, w) patch size applied to the latents
K_TEXT = 4                    # causal 1D depthwise kernel over text tokens
K_VIS = 3                     # 3x3x3 depthwise kernel over the visual grid


def latent_grid(frames: int, height: int, width: int) -> Tuple[int, int, int]:
    """(t, h, w) patch grid of a clip of ``frames`` frames at height x width.

    A causal video VAE keeps the first frame and compresses the remaining ones
    by the temporal factor; images are the ``frames == 1`` case.
    """
    ct, ch, cw = VAE_COMPRESSION
    pt, ph, pw = PATCHIFY
    if frames < 1 or (frames - 1) % ct:
        raise ValueError("frames must be 1 + a multiple of the temporal compression")
    t = (1 + (frames - 1) // ct) // pt
    if height % (ch * ph) or width % (cw * pw):
        raise ValueError("height/width must be multiples of the spatial downsampling")
    return (t, height // (ch * ph), width // (cw * pw))


@dataclass(frozen=True)
class StreamConfig:
    """One token-mixer workload: batch, heads, head dims, stream structure, dtype."""

    name: str
    B: int
    H: int
    dk: int
    dv: int
    n_text: int
    grid: Tuple[int, int, int]
    dtype: str                      # "f32" or "bf16"
    causal_t: int = 0               # 0: symmetric temporal padding, 1: time-causal
    seed: int = 0

    @property
    def n_vis(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def T(self) -> int:
        return self.n_text + self.n_vis

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "StreamConfig":
        return replace(self, **kw)


# The five stream workloads.  Seeds are 1000 + index.
WORKLOADS = [
    StreamConfig("tiny_fp32", B=1, H=2, dk=64, dv=64, n_text=32, grid=(4, 10, 12),
                 dtype="f32", seed=1000),
    StreamConfig("proxy_image_1024px", B=8, H=4, dk=128, dv=128, n_text=512,
                 grid=latent_grid(1, 1024, 1024), dtype="bf16", seed=1001),
    StreamConfig("video_5s_480x832", B=1, H=16, dk=128, dv=128, n_text=512,
                 grid=latent_grid(81, 480, 832), dtype="bf16", seed=1002),
    StreamConfig("image_4096px", B=1, H=16, dk=128, dv=128, n_text=512,
                 grid=latent_grid(1, 4096, 4096), dtype="bf16", seed=1003),
    StreamConfig("video_30s_480x832", B=1, H=16, dk=128, dv=128, n_text=512,
                 grid=latent_grid(481, 480, 832), dtype="bf16", seed=1004),
]
WORKLOAD = {c.name: c for c in WORKLOADS}


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-12)).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def make_inputs(cfg: StreamConfig, seed: Optional[int] = None,
                alpha_mean: float = 3.0) -> Dict[str, torch.Tensor]:
    """Seeded CPU tensors for one workload, already rounded to ``cfg.dtype``.

    Keys: q, k [B,T,H,dk]; v [B,T,H,dv]; alpha [B,T,H,dk]; beta [B,T,H];
    w_text_{q,k,v} [H*d, 4]; w_vis_{q,k,v} [H*d, 27].
    Draw order: q, k, v, alpha logits, beta logits, text weights (q, k, v),
    visual weights (q, k, v).
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, T, H, dk, dv = cfg.B, cfg.T, cfg.H, cfg.dk, cfg.dv
    f32 = np.float32
    q = _l2_normalise(rng.standard_normal((B, T, H, dk), dtype=f32))
    k = _l2_normalise(rng.standard_normal((B, T, H, dk), dtype=f32))
    v = rng.standard_normal((B, T, H, dv), dtype=f32)
    alpha = _sigmoid(rng.standard_normal((B, T, H, dk), dtype=f32) + f32(alpha_mean))
    beta = _sigmoid(rng.standard_normal((B, T, H), dtype=f32))
    out = {"q": q, "k": k, "v": v, "alpha": alpha, "beta": beta}
    ntap_t, ntap_v = K_TEXT, K_VIS ** 3
    for s, d in (("q", dk), ("k", dk), ("v", dv)):
        out[f"w_text_{s}"] = (rng.standard_normal((H * d, ntap_t), dtype=f32)
                              * f32(1.0 / np.sqrt(ntap_t)))
    for s, d in (("q", dk), ("k", dk), ("v", dv)):
        out[f"w_vis_{s}"] = (rng.standard_normal((H * d, ntap_v), dtype=f32)
                             * f32(1.0 / np.sqrt(ntap_v)))
    tdt = cfg.torch_dtype
    return {name: torch.from_numpy(a).to(tdt) for name, a in out.items()}


def token_index(cfg: StreamConfig, t: int, h: int, w: int) -> int:
    """Stream position of visual token (t, h, w): text first, then raster order."""
    _, gh, gw = cfg.grid
    return cfg.n_text + (t * gh + h) * gw + w


# ---- the MLA layers' attention core (one of every four token-mixer layers) ----------

@dataclass(frozen=True)
class MlaConfig:
    """Attention-core shapes of one MLA layer over a token stream of T tokens.

    Per head: a d_nope-wide key part decompressed from the latent, a d_dir-wide
    key part shared by all heads (K_direct), and dv-wide values.  The latent
    path maps d_model-wide hidden states to a d_c-wide latent; d_c = d_model / 4
    is a reading (the pages fix the compression ratio across scales but do not
    state it), d_model = H * 128 the layer widths of the pages' models.
    """

    name: str
    B: int
    T: int
    H: int
    d_nope: int = 128
    d_dir: int = 64
    dv: int = 128
    seed: int = 0
    d_model: int = 0      # 0: H * 128
    d_c: int = 0          # 0: d_model / 4

    @property
    def model_width(self) -> int:
        return self.d_model or self.H * 128

    @property
    def latent_width(self) -> int:
        return self.d_c or self.model_width // 4

    def with_(self, **kw) -> "MlaConfig":
        return replace(self, **kw)


MLA_WORKLOADS = [
    MlaConfig("mla_tiny", B=2, T=333, H=2, seed=21),
    MlaConfig("mla_image_1024px", B=8, T=4608, H=4, seed=22),     # the proxy-width image stream
    MlaConfig("mla_video_5s_480x832", B=1, T=33272, H=16, seed=23),
]
MLA_WORKLOAD = {c.name: c for c in MLA_WORKLOADS}


def make_mla_inputs(cfg: MlaConfig, seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Seeded bf16 CPU tensors: q_nope, k_nope [B,T,H,d_nope]; q_dir [B,T,H,d_dir];
    k_dir [B,T,d_dir]; v [B,T,H,dv].  Every entry ~ N(0, 1), drawn in that
    order in fp32 and rounded to bf16."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, T, H = cfg.B, cfg.T, cfg.H
    f32 = np.float32
    out = {"q_nope": rng.standard_normal((B, T, H, cfg.d_nope), dtype=f32),
           "k_nope": rng.standard_normal((B, T, H, cfg.d_nope), dtype=f32),
           "q_dir": rng.standard_normal((B, T, H, cfg.d_dir), dtype=f32),
           "k_dir": rng.standard_normal((B, T, cfg.d_dir), dtype=f32),
           "v": rng.standard_normal((B, T, H, cfg.dv), dtype=f32)}
    return {name: torch.from_numpy(a).to(torch.bfloat16) for name, a in out.items()}


def make_mla_latent_inputs(cfg: MlaConfig, seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Seeded bf16 CPU tensors of one MLA layer from hidden states: x [B,T,d_model] ~ N(0, 1);
    linear-layer weights w_dkv [d_c, d_model], w_kr [d_dir, d_model], w_uk [H*d_nope, d_c],
    w_uv [H*dv, d_c], each ~ N(0, 1/fan_in) so that every projection stays of unit scale;
    queries q_nope [B,T,H,d_nope], q_dir [B,T,H,d_dir] ~ N(0, 1).  Drawn in that order in fp32
    and rounded to bf16."""
    rng = np.random.default_rng((cfg.seed if seed is None else seed) + 1000)
    B, T, H = cfg.B, cfg.T, cfg.H
    dm, dc = cfg.model_width, cfg.latent_width
    f32 = np.float32

    def w(rows, fan_in):
        return (rng.standard_normal((rows, fan_in), dtype=f32) / np.sqrt(fan_in)).astype(f32)

    out = {"x": rng.standard_normal((B, T, dm), dtype=f32),
           "w_dkv": w(dc, dm), "w_kr": w(cfg.d_dir, dm),
           "w_uk": w(H * cfg.d_nope, dc), "w_uv": w(H * cfg.dv, dc),
           "q_nope": rng.standard_normal((B, T, H, cfg.d_nope), dtype=f32),
           "q_dir": rng.standard_normal((B, T, H, cfg.d_dir), dtype=f32)}
    return {name: torch.from_numpy(a).to(torch.bfloat16) for name, a in out.items()}

