"""fp64 oracle of the multi-head latent attention (MLA) core.

TEST INFRASTRUCTURE ONLY, under the same rules as the rest of ``oracle/``:
only ``tests/``, ``__graft_entry__.smoke()`` and bench.py's CPU-baseline leg
may import it, and it shares no code with the HIP path.

What it computes (Chimera pages, paper.rainbus.top, prerequisites section,
the Multi-head Latent Attention paragraph; DeepSeek-V2 style MLA): keys and
values are decompressed from a low-dimensional latent by plain projections
(not part of this function), and every head additionally sees one key part
that all heads share (K_direct).  Attention is full and bidirectional.  For
stream b, head h, query i and key j:

    s[b,h,i,j] = scale * (q_nope[b,i,h] . k_nope[b,j,h] + q_dir[b,i,h] . k_dir[b,j])
    o[b,i,h]   = sum_j softmax_j(s[b,h,i,:]) v[b,j,h]

Readings (the pages give neither): scale = 1 / sqrt(d_nope + d_dir) by
default, and the shared part is a plain second dot product (no position
encoding: the backbone has none).

The latent path (same paragraph): the hidden state x is compressed to the
latent c by one projection, the per-head key part and the values are
decompressed from c by two more, and K_direct is a projection of x beside the
latent.  Weights are stored as a linear layer's [out, in]:

    c = x W_dkv^T,   k_dir = x W_kr^T,   k_nope = c W_uk^T,   v = c W_uv^T

with k_nope and v split into H heads of d_nope and dv.  The queries are taken
as given (the paragraph compresses keys and values only).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().double().numpy()
    return np.asarray(a, dtype=np.float64)


def default_scale(d_nope: int, d_dir: int) -> float:
    return 1.0 / float(np.sqrt(d_nope + d_dir))


def mla_attention(q_nope, q_dir, k_nope, k_dir, v, scale: Optional[float] = None,
                  rows: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None) -> np.ndarray:
    """o for queries ``rows`` (default: all) of heads ``heads`` (default: all).

    q_nope, k_nope [B,T,H,d_nope]; q_dir [B,T,H,d_dir]; k_dir [B,T,d_dir] (one
    per token, shared by the heads); v [B,T,H,dv].  Returns fp64
    [B, len(rows), len(heads), dv].  Each softmax subtracts its row maximum
    first (exact in real arithmetic) so that exp never overflows.
    """
    qn, qd, kn, kd, vv = (_f64(a) for a in (q_nope, q_dir, k_nope, k_dir, v))
    B, T, H, dn = qn.shape
    dr = qd.shape[-1]
    sc = default_scale(dn, dr) if scale is None else float(scale)
    rows = list(range(T)) if rows is None else list(rows)
    heads = list(range(H)) if heads is None else list(heads)
    out = np.zeros((B, len(rows), len(heads), vv.shape[-1]))
    for b in range(B):
        for hi, h in enumerate(heads):
            s = qn[b, rows, h] @ kn[b, :, h].T + qd[b, rows, h] @ kd[b].T
            s *= sc
            s -= s.max(axis=1, keepdims=True)
            p = np.exp(s)
            out[b, :, hi] = (p @ vv[b, :, h]) / p.sum(axis=1, keepdims=True)
    return out


def mla_latent(x, w_dkv, w_kr, w_uk, w_uv, H: int):
    """The latent projections in fp64: x [..., d_model] -> (c [..., d_c], k_dir [..., d_dir],
    k_nope [..., H, d_nope], v [..., H, dv]).  The decompression reads the unrounded latent."""
    X, Wd, Wr, Wk, Wv = (_f64(a) for a in (x, w_dkv, w_kr, w_uk, w_uv))
    lead = X.shape[:-1]
    X2 = X.reshape(-1, X.shape[-1])
    c = X2 @ Wd.T
    k_dir = X2 @ Wr.T
    k_nope = c @ Wk.T
    v = c @ Wv.T
    return (c.reshape(lead + (Wd.shape[0],)), k_dir.reshape(lead + (Wr.shape[0],)),
            k_nope.reshape(lead + (H, Wk.shape[0] // H)), v.reshape(lead + (H, Wv.shape[0] // H)))


def mla_layer(x, q_nope, q_dir, w_dkv, w_kr, w_uk, w_uv, scale: Optional[float] = None,
              rows: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None) -> np.ndarray:
    """o of the MLA token mixer from hidden states: the latent projections, then attention."""
    H = q_nope.shape[2]
    _, k_dir, k_nope, v = mla_latent(x, w_dkv, w_kr, w_uk, w_uv, H)
    return mla_attention(q_nope, q_dir, k_nope, k_dir, v, scale=scale, rows=rows, heads=heads)

