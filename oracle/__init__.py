"""fp64 CPU oracle for the conv + KDA token mixer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP path and never imports it.

``short_conv`` and ``kda_recurrence`` call the plain C implementation in
``kda_oracle.c`` (the definitions written out, fp64, sequential per output).
``chunked.kda_chunked`` is a second, independent path (numpy fp64) that
restates the recurrence chunk by chunk; it exists to pin the chunk algebra the
HIP kernels implement, never to produce expected values for them.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_short_conv.restype = ctypes.c_int
    lib.oracle_short_conv.argtypes = [ctypes.c_int] * 9 + [dp] * 4
    lib.oracle_kda_recurrence.restype = ctypes.c_int
    lib.oracle_kda_recurrence.argtypes = [ctypes.c_int] * 5 + [dp] * 8
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):           # torch tensor: upcast exactly to fp64
        a = a.detach().cpu().double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> int:
    """OpenMP threads of the following oracle calls; returns the count in effect."""
    return int(_load().oracle_set_num_threads(int(n)))


def short_conv(x, w_text, w_vis, n_text: int, grid, causal_t: int = 0,
               k_text: int = 4, k_vis: int = 3) -> np.ndarray:
    """Modality-aware depthwise conv of one stream.

    x: [B, T, channels] (any float dtype; upcast to fp64), w_text: [channels, k_text],
    w_vis: [channels, k_vis**3].  Returns fp64 [B, T, channels].
    """
    x = _f64(x)
    if x.ndim != 3:
        raise ValueError("x must be [B, T, channels]")
    B, T, Cc = x.shape
    gt, gh, gw = (int(g) for g in grid)
    if T != n_text + gt * gh * gw:
        raise ValueError("T does not match n_text + grid volume")
    wt, wv = _f64(w_text), _f64(w_vis)
    if wt.shape != (Cc, k_text) or wv.shape != (Cc, k_vis ** 3):
        raise ValueError("weight shapes do not match channels/taps")
    y = np.empty_like(x)
    rc = _load().oracle_short_conv(B, n_text, gt, gh, gw, Cc, k_text, k_vis, causal_t,
                                   _ptr(x), _ptr(wt), _ptr(wv), _ptr(y))
    if rc != 0:
        raise RuntimeError("oracle_short_conv failed: %d" % rc)
    return y


def short_conv_heads(x, w_text, w_vis, n_text, grid, causal_t=0):
    """short_conv on a [B, T, H, d] tensor with [H*d, taps] weights."""
    x = _f64(x)
    B, T, H, d = x.shape
    y = short_conv(x.reshape(B, T, H * d), w_text, w_vis, n_text, grid, causal_t)
    return y.reshape(B, T, H, d)


def kda_recurrence(q, k, v, alpha, beta, S0=None,
                   want_state: bool = True) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """KDA forward by the sequential recurrence.  Returns (o [B,T,H,dv], S_T [B,H,dk,dv])."""
    q, k, v, alpha, beta = (_f64(a) for a in (q, k, v, alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or alpha.shape != q.shape or v.shape[:3] != (B, T, H) \
            or beta.shape != (B, T, H):
        raise ValueError("inconsistent KDA input shapes")
    s0 = None if S0 is None else _f64(S0)
    if s0 is not None and s0.shape != (B, H, dk, dv):
        raise ValueError("S0 must be [B, H, dk, dv]")
    o = np.empty((B, T, H, dv), dtype=np.float64)
    st = np.empty((B, H, dk, dv), dtype=np.float64) if want_state else None
    rc = _load().oracle_kda_recurrence(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(alpha), _ptr(beta), _ptr(s0), _ptr(o), _ptr(st))
    if rc != 0:
        raise RuntimeError("oracle_kda_recurrence failed: %d" % rc)
    return o, st


def conv_kda_forward(inp: dict, n_text: int, grid, causal_t: int = 0, S0=None):
    """End-to-end oracle: conv of q, k, v then the KDA recurrence (all fp64).

    ``inp`` holds q, k, v, alpha, beta and w_text_{q,k,v}, w_vis_{q,k,v}.
    Returns (q', k', v', o, S_T).
    """
    qc = short_conv_heads(inp["q"], inp["w_text_q"], inp["w_vis_q"], n_text, grid, causal_t)
    kc = short_conv_heads(inp["k"], inp["w_text_k"], inp["w_vis_k"], n_text, grid, causal_t)
    vc = short_conv_heads(inp["v"], inp["w_text_v"], inp["w_vis_v"], n_text, grid, causal_t)
    o, st = kda_recurrence(qc, kc, vc, inp["alpha"], inp["beta"], S0)
    return qc, kc, vc, o, st


def rel_err(x, ref) -> float:
    """max over (b, h) of  max_{t,j} |x - ref| / max_{t,j} |ref|.

    x, ref: [B, T, H, d] (or [B, H, dk, dv] states, with the (b, h) pair as the
    leading two axes when ``states`` layout is passed through ``rel_err_state``).
    """
    x, ref = _f64(x), _f64(ref)
    diff = np.abs(x - ref).max(axis=(1, 3))
    den = np.abs(ref).max(axis=(1, 3))
    return float(np.max(diff / np.maximum(den, 1e-300)))


def rel_err_state(x, ref) -> float:
    """rel_err for [B, H, dk, dv] states: per (b, h) max-abs difference over max-abs ref."""
    x, ref = _f64(x), _f64(ref)
    diff = np.abs(x - ref).max(axis=(2, 3))
    den = np.abs(ref).max(axis=(2, 3))
    return float(np.max(diff / np.maximum(den, 1e-300)))


def rel_err_elementwise(x, ref, floor: float = 1e-6, layout: str = "tokens") -> float:
    """Secondary, element-wise relative error (reported beside ``rel_err``, not gated).

    max over elements of |x - ref| / max(|ref|, floor * M), where M is the
    max |ref| of the element's (b, h) slice: [B, T, H, d] (layout "tokens")
    or [B, H, dk, dv] (layout "state").  The floor keeps elements whose
    reference is (close to) zero from dominating.
    """
    x, ref = _f64(x), _f64(ref)
    if layout == "tokens":
        m = np.abs(ref).max(axis=(1, 3), keepdims=True)
    elif layout == "state":
        m = np.abs(ref).max(axis=(2, 3), keepdims=True)
    else:
        raise ValueError("layout must be 'tokens' or 'state'")
    den = np.maximum(np.abs(ref), np.maximum(floor * m, 1e-300))
    return float(np.max(np.abs(x - ref) / den))
